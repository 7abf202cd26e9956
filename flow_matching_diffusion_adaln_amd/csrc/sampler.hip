// Kernels of the denoise step around the block stack: the small linear
// layers (token embedders, the timestep MLP and modulation, proj_out), the
// timestep sinusoids, and the guided Euler update of the latent.
//
// The linear layers are a few GFLOP per step against the stack's tens of
// TFLOP, and several have only one or two rows (the timestep path), so the
// linear kernel is a plain MFMA tile that reads its fragments straight from
// global memory (L1 / L2 serve the reuse) rather than the LDS-pipelined GEMM
// of the block.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int LIN_BM = 32;   // rows per workgroup
constexpr int LIN_BN = 128;  // outputs per workgroup: 4 waves x 32
constexpr int LIN_KC = 4;    // k steps of 16 per load batch

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }

// y[m, n] = act(sum_k x[m, k] w[n, k] + b[n]) for m < M, n < N.  K is a
// multiple of 16, N of 32.  Wave w of the workgroup computes the 32 x 32
// block (rows m0 .. m0 + 31, outputs n0 + 32 w ..): the weights are the MFMA's
// A operand, so lane (ln, hl) ends with row m0 + ln and outputs
// 8 rr + 4 hl .. + 3 of the block in registers 4 rr .. 4 rr + 3.  Each
// fragment is 8 consecutive k of one row: 16 contiguous bytes per lane.
__global__ __launch_bounds__(256) void linear_kernel(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ w,
                                                     const uint16_t* __restrict__ b,
                                                     uint16_t* __restrict__ y, int M, int N, int K,
                                                     int ldx, int ldy, int act) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 31, hl = lane >> 5;
  const int m0 = blockIdx.y * LIN_BM;
  const int n0 = blockIdx.x * LIN_BN + wave * 32;
  if (n0 >= N) return;  // whole wave past the last output block
  const int xr = min(m0 + ln, M - 1);  // rows past M load row M - 1, never stored
  const bf16x8* xp = reinterpret_cast<const bf16x8*>(x + (size_t)xr * ldx + 8 * hl);
  const bf16x8* wp = reinterpret_cast<const bf16x8*>(w + (size_t)(n0 + ln) * K + 8 * hl);
  const int ks = K / 16;  // k steps; fragment j of step s is at index 2 s
  f32x16 acc = {};
  bf16x8 fx[2][LIN_KC], fw[2][LIN_KC];
  auto load = [&](int buf, int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < LIN_KC; ++c) {
      const int s = min(s0 + c, ks - 1);  // past the end: reload the last step, unused
      fx[buf][c] = xp[2 * s];
      fw[buf][c] = wp[2 * s];
    }
  };
  load(0, 0);
  int s0 = 0;
  for (; s0 + LIN_KC < ks; s0 += 2 * LIN_KC) {
    load(1, s0 + LIN_KC);
#pragma unroll
    for (int c = 0; c < LIN_KC; ++c)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[0][c], fx[0][c], acc, 0, 0, 0);
    if (s0 + 2 * LIN_KC < ks) load(0, s0 + 2 * LIN_KC);
#pragma unroll
    for (int c = 0; c < LIN_KC; ++c)
      if (s0 + LIN_KC + c < ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[1][c], fx[1][c], acc, 0, 0, 0);
  }
  if (s0 < ks) {
#pragma unroll
    for (int c = 0; c < LIN_KC; ++c)
      if (s0 + c < ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[0][c], fx[0][c], acc, 0, 0, 0);
  }
  const int m = m0 + ln;
  if (m >= M) return;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int n = n0 + 8 * rr + 4 * hl;
    float v[4] = {acc[4 * rr], acc[4 * rr + 1], acc[4 * rr + 2], acc[4 * rr + 3]};
    if (b) {
      const uint2 bv = *reinterpret_cast<const uint2*>(b + n);
      v[0] += lo2f(bv.x);
      v[1] += hi2f(bv.x);
      v[2] += lo2f(bv.y);
      v[3] += hi2f(bv.y);
    }
    if (act == 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = silu_f(v[e]);
    }
    *reinterpret_cast<uint2*>(y + (size_t)m * ldy + n) =
        make_uint2(pack2(v[0], v[1]), pack2(v[2], v[3]));
  }
}

struct Times {
  double t[4];
};

// out[r, i] = cos(scale t_r f_i), out[r, half + i] = sin(scale t_r f_i), with
// f_i = max_period^(-i / half), in double, rounded to bf16.
__global__ __launch_bounds__(256) void sinusoid_kernel(Times ts, int n_t, int dim, double scale,
                                                       double log_max_period, uint16_t* out) {
  const int half = dim / 2;
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < n_t * half;
       idx += gridDim.x * blockDim.x) {
    const int r = idx / half, i = idx - r * half;
    const double f = exp(-log_max_period * (double)i / (double)half);
    const double a = scale * ts.t[r] * f;
    const uint32_t cs = pack2((float)cos(a), (float)sin(a));
    out[(size_t)r * dim + i] = (uint16_t)(cs & 0xffffu);
    out[(size_t)r * dim + half + i] = (uint16_t)(cs >> 16);
  }
}

// z += dsigma * (neg + scale (cond - neg)) (or dsigma * cond without neg),
// in fp32 on bf16 values, 8 per thread; the guided velocity goes to v_out
// when given.  HBM-bound: 8 (10 with v_out) bytes per element.
__global__ __launch_bounds__(256) void euler_cfg_kernel(uint16_t* __restrict__ z,
                                                        const uint16_t* __restrict__ cond,
                                                        const uint16_t* __restrict__ neg,
                                                        uint16_t* __restrict__ v_out, long long n8,
                                                        float scale, float dsigma) {
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n8;
       i += (long long)gridDim.x * blockDim.x) {
    const uint4 zc = reinterpret_cast<const uint4*>(z)[i];
    const uint4 c = reinterpret_cast<const uint4*>(cond)[i];
    const uint4 n = neg ? reinterpret_cast<const uint4*>(neg)[i] : c;
    const uint32_t zw[4] = {zc.x, zc.y, zc.z, zc.w}, cw[4] = {c.x, c.y, c.z, c.w},
                   nw[4] = {n.x, n.y, n.z, n.w};
    uint32_t zo[4], vo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v0 = lo2f(cw[j]), v1 = hi2f(cw[j]);
      if (neg) {
        v0 = fmaf(scale, v0 - lo2f(nw[j]), lo2f(nw[j]));
        v1 = fmaf(scale, v1 - hi2f(nw[j]), hi2f(nw[j]));
      }
      zo[j] = pack2(fmaf(dsigma, v0, lo2f(zw[j])), fmaf(dsigma, v1, hi2f(zw[j])));
      vo[j] = pack2(v0, v1);
    }
    reinterpret_cast<uint4*>(z)[i] = make_uint4(zo[0], zo[1], zo[2], zo[3]);
    if (v_out) reinterpret_cast<uint4*>(v_out)[i] = make_uint4(vo[0], vo[1], vo[2], vo[3]);
  }
}

}  // namespace

hipError_t launch_linear(const uint16_t* x, const uint16_t* w, const uint16_t* b, uint16_t* y,
                         int M, int N, int K, int ldx, int ldy, int act, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const dim3 grid((N + LIN_BN - 1) / LIN_BN, (M + LIN_BM - 1) / LIN_BM);
  hipLaunchKernelGGL(linear_kernel, grid, dim3(256), 0, stream, x, w, b, y, M, N, K, ldx, ldy,
                     act);
  return hipGetLastError();
}

hipError_t launch_sinusoid(const double* t, int n_t, int dim, double scale, double max_period,
                           uint16_t* out, hipStream_t stream) {
  Times ts{};
  for (int i = 0; i < n_t; ++i) ts.t[i] = t[i];
  const int total = n_t * (dim / 2);
  hipLaunchKernelGGL(sinusoid_kernel, dim3((total + 255) / 256), dim3(256), 0, stream, ts, n_t,
                     dim, scale, log(max_period), out);
  return hipGetLastError();
}

hipError_t launch_euler_cfg(uint16_t* z, const uint16_t* cond, const uint16_t* neg,
                            uint16_t* v_out, long long n, float scale, float dsigma,
                            hipStream_t stream) {
  const long long n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  const int grid = (int)((n8 + 255) / 256 < 2048 ? (n8 + 255) / 256 : 2048);
  hipLaunchKernelGGL(euler_cfg_kernel, dim3(grid), dim3(256), 0, stream, z, cond, neg, v_out, n8,
                     scale, dsigma);
  return hipGetLastError();
}

}  // namespace dit
