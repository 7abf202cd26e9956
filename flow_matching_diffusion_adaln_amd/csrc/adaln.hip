// Per-stream AdaLN modulation: u = LN(x) * (1 + scale_s) + shift_s.
//
// Source: "Welcome FLUX.3 Image Klein in Diffusers", section "How it works"
// (attention and the MLP share one normalized input; shift and scale come from
// a timestep modulation set separately for text, image and reference tokens).
// The norm is read as LayerNorm without affine and with the biased variance.
//
// HBM-bound: one read of x and one write of u (4 N D bytes).  One wavefront
// owns one row; the row stays in registers (width / 64 values per lane) so the
// two-pass statistics (mean, then the mean square deviation) cost no second
// read.  Loads and stores are 16 bytes per lane and fully coalesced.
//
// FP8 variant: u is rounded to bf16 as above, then quantized rowwise to OCP
// e4m3 with the row's scale (the same rule as quant.hip: inv = 448 / max|u|,
// q = e4m3(clamp(u * inv)), s = max|u| / 448), and only the codes (1 byte per
// element) and the scale are written: the FP8 input projection reads them.
#include "common.h"
#include "kernels.h"

namespace dit {

template <int CPL, bool F8>  // 16-byte chunks per lane: width = 512 * CPL
__global__ __launch_bounds__(256) void adaln_kernel(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ mod,
                                                    uint16_t* __restrict__ out,
                                                    uint8_t* __restrict__ q8,
                                                    float* __restrict__ q_scale, int n_rows,
                                                    int e0, int e1, float eps,
                                                    int* __restrict__ clear, int n_clear) {
  constexpr int W = 512 * CPL;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n_clear; i += 256) clear[i] = 0;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;

  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)row * W);
  uint4 v[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) v[i] = xr[lane + 64 * i];
  // the stream's shift and scale are loaded with x, before the statistics,
  // so the wave waits for memory once rather than once per chunk
  const int st = stream_of(row, e0, e1);
  const uint4* shift = reinterpret_cast<const uint4*>(mod + (size_t)st * 3 * W);
  const uint4* scale = reinterpret_cast<const uint4*>(mod + (size_t)st * 3 * W + W);
  uint4 shv[CPL], scv[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    shv[i] = shift[lane + 64 * i];
    scv[i] = scale[lane + 64 * i];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the loads above the statistics

  float s = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) s += lo2f(w[t]) + hi2f(w[t]);
  }
  const float mean = wave_sum(s) * (1.0f / W);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float a = lo2f(w[t]) - mean, b = hi2f(w[t]) - mean;
      ss += a * a + b * b;
    }
  }
  const float rstd = rsqrtf(wave_sum(ss) * (1.0f / W) + eps);

  uint4* orow = reinterpret_cast<uint4*>(out + (size_t)row * W);
  uint4 ob[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const uint4 sh = shv[i], sc = scv[i];
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    const uint32_t a[4] = {sh.x, sh.y, sh.z, sh.w};
    const uint32_t b[4] = {sc.x, sc.y, sc.z, sc.w};
    uint32_t o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float lo = (lo2f(w[t]) - mean) * rstd * (1.f + lo2f(b[t])) + lo2f(a[t]);
      const float hi = (hi2f(w[t]) - mean) * rstd * (1.f + hi2f(b[t])) + hi2f(a[t]);
      o[t] = pack2(lo, hi);
    }
    ob[i] = make_uint4(o[0], o[1], o[2], o[3]);
    if constexpr (!F8) orow[lane + 64 * i] = ob[i];
  }
  if constexpr (F8) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const uint32_t w[4] = {ob[i].x, ob[i].y, ob[i].z, ob[i].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) m = fmaxf(m, fmaxf(fabsf(lo2f(w[t])), fabsf(hi2f(w[t]))));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float inv = m > 0.f ? 448.0f / m : 0.f;
    if (lane == 0) q_scale[row] = m / 448.0f;
    uint2* qrow = reinterpret_cast<uint2*>(q8 + (size_t)row * W);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const uint32_t w[4] = {ob[i].x, ob[i].y, ob[i].z, ob[i].w};
      float f[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f[2 * t] = fminf(fmaxf(lo2f(w[t]) * inv, -448.f), 448.f);
        f[2 * t + 1] = fminf(fmaxf(hi2f(w[t]) * inv, -448.f), 448.f);
      }
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
      qrow[lane + 64 * i] = make_uint2((uint32_t)lo, (uint32_t)hi);
    }
  }
}

namespace {

template <bool F8>
hipError_t adaln_launch(const uint16_t* x, const uint16_t* mod, uint16_t* out, uint8_t* q8,
                        float* q_scale, int n_rows, int width, int e0, int e1, float eps,
                        hipStream_t stream, int* clear, int n_clear) {
  const dim3 grid((n_rows + 3) / 4), block(256);
  switch (width / 512) {
#define DIT_ADALN_CASE(C)                                                                        \
  case C:                                                                                        \
    hipLaunchKernelGGL((adaln_kernel<C, F8>), grid, block, 0, stream, x, mod, out, q8, q_scale,  \
                       n_rows, e0, e1, eps, clear, n_clear);                                     \
    break;
    DIT_ADALN_CASE(1) DIT_ADALN_CASE(2) DIT_ADALN_CASE(3) DIT_ADALN_CASE(4)
    DIT_ADALN_CASE(5) DIT_ADALN_CASE(6) DIT_ADALN_CASE(7) DIT_ADALN_CASE(8)
    DIT_ADALN_CASE(9) DIT_ADALN_CASE(10) DIT_ADALN_CASE(11) DIT_ADALN_CASE(12)
    DIT_ADALN_CASE(13) DIT_ADALN_CASE(14) DIT_ADALN_CASE(15) DIT_ADALN_CASE(16)
#undef DIT_ADALN_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_adaln(const uint16_t* x, const uint16_t* mod, uint16_t* out, int n_rows,
                        int width, int e0, int e1, float eps, hipStream_t stream, int* clear,
                        int n_clear) {
  return adaln_launch<false>(x, mod, out, nullptr, nullptr, n_rows, width, e0, e1, eps, stream,
                             clear, n_clear);
}

hipError_t launch_adaln_fp8(const uint16_t* x, const uint16_t* mod, uint8_t* q8, float* q_scale,
                            int n_rows, int width, int e0, int e1, float eps,
                            hipStream_t stream, int* clear, int n_clear) {
  return adaln_launch<true>(x, mod, nullptr, q8, q_scale, n_rows, width, e0, e1, eps, stream,
                            clear, n_clear);
}

}  // namespace dit
