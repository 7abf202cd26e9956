// Rowwise FP8 quantization (OCP e4m3, gfx950's FP8 MFMA format) of bf16
// matrices: the input side of the rowwise-scaled FP8 ("fp8r") projections
// that the SGLang FLUX.3 page ships for its linear layers.
//
// Per row r: a_r = max |x_r|, inv_r = 448 / a_r and s_r = a_r / 448 (both
// float32, correctly rounded), q = e4m3(clamp(x * inv_r, +-448)) with the
// hardware's round-to-nearest-even convert, so that x ~ q * s_r.  An all-zero
// row gets s_r = 0 and q = 0.  HBM-bound: one read of the row (the second
// pass over it hits L2), 1 byte written per element.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int QT = 256;  // threads per row

__global__ __launch_bounds__(QT) void quant_rows_kernel(const uint16_t* __restrict__ x,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ scale, int K) {
  __shared__ float red[QT / 64];
  const int row = blockIdx.x, tid = threadIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)row * K);
  const int n8 = K / 8;
  float m = 0.f;
  for (int c = tid; c < n8; c += QT) {
    const uint4 v = xr[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) m = fmaxf(m, fmaxf(fabsf(lo2f(w[t])), fabsf(hi2f(w[t]))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = m > 0.f ? 448.0f / m : 0.f;
  if (tid == 0) scale[row] = m / 448.0f;
  uint2* qr = reinterpret_cast<uint2*>(q + (size_t)row * K);
  for (int c = tid; c < n8; c += QT) {
    const uint4 v = xr[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
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
    qr[c] = make_uint2((uint32_t)lo, (uint32_t)hi);
  }
}

}  // namespace

hipError_t launch_quant_rows(const uint16_t* x, uint8_t* q, float* scale, int M, int K,
                             hipStream_t stream) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel, dim3(M), dim3(QT), 0, stream, x, q, scale, K);
  return hipGetLastError();
}

}  // namespace dit
