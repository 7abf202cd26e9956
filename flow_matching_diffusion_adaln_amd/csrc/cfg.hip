// Classifier-free guidance combine (the miles page "FLUX 3 Image Klein",
// section 3: neg + scale * (pos - neg)) on bf16 rows, in fp32, rounded to
// nearest even.  HBM-bound: 6 bytes per element (two reads, one write).
#include "common.h"
#include "kernels.h"

namespace dit {

__global__ __launch_bounds__(256) void cfg_combine_kernel(const uint16_t* __restrict__ cond,
                                                          const uint16_t* __restrict__ neg,
                                                          uint16_t* __restrict__ out,
                                                          long long n8, float scale) {
  // 8 elements (16 bytes) per thread and step
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n8;
       i += (long long)gridDim.x * blockDim.x) {
    const uint4 c = reinterpret_cast<const uint4*>(cond)[i];
    const uint4 n = reinterpret_cast<const uint4*>(neg)[i];
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w}, nw[4] = {n.x, n.y, n.z, n.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = fmaf(scale, lo2f(cw[j]) - lo2f(nw[j]), lo2f(nw[j]));
      const float hi = fmaf(scale, hi2f(cw[j]) - hi2f(nw[j]), hi2f(nw[j]));
      o[j] = pack2(lo, hi);
    }
    reinterpret_cast<uint4*>(out)[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_cfg_combine(const uint16_t* cond, const uint16_t* neg, uint16_t* out,
                              long long n, float scale, hipStream_t stream) {
  const long long n8 = n / 8;  // n is a multiple of 512 (rows of width D)
  const int grid = (int)((n8 + 255) / 256 < 2048 ? (n8 + 255) / 256 : 2048);
  hipLaunchKernelGGL(cfg_combine_kernel, dim3(grid), dim3(256), 0, stream, cond, neg, out, n8,
                     scale);
  return hipGetLastError();
}

}  // namespace dit
