// Internal launchers of the block's kernels (host side).  Arguments are
// validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace dit {

hipError_t launch_adaln(const uint16_t* x, const uint16_t* mod, uint16_t* out, int n_rows,
                        int width, int e0, int e1, float eps, hipStream_t stream);

hipError_t launch_rope4(uint16_t* q, uint16_t* k, const int32_t* pos, const uint16_t* q_scale,
                        const uint16_t* k_scale, int n_tokens, int n_heads, float theta,
                        float eps, hipStream_t stream);

hipError_t launch_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                       int N, int H, int ld_qkv, int ld_o, float softmax_scale,
                       hipStream_t stream);

hipError_t launch_gemm_in(const uint16_t* u, const uint16_t* w_in, int M, int D, int F,
                          uint16_t* q, uint16_t* k, uint16_t* v, uint16_t* cat,
                          hipStream_t stream);

hipError_t launch_gemm_out(const uint16_t* cat, const uint16_t* w_out, int M, int D, int F,
                           const uint16_t* x, const uint16_t* mod, uint16_t* y, int e0, int e1,
                           uint32_t flags, hipStream_t stream);

}  // namespace dit
