// Internal launchers of the library's kernels (host side).  Arguments are
// validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace dit {

// Pieces a GEMM's tail round may be split into, and the fp32 scratch the
// split needs (2 partial 256 x 256 tiles per piece).
#define GEMM_MAX_SPLIT_PIECES 256
constexpr size_t kGemmPartialBytes = (size_t)2 * GEMM_MAX_SPLIT_PIECES * 256 * 256 * 4;

// Compute units of the current device (queried once per device).
int device_cus();

// `clear` (may be null): n_clear ints the kernel sets to zero on the way
// (the attention split counters of the same block).
hipError_t launch_adaln(const uint16_t* x, const uint16_t* mod, uint16_t* out, int n_rows,
                        int width, int e0, int e1, float eps, hipStream_t stream,
                        int* clear = nullptr, int n_clear = 0);

// FP8 variant: u rounded to bf16, then quantized rowwise to e4m3 codes q8
// [n_rows, width] with one float scale per row (u ~ q8 * q_scale).
hipError_t launch_adaln_fp8(const uint16_t* x, const uint16_t* mod, uint8_t* q8, float* q_scale,
                            int n_rows, int width, int e0, int e1, float eps,
                            hipStream_t stream, int* clear = nullptr, int n_clear = 0);

// Rowwise e4m3 quantization of bf16 x [M, K] (K a multiple of 8): codes q
// [M, K], scales [M] with x ~ q * scale.
hipError_t launch_quant_rows(const uint16_t* x, uint8_t* q, float* scale, int M, int K,
                             hipStream_t stream);

// q_mul multiplies q after the norm and rotation (1 for plain RoPE; the
// block passes the softmax's log2 e / sqrt(d), see launch_attn)
hipError_t launch_rope4(uint16_t* q, uint16_t* k, const int32_t* pos, const uint16_t* q_scale,
                        const uint16_t* k_scale, int n_tokens, int n_heads, float theta,
                        float eps, float q_mul, hipStream_t stream);

// Scratch that lets attention cut its work into one equal share per CU:
// `part` holds the fp32 partials of the items cut between two shares (one
// slot per cut, attn_split_bytes(slots) bytes for `slots` slots), `counters`
// one int per slot, all zero when the launch starts (with `clear` the launch
// zeroes them first, otherwise the caller has).  Without it (null) every
// workgroup runs one whole (head, 256-query) item.
struct AttnSplit {
  void* part;
  size_t part_bytes;
  int* counters;
  int n_counters;
  bool clear;
};
size_t attn_split_bytes(int n_slots);

// q_scale / k_scale (both or neither): the QK RMSNorm scales q and k were
// normalized with.  q_prescaled: q already carries softmax_scale * log2 e.
// With both, the scores are bounded and the kernel may use a fixed softmax
// reference, P = exp2(q k), instead of a running max.
hipError_t launch_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                       int N, int H, int ld_qkv, int ld_o, float softmax_scale,
                       const uint16_t* q_scale, const uint16_t* k_scale, int q_prescaled,
                       const AttnSplit* split, hipStream_t stream);

// q_mul multiplies the normalized, rotated q before it is stored
hipError_t launch_gemm_in(const uint16_t* u, const uint16_t* w_in, int M, int D, int F,
                          uint16_t* q, uint16_t* k, uint16_t* v, uint16_t* cat,
                          const int32_t* pos, const uint16_t* q_scale, const uint16_t* k_scale,
                          float theta, float qk_eps, float q_mul, float* partial,
                          hipStream_t stream);

// counters (may be null): n_counters zeroed ints that let a short sequence
// run the weight-streaming output projection with its K split (see below)
hipError_t launch_gemm_out(const uint16_t* cat, const uint16_t* w_out, int M, int D, int F,
                           const uint16_t* x, const uint16_t* mod, uint16_t* y, int e0, int e1,
                           uint32_t flags, float* partial, hipStream_t stream,
                           int* counters = nullptr, int n_counters = 0);

// Projections of short sequences (at most kThinMaxTokens tokens) as weight
// streams: a workgroup per 128 weight rows, every token in the MFMAs' other
// operand, epilogues fused (thin.hip).  thin_fits: the shapes they take.
// The output projection cuts K into pieces whose fp32 partials
// (thin_partial_bytes) are summed by the last piece to arrive, counted in
// `counters` (D / 128 ints, zero at launch, left zero); with too little
// scratch it runs whole columns instead.
constexpr int kThinMaxTokens = 160;
constexpr int kThinMaxPieces = 32;
bool thin_fits(int M, int D, int F);
size_t thin_partial_bytes(int M, int D, int pieces);
hipError_t launch_thin_in(const uint16_t* u, const uint16_t* w_in, int M, int D, int F,
                          uint16_t* q, uint16_t* k, uint16_t* v, uint16_t* cat,
                          const int32_t* pos, const uint16_t* q_scale, const uint16_t* k_scale,
                          float theta, float qk_eps, float q_mul, hipStream_t stream);
hipError_t launch_thin_out(const uint16_t* cat, const uint16_t* w_out, int M, int D, int F,
                           const uint16_t* x, const uint16_t* mod, uint16_t* y, int e0, int e1,
                           uint32_t flags, float* partial, size_t partial_bytes, int* counters,
                           int n_counters, hipStream_t stream);

// FP8 projections: e4m3 operands with rowwise scales (u8 / cat8 rows scaled
// by u_scale / cat_scale, weight rows by w_*_scale), epilogues as above.
hipError_t launch_gemm_in_fp8(const uint8_t* u8, const float* u_scale, const uint8_t* w_in8,
                              const float* w_in_scale, int M, int D, int F, uint16_t* q,
                              uint16_t* k, uint16_t* v, uint16_t* cat, const int32_t* pos,
                              const uint16_t* q_scale, const uint16_t* k_scale, float theta,
                              float qk_eps, float q_mul, float* partial, hipStream_t stream);

hipError_t launch_gemm_out_fp8(const uint8_t* cat8, const float* cat_scale,
                               const uint8_t* w_out8, const float* w_out_scale, int M, int D,
                               int F, const uint16_t* x, const uint16_t* mod, uint16_t* y,
                               int e0, int e1, uint32_t flags, float* partial,
                               hipStream_t stream);

// out = neg + scale * (cond - neg) elementwise over n bf16 values (n a multiple of 8)
hipError_t launch_cfg_combine(const uint16_t* cond, const uint16_t* neg, uint16_t* out,
                              long long n, float scale, hipStream_t stream);

// y[m, n] = act(x[m, :] . w[n, :] + b[n]) (act 0: none, 1: SiLU), bf16 in and
// out, fp32 accumulation.  w is [N, K] row-major; b may be null.  K must be
// a multiple of 16, N of 32; row strides ldx, ldy in elements.
hipError_t launch_linear(const uint16_t* x, const uint16_t* w, const uint16_t* b, uint16_t* y,
                         int M, int N, int K, int ldx, int ldy, int act, hipStream_t stream);

// out [n_t, dim] bf16: [cos | sin] of scale * t_r * max_period^(-i / (dim / 2)),
// n_t <= 4, dim even.
hipError_t launch_sinusoid(const double* t, int n_t, int dim, double scale, double max_period,
                           uint16_t* out, hipStream_t stream);

// z += dsigma * (neg + scale * (cond - neg)) over n bf16 values (n a multiple
// of 8; neg null: dsigma * cond); v_out (optional) gets the guided velocity.
hipError_t launch_euler_cfg(uint16_t* z, const uint16_t* cond, const uint16_t* neg,
                            uint16_t* v_out, long long n, float scale, float dsigma,
                            hipStream_t stream);

}  // namespace dit
