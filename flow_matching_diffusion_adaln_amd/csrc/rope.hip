// Per-head QK RMSNorm followed by 4-axis RoPE, in place on q and k.
//
// Sources: the miles page "FLUX 3 Image Klein", section 3 "Family config"
// (query_norm.scale / key_norm.scale: a learnable per-head RMSNorm on q and k);
// "Welcome FLUX.3 Image Klein in Diffusers", section "How it works" (RoPE over
// four axes t, h, w, l, each owning 32 of the 128 head dims).  Pair layout
// and frequencies follow the usual per-axis RoPE: pair j = adjacent dims
// (2j, 2j + 1) of the axis, angle pos_a * theta^(-2j / 32).
//
// HBM-bound: q and k are read once and written once (8 N D bytes).  One
// wavefront owns one token: 16 lanes hold one 128-dim head vector (16 bytes
// each), so the RMS reduction is 4 butterfly steps inside the 16-lane group
// and the 4 angles a lane needs are computed once per token and reused for
// all 2 H head vectors of that token.  A lane loads up to RB of its head
// vectors before it rotates any, so a short sequence (a few waves in all)
// does not wait one memory round trip per vector.  Angles: the turn count
// pos * theta^(-2j / 32) / (2 pi) in fp64, reduced to [0, 1), then the
// hardware sin / cos of 2 pi times that fraction (as the input projection's
// fused epilogue does).
#include "common.h"
#include "kernels.h"

namespace dit {

// theta^(-2j / 32) / (2 pi) for the 16 pairs of an axis: turns per position step
struct RopeRev {
  double rev[16];
};

__global__ __launch_bounds__(256) void rope4_kernel(uint16_t* __restrict__ q,
                                                    uint16_t* __restrict__ k,
                                                    const int32_t* __restrict__ pos,
                                                    const uint16_t* __restrict__ q_scale,
                                                    const uint16_t* __restrict__ k_scale,
                                                    int n_tokens, int n_heads, RopeRev rr,
                                                    float eps, int do_norm, float q_mul) {
  constexpr int RB = 6;  // head vectors in flight per lane
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tok >= n_tokens) return;
  const int c = lane & 15;    // 8-dim chunk of the head vector: dims 8c .. 8c + 7
  const int slot = lane >> 4;  // which of the 4 head vectors this group handles
  const int axis = c >> 2;     // 32 dims = 4 chunks per axis
  const int D = n_heads * 128;
  const int nv = 2 * n_heads;  // q heads, then k heads
  auto vec_ptr = [&](int vec) {
    const int which = vec >= n_heads;
    const int h = vec - which * n_heads;
    return reinterpret_cast<uint4*>((which ? k : q) + (size_t)tok * D + h * 128) + c;
  };
  // first loads go out before the angle and scale set-up
  uint4 raw[RB];
#pragma unroll
  for (int u = 0; u < RB; ++u)
    if (slot + 4 * u < nv) raw[u] = *vec_ptr(slot + 4 * u);

  const int4 p4 = reinterpret_cast<const int4*>(pos)[tok];
  const int p = axis == 0 ? p4.x : axis == 1 ? p4.y : axis == 2 ? p4.z : p4.w;
  float cs[4], sn[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = 4 * (c & 3) + t;  // pair index inside the axis, 0..15
    const double turns = (double)p * rr.rev[j];
    const float fr = (float)(turns - floor(turns));
    sn[t] = __builtin_amdgcn_sinf(fr);
    cs[t] = __builtin_amdgcn_cosf(fr);
  }
  float g[2][8];
  if (do_norm) {
    const uint4 gq = reinterpret_cast<const uint4*>(q_scale)[c];
    const uint4 gk = reinterpret_cast<const uint4*>(k_scale)[c];
    const uint32_t wq[4] = {gq.x, gq.y, gq.z, gq.w}, wk[4] = {gk.x, gk.y, gk.z, gk.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      g[0][2 * t] = lo2f(wq[t]);
      g[0][2 * t + 1] = hi2f(wq[t]);
      g[1][2 * t] = lo2f(wk[t]);
      g[1][2 * t + 1] = hi2f(wk[t]);
    }
  }
  for (int v0 = slot; v0 < nv; v0 += 4 * RB) {
    if (v0 != slot) {
#pragma unroll
      for (int u = 0; u < RB; ++u)
        if (v0 + 4 * u < nv) raw[u] = *vec_ptr(v0 + 4 * u);
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int vec = v0 + 4 * u;
      if (vec >= nv) break;
      const int which = vec >= n_heads;  // 0: q, 1: k
      const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
      float e[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        e[2 * t] = lo2f(w[t]);
        e[2 * t + 1] = hi2f(w[t]);
      }
      if (do_norm) {
        float ss = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) ss += e[t] * e[t];
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o, 64);
        const float r = rsqrtf(ss * (1.0f / 128.0f) + eps);
#pragma unroll
        for (int t = 0; t < 8; ++t) e[t] = e[t] * r * g[which][t];
      }
      const float mul = which ? 1.0f : q_mul;
      uint32_t o[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float x0 = e[2 * t] * mul, x1 = e[2 * t + 1] * mul;
        o[t] = pack2(x0 * cs[t] - x1 * sn[t], x0 * sn[t] + x1 * cs[t]);
      }
      *vec_ptr(vec) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

hipError_t launch_rope4(uint16_t* q, uint16_t* k, const int32_t* pos, const uint16_t* q_scale,
                        const uint16_t* k_scale, int n_tokens, int n_heads, float theta,
                        float eps, float q_mul, hipStream_t stream) {
  const int do_norm = q_scale != nullptr;
  RopeRev rr;
  const double two_pi = 6.283185307179586;
  for (int j = 0; j < 16; ++j) rr.rev[j] = pow((double)theta, -2.0 * j / 32.0) / two_pi;
  hipLaunchKernelGGL(rope4_kernel, dim3((n_tokens + 3) / 4), dim3(256), 0, stream, q, k, pos,
                     q_scale, k_scale, n_tokens, n_heads, rr, eps, do_norm, q_mul);
  return hipGetLastError();
}
}  // namespace dit
