// Full joint attention, o = softmax(q k^T * scale) v per head, flash style.
//
// Source: "Welcome FLUX.3 Image Klein in Diffusers", section "How it works"
// (the 28 joint blocks run full attention over the concatenated streams,
// prompt padding included) and the miles page "FLUX 3 Image Klein", section 3
// (the DiT takes no padding mask).  No mask is applied.
//
// Design (gfx950, 64-wide waves, 32x32x16 bf16 MFMA):
//  * A workgroup is one head x 128 queries; each of its 4 waves owns 32
//    queries for the whole key loop.  Keys stream through LDS in tiles of 64,
//    double-buffered, loaded once per workgroup and shared by the 4 waves.
//  * Scores are computed transposed, S^T = K Q^T (A = K from LDS, B = Q held
//    in registers).  In the 32x32 MFMA result a lane holds one column, so
//    each lane owns one query: the row max and row sum of the softmax are
//    in-lane reductions plus one exchange with the other half-wave.
//  * The K rows fed to the A operand are permuted (key_slot below) so that
//    the 16 scores a lane ends up holding are exactly the 16 keys it must
//    supply as the B operand of O^T = V^T P^T.  P never leaves registers.
//  * V is stored transposed in LDS (V^T[dim][key]) while staging, so the
//    A operand V^T reads 16 contiguous bytes per lane.
//  * Online softmax in fp32 with exp2 (scale * log2 e folded into one FMA),
//    P rounded to bf16 for the MFMA, one division by the row sum at the end.
//  * Workgroups of one head are kept on one XCD so its K and V stay in that
//    XCD's L2.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int BQ = 128;  // queries per workgroup
constexpr int BKEY = 64; // keys per tile
constexpr int HD = 128;  // head dim

// K tile in LDS: [64 keys][128 dims], 16 chunks of 16 B per row, chunk index
// xor-swizzled so the permuted-row A reads and the row-wise stores are
// conflict free.
__device__ __forceinline__ int kswz(int row) { return (row & 3) | ((row >> 1) & 4); }

// Key held by A-operand row m of a 32-key block (m = 8r + 4h + j maps to
// 16(r/2) + 8h + 4(r%2) + j): with this order the MFMA output register
// 4r + j of half-wave h is the key the PV MFMA wants in B slot 8(r%2) + j
// of k-step r/2.
__device__ __forceinline__ int key_slot(int m) {
  const int r = m >> 3, h = (m >> 2) & 1, j = m & 3;
  return 16 * (r >> 1) + 8 * h + 4 * (r & 1) + j;
}

// 16-bit element e (0..7) of a 16-byte vector, zero-extended
__device__ __forceinline__ uint32_t half16(const uint4& v, int e) {
  const uint32_t d = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? (d >> 16) : (d & 0xffffu);
}

}  // namespace

__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          uint16_t* __restrict__ o, int N,
                                                          int H, int ld_qkv, int ld_o,
                                                          float c) {
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][BKEY * HD];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][HD * BKEY];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, hl = lane >> 5;
  const int nqt = (N + BQ - 1) / BQ;
  const int id = xcd_remap(blockIdx.x, nqt * H);
  const int h = id / nqt, qt = id % nqt;
  const int q0 = qt * BQ + wave * 32;
  const size_t hoff = (size_t)h * HD;

  // Q fragments (B operand of S^T = K Q^T): lane holds q[q0 + ln][16 s + 8 hl .. + 8]
  bf16x8 qf[8];
  {
    const int qi = min(q0 + ln, N - 1);
    const uint4* qp = reinterpret_cast<const uint4*>(q + (size_t)qi * ld_qkv + hoff);
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = __builtin_bit_cast(bf16x8, qp[2 * s + hl]);
  }

  f32x16 acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // staging: K chunk (row = id >> 4, chunk = id & 15) for id = tid + 256 i;
  // V: 4 consecutive keys (group u) x 8 dims (chunk cv) per thread
  const int vu = tid & 15, vc = tid >> 4;
  uint4 kreg[4], vreg[4];
  const int ntiles = (N + BKEY - 1) / BKEY;

  auto gload = [&](int t) {
    const int key0 = t * BKEY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int key = min(key0 + (idx >> 4), N - 1);
      kreg[i] = *reinterpret_cast<const uint4*>(k + (size_t)key * ld_qkv + hoff + (idx & 15) * 8);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int key = min(key0 + 4 * vu + kk, N - 1);
      vreg[kk] = *reinterpret_cast<const uint4*>(v + (size_t)key * ld_qkv + hoff + vc * 8);
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int row = idx >> 4, ch = idx & 15;
      *reinterpret_cast<uint4*>(&s_k[st][row * HD + ((ch ^ kswz(row)) << 3)]) = kreg[i];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t lo = half16(vreg[0], e) | (half16(vreg[1], e) << 16);
      const uint32_t hi = half16(vreg[2], e) | (half16(vreg[3], e) << 16);
      const int row = 8 * vc + e;  // dim
      const int ch = (vu >> 1) ^ (row & 7);
      *reinterpret_cast<uint2*>(&s_vt[st][row * BKEY + ch * 8 + (vu & 1) * 4]) = make_uint2(lo, hi);
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < ntiles) gload(t + 1);

    // S^T = K Q^T for two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      const int row = 32 * kb + key_slot(ln);
      const uint16_t* kr = &s_k[cur][row * HD];
      const int sw = kswz(row);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + (((2 * st + hl) ^ sw) << 3));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kb], 0, 0, 0);
      }
    }

    // keys past N (last tile only) get no weight
    if ((t + 1) * BKEY > N) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t * BKEY + 32 * kb + 16 * (r >> 3) + 8 * hl + (r & 7);
          if (key >= N) s[kb][r] = -INFINITY;
        }
    }

    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f((m_run - m_new) * c);
    const float mc = m_new * c;
    m_run = m_new;

    bf16x8 pb[4];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(fmaf(s[kb][r], c, -mc));
        psum += p;
        pb[2 * kb + (r >> 3)][r & 7] = (__bf16)p;
      }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int row = 32 * d + ln;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &s_vt[cur][row * BKEY + (((2 * ks + hl) ^ (row & 7)) << 3)]);
        acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks], acc[d], 0, 0, 0);
      }
    }

    if (t + 1 < ntiles) sstore(cur ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  const int qi = q0 + ln;
  if (qi < N) {
    uint16_t* op = o + (size_t)qi * ld_o + hoff;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int dim = 32 * d + 8 * r + 4 * hl;
        const uint32_t lo = pack2(acc[d][4 * r] * inv, acc[d][4 * r + 1] * inv);
        const uint32_t hi = pack2(acc[d][4 * r + 2] * inv, acc[d][4 * r + 3] * inv);
        *reinterpret_cast<uint2*>(op + dim) = make_uint2(lo, hi);
      }
  }
}

hipError_t launch_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                       int N, int H, int ld_qkv, int ld_o, float softmax_scale,
                       hipStream_t stream) {
  const int nqt = (N + BQ - 1) / BQ;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(nqt * H), dim3(256), 0, stream, q, k, v, o, N, H,
                     ld_qkv, ld_o, softmax_scale * DIT_LOG2E);
  return hipGetLastError();
}

}  // namespace dit
