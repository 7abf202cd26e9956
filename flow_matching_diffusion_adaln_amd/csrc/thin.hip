// Input and output projections of short sequences (at most 160 tokens).
//
// The text-only stage-1 blocks run on prompts of 80-token multiples ("Welcome
// FLUX.3 Image Klein in Diffusers", "How it works"): at that length a
// projection is a stream of its weights (170 MB for the input projection at
// width 3072, 75 MB for the output one) past a few kilobytes of activations,
// so it is bound by reading each weight byte once from HBM, not by the MFMAs.
//
// A workgroup owns 128 weight rows (output columns) and runs its whole K
// range (input projection), or 64 rows and one K piece (output projection,
// whose 48 column blocks are too few to keep the CUs streaming).  Its waves
// own 32 rows each and share the activation tile; every token of the sequence sits in
// the MFMAs' other operand (up to 5 blocks of 32).  The loads go straight to
// LDS through a 4-stage ring.  The epilogues run in the same kernel:
//  * input projection: a 128-row block is one q or k head (per-head RMSNorm
//    with the learnable scale, then the 4-axis RoPE, 32 dims per axis: the
//    miles page "FLUX 3 Image Klein", section 3; "How it works"), a v head,
//    or 64 hidden units of the MLP (gate and up rows of the same units, so
//    the SwiGLU product is formed in registers);
//  * output projection: the pieces of a column block store fp32 partials and
//    count themselves in; the last to arrive sums all pieces in piece order
//    (bitwise reproducible) and applies y = x + gate_s r.
#include "common.h"
#include "kernels.h"

namespace dit {
namespace {

constexpr int TBK = 64;   // k per LDS tile: rows of 128 bytes
constexpr int TNS = 4;    // ring stages
constexpr int kScopeDevice = 16;  // cache-policy bits of device-scope (sc1) buffer accesses
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

enum { TH_IN = 0, TH_OUT = 1 };

struct ThinArgs {
  const uint16_t* A;  // activations [M, K]
  const uint16_t* W;  // weights, rows of K
  int M, K, KT;       // KT = K / 64, a multiple of TNS
  int D, F, H;
  int n_cb;           // column blocks (128 weight rows in, 64 out)
  int pieces;         // K pieces per column block
  // input projection
  uint16_t* q;
  uint16_t* k;
  uint16_t* v;
  uint16_t* cat;      // m goes to columns [D, D + F) of rows of D + F
  const int32_t* pos;
  const uint16_t* q_scale;
  const uint16_t* k_scale;
  float qk_eps;
  float q_mul;
  double rope_rev[16];  // theta^(-2j / 32) / (2 pi)
  // output projection
  const uint16_t* x;
  const uint16_t* mod;
  uint16_t* y;
  int e0, e1;
  uint32_t flags;
  float* partial;
  int* counters;      // n_cb, zero at launch; each is reset by its last arriver
};

// 16-byte chunk c of LDS row r sits at chunk c ^ ((r >> 1) & 7): the 16 rows
// one fragment read touches then land on 16 distinct bank slots (a row of
// 128 B covers half of the 64 banks).
__device__ __forceinline__ int tswz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ float silu_hw(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

__device__ __forceinline__ uint2 pack4f(float a, float b, float c, float d) {
  return make_uint2(pack2(a, b), pack2(c, d));
}

// weight row feeding row r of column block cb (BNW rows per block)
template <int EPI, int BNW>
__device__ __forceinline__ int thin_weight_row(const ThinArgs& g, int cb, int r) {
  if (EPI == TH_IN) {
    const int n_qkv = 3 * g.H;
    if (cb < n_qkv) return cb * BNW + r;
    // 64 hidden units: wave w's 32 rows are 16 gate rows, then the up rows
    // of the same 16 units
    const int w = r >> 5, i = r & 31;
    return 3 * g.D + (i >= 16 ? g.F : 0) + (cb - n_qkv) * 64 + 16 * w + (i & 15);
  }
  return cb * BNW + r;
}

// NWV waves of 32 weight rows each: 4 (128 rows, a whole head) for the input
// projection, 2 for the output projection, whose last-arriving piece then
// sums half as many partial rows.
template <int EPI, int MB, int NWV>
__global__ __launch_bounds__(64 * NWV, 1) void thin_kernel(ThinArgs g) {
  constexpr int BNW = 32 * NWV;  // weight rows per workgroup
  static_assert(EPI == TH_OUT || NWV == 4, "a q / k block is one 128-dim head");
  // one LDS array per stage (see the big GEMM: the compiler then knows the
  // fragment reads of one stage do not alias the loads into the others)
  __shared__ __attribute__((aligned(16))) uint16_t s_w0[BNW * TBK];
  __shared__ __attribute__((aligned(16))) uint16_t s_w1[BNW * TBK];
  __shared__ __attribute__((aligned(16))) uint16_t s_w2[BNW * TBK];
  __shared__ __attribute__((aligned(16))) uint16_t s_w3[BNW * TBK];
  __shared__ __attribute__((aligned(16))) uint16_t s_a0[MB * 32 * TBK];
  __shared__ __attribute__((aligned(16))) uint16_t s_a1[MB * 32 * TBK];
  __shared__ __attribute__((aligned(16))) uint16_t s_a2[MB * 32 * TBK];
  __shared__ __attribute__((aligned(16))) uint16_t s_a3[MB * 32 * TBK];
  __shared__ float s_ss[4][MB * 32];
  __shared__ int s_arrival;
  uint16_t* const ring_w[TNS] = {s_w0, s_w1, s_w2, s_w3};
  uint16_t* const ring_a[TNS] = {s_a0, s_a1, s_a2, s_a3};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, hl = lane >> 5;

  // item = piece * n_cb + cb: the column blocks of one piece (which read the
  // same activation columns) sit next to each other, on one XCD
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int piece = item / g.n_cb, cb = item - piece * g.n_cb;
  const int units = g.KT / TNS;
  const int k0 = (int)((long long)piece * units / g.pieces) * TNS;
  const int k1 = (int)((long long)(piece + 1) * units / g.pieces) * TNS;

  // Direct-to-LDS loads: one wave instruction fills 1 KB = 8 rows of 128 B;
  // lane i lands in row 8 s + i / 8 at physical chunk i % 8, so it fetches
  // logical chunk (i % 8) ^ tswz(row).  Wave w fills W slabs 4 w .. 4 w + 3
  // and activation slabs MB w .. MB w + MB - 1.  Activation rows past M
  // reload row M - 1 (their outputs are dropped).
  const int lrow = lane >> 3, lch = lane & 7;
  const uint32_t rowb = (uint32_t)g.K * 2u;
  // fixed bounds (not MB): an array of template-dependent type would make
  // the direct-load builtins dependent, and the host pass would then drop the
  // kernel's host stub
  constexpr int AJ = 4 * MB / NWV;  // activation slabs per wave
  uint32_t woff[4], aoff[16];
  static_assert(AJ * NWV == 4 * MB && AJ <= 16, "activation load offsets");
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = (4 * wave + j) * 8 + lrow;
    woff[j] = (uint32_t)thin_weight_row<EPI, BNW>(g, cb, r) * rowb +
              (uint32_t)((lch ^ tswz(r)) * 16);
  }
#pragma unroll
  for (int j = 0; j < AJ; ++j) {
    const int r = (AJ * wave + j) * 8 + lrow;
    aoff[j] = (uint32_t)min(r, g.M - 1) * rowb + (uint32_t)((lch ^ tswz(r)) * 16);
  }
  const char* wbase = reinterpret_cast<const char*>(g.W);
  const char* abase = reinterpret_cast<const char*>(g.A);
  // k tile kt into ring stage st; past k1 the last tile is reloaded into a
  // stage that is never read, so every iteration issues the same loads
  auto gload = [&](int kt, int st) __attribute__((always_inline)) {
    const uint32_t ko = (uint32_t)min(kt, k1 - 1) * (TBK * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(wbase + (woff[j] + ko),
                                       (lds_ptr)(ring_w[st] + (4 * wave + j) * 8 * TBK), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < AJ; ++j)
      __builtin_amdgcn_global_load_lds(abase + (aoff[j] + ko),
                                       (lds_ptr)(ring_a[st] + (AJ * wave + j) * 8 * TBK), 16, 0, 0);
  };
  constexpr int NLD = 4 + AJ;  // loads per wave per stage
  // s_waitcnt with vmcnt(n) only (expcnt, lgkmcnt left alone)
  constexpr int VM_WAIT = ((TNS - 2) * NLD & 15) | (((TNS - 2) * NLD >> 4) << 14) | 0x0F70;

  f32x16 acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  auto frag = [&](const uint16_t* base, int r, int c) __attribute__((always_inline)) {
    return __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + r * 128 +
                                                ((c ^ tswz(r)) << 4)));
  };
  // one k tile from stage st: 4 k steps of MB MFMAs (C^T = W A^T: lane
  // (ln, hl) then holds token 32 i + ln and weight rows 32 w + 8 rr + 4 hl + e
  // in register 4 rr + e of acc[i])
  auto ktile = [&](int kt, int st) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(VM_WAIT);  // tile kt has landed (this wave's loads)
    __builtin_amdgcn_s_waitcnt(0xC07F);   // this wave's reads of the stage refilled next are done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    gload(kt + TNS - 1, (st + TNS - 1) % TNS);
    bf16x8 fw[4], fa[4][MB];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      fw[ks] = frag(ring_w[st], 32 * wave + ln, 2 * ks + hl);
#pragma unroll
      for (int i = 0; i < MB; ++i) fa[ks][i] = frag(ring_a[st], 32 * i + ln, 2 * ks + hl);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < MB; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[ks], fa[ks][i], acc[i], 0, 0, 0);
  };

#pragma unroll
  for (int s = 0; s < TNS - 1; ++s) gload(k0 + s, s);
  for (int kt = k0; kt < k1; kt += TNS) {
#pragma unroll
    for (int s = 0; s < TNS; ++s) ktile(kt + s, s);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load into LDS still in flight

  if constexpr (EPI == TH_IN) {
    const int n_h = g.H;
    if (cb < 2 * n_h) {
      // q or k head cb % H: RMSNorm over its 128 dims (spread over the 4
      // waves), scale, then RoPE; wave w holds axis w, lane dims 8 rr + 4 hl
      // + e of it, pair 4 rr + 2 hl + e / 2
      const bool is_k = cb >= n_h;
      const int head = is_k ? cb - n_h : cb;
      const uint16_t* sc = is_k ? g.k_scale : g.q_scale;
      const float qmul = is_k ? 1.0f : g.q_mul;
      uint16_t* const dst = (is_k ? g.k : g.q) + head * 128 + 32 * wave + 4 * hl;
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        float ss = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) ss = fmaf(acc[i][r], acc[i][r], ss);
        ss += __shfl_xor(ss, 32, 64);
        s_ss[wave][32 * i + ln] = ss;  // both half-waves: same sum, same address
      }
      uint2 gsc[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        gsc[rr] = *reinterpret_cast<const uint2*>(sc + 32 * wave + 8 * rr + 4 * hl);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int t = 32 * i + ln;
        if (t >= g.M) continue;
        const float ss = s_ss[0][t] + s_ss[1][t] + s_ss[2][t] + s_ss[3][t];
        const float rstd = rsqrtf(ss * (1.0f / 128.0f) + g.qk_eps) * qmul;
        const double p = (double)g.pos[4 * t + wave];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const uint2 gs = gsc[rr];
          const float xv[4] = {acc[i][4 * rr] * rstd * lo2f(gs.x),
                               acc[i][4 * rr + 1] * rstd * hi2f(gs.x),
                               acc[i][4 * rr + 2] * rstd * lo2f(gs.y),
                               acc[i][4 * rr + 3] * rstd * hi2f(gs.y)};
          float yv[4];
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            // turn count reduced to [0, 1) in double, then sin / cos of 2 pi r
            const double tt = p * g.rope_rev[4 * rr + 2 * hl + pr];
            const float rv = (float)(tt - floor(tt));
            const float sn = __builtin_amdgcn_sinf(rv), cs = __builtin_amdgcn_cosf(rv);
            yv[2 * pr] = xv[2 * pr] * cs - xv[2 * pr + 1] * sn;
            yv[2 * pr + 1] = xv[2 * pr] * sn + xv[2 * pr + 1] * cs;
          }
          *reinterpret_cast<uint2*>(dst + (size_t)t * g.D + 8 * rr) =
              pack4f(yv[0], yv[1], yv[2], yv[3]);
        }
      }
    } else if (cb < 3 * n_h) {
      uint16_t* const dst = g.v + (cb - 2 * n_h) * 128 + 32 * wave + 4 * hl;
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int t = 32 * i + ln;
        if (t >= g.M) continue;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          *reinterpret_cast<uint2*>(dst + (size_t)t * g.D + 8 * rr) =
              pack4f(acc[i][4 * rr], acc[i][4 * rr + 1], acc[i][4 * rr + 2], acc[i][4 * rr + 3]);
      }
    } else {
      // registers 4 rr + e (rr = 0, 1) are gate rows 8 rr + 4 hl + e of the
      // wave's 16 units, registers 4 (rr + 2) + e the up rows of the same units
      uint16_t* const dst = g.cat + g.D + (cb - 3 * n_h) * 64 + 16 * wave + 4 * hl;
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int t = 32 * i + ln;
        if (t >= g.M) continue;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const f32x16& a = acc[i];
          *reinterpret_cast<uint2*>(dst + (size_t)t * (g.D + g.F) + 8 * rr) =
              pack4f(silu_hw(a[4 * rr]) * a[4 * rr + 8], silu_hw(a[4 * rr + 1]) * a[4 * rr + 9],
                     silu_hw(a[4 * rr + 2]) * a[4 * rr + 10],
                     silu_hw(a[4 * rr + 3]) * a[4 * rr + 11]);
        }
      }
    }
  } else {
    // y = x + gate_s r (flags: bit 0 no residual, bit 1 no gate).  The gate
    // and residual are loaded before the pieces count themselves in, so the
    // last to arrive (the launch's tail) does not wait for them after its sum.
    const bool use_gate = !(g.flags & 2u), use_res = !(g.flags & 1u);
    const int c0 = cb * BNW + 32 * wave + 4 * hl;
    uint2 gv[MB][4], xv[MB][4];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int t = min(32 * i + ln, g.M - 1);
      const uint16_t* gate = g.mod + (size_t)stream_of(t, g.e0, g.e1) * 3 * g.D + 2 * g.D + c0;
      const uint16_t* xr = g.x + (size_t)t * g.D + c0;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        gv[i][rr] = use_gate ? *reinterpret_cast<const uint2*>(gate + 8 * rr)
                             : make_uint2(0x3f803f80u, 0x3f803f80u);
        xv[i][rr] = use_res ? *reinterpret_cast<const uint2*>(xr + 8 * rr) : make_uint2(0u, 0u);
      }
    }
    if (g.pieces > 1) {
      // Partials: slot (cb, piece), 4 waves x MB x 4 groups of 16 B x 64
      // lanes, lane-fastest so a wave store moves 1 KB.  The pieces of a
      // column block may run on different XCDs, whose L2s are not coherent:
      // device-scope (sc1) stores and loads go to the device's coherence
      // point, and every wave's stores complete before the barrier that
      // precedes the count.
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          g.partial, 0, (int)((size_t)g.n_cb * g.pieces * NWV * MB * 4 * 64 * 16), 0x00020000);
      auto goff = [&](int slot, int i, int rr) __attribute__((always_inline)) {
        return (int)(((((slot * NWV + wave) * MB + i) * 4 + rr) * 64 + lane) * 16);
      };
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const f32x4 w4 = {acc[i][4 * rr], acc[i][4 * rr + 1], acc[i][4 * rr + 2],
                            acc[i][4 * rr + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, w4), rsrc,
                                                 goff(cb * g.pieces + piece, i, rr), 0,
                                                 kScopeDevice);
        }
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (tid == 0)
        s_arrival = __hip_atomic_fetch_add(&g.counters[cb], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (__builtin_amdgcn_readfirstlane(s_arrival) != g.pieces - 1) return;
      if (tid == 0)  // ready for the next launch
        __hip_atomic_store(&g.counters[cb], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // the sum in piece order, this piece's own part from registers
      f32x16 sum[MB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum[i][r] = 0.f;
      for (int pc = 0; pc < g.pieces; ++pc) {
        if (pc == piece) {
#pragma unroll
          for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum[i][r] += acc[i][r];
          continue;
        }
        f32x4 part[MB][4];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            part[i][rr] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, goff(cb * g.pieces + pc, i, rr),
                                                             0, kScopeDevice));
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int e = 0; e < 4; ++e) sum[i][4 * rr + e] += part[i][rr][e];
      }
#pragma unroll
      for (int i = 0; i < MB; ++i) acc[i] = sum[i];
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int t = 32 * i + ln;
      if (t >= g.M) continue;
      uint16_t* yr = g.y + (size_t)t * g.D + c0;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        *reinterpret_cast<uint2*>(yr + 8 * rr) =
            pack4f(fmaf(lo2f(gv[i][rr].x), acc[i][4 * rr], lo2f(xv[i][rr].x)),
                   fmaf(hi2f(gv[i][rr].x), acc[i][4 * rr + 1], hi2f(xv[i][rr].x)),
                   fmaf(lo2f(gv[i][rr].y), acc[i][4 * rr + 2], lo2f(xv[i][rr].y)),
                   fmaf(hi2f(gv[i][rr].y), acc[i][4 * rr + 3], hi2f(xv[i][rr].y)));
    }
  }
}

template <int EPI, int NWV>
hipError_t launch_thin(const ThinArgs& g, hipStream_t stream) {
  const dim3 grid(g.n_cb * g.pieces), block(64 * NWV);
  switch ((g.M + 31) / 32) {
    case 1: hipLaunchKernelGGL((thin_kernel<EPI, 1, NWV>), grid, block, 0, stream, g); break;
    case 2: hipLaunchKernelGGL((thin_kernel<EPI, 2, NWV>), grid, block, 0, stream, g); break;
    case 3: hipLaunchKernelGGL((thin_kernel<EPI, 3, NWV>), grid, block, 0, stream, g); break;
    case 4: hipLaunchKernelGGL((thin_kernel<EPI, 4, NWV>), grid, block, 0, stream, g); break;
    default: hipLaunchKernelGGL((thin_kernel<EPI, 5, NWV>), grid, block, 0, stream, g); break;
  }
  return hipGetLastError();
}

// Rows per workgroup of the output projection (2 waves of 32).
constexpr int kOutRows = 64;

}  // namespace

bool thin_fits(int M, int D, int F) {
  return M >= 1 && M <= kThinMaxTokens && D % 128 == 0 && F % 64 == 0 && D % (TBK * TNS) == 0 &&
         (D + F) % (TBK * TNS) == 0;
}

size_t thin_partial_bytes(int M, int D, int pieces) {
  // per piece and 32 output columns: a wave's 4 KB groups for each token block
  return (size_t)(D / 32) * pieces * ((M + 31) / 32) * 4 * 64 * 16;
}

hipError_t launch_thin_in(const uint16_t* u, const uint16_t* w_in, int M, int D, int F,
                          uint16_t* q, uint16_t* k, uint16_t* v, uint16_t* cat,
                          const int32_t* pos, const uint16_t* q_scale, const uint16_t* k_scale,
                          float theta, float qk_eps, float q_mul, hipStream_t stream) {
  ThinArgs g{};
  g.A = u;
  g.W = w_in;
  g.M = M;
  g.K = D;
  g.KT = D / TBK;
  g.D = D;
  g.F = F;
  g.H = D / 128;
  g.n_cb = 3 * g.H + F / 64;
  g.pieces = 1;
  g.q = q;
  g.k = k;
  g.v = v;
  g.cat = cat;
  g.pos = pos;
  g.q_scale = q_scale;
  g.k_scale = k_scale;
  g.qk_eps = qk_eps;
  g.q_mul = q_mul;
  const double two_pi = 6.283185307179586;
  for (int j = 0; j < 16; ++j) g.rope_rev[j] = pow((double)theta, -2.0 * j / 32.0) / two_pi;
  return launch_thin<TH_IN, 4>(g, stream);
}

int thin_out_pieces(int D, int F) {
  const int n_cb = D / kOutRows, units = (D + F) / (TBK * TNS);
  // one round of workgroups (a second round would repeat the whole stream time)
  int p = device_cus() / n_cb;
  if (p > units) p = units;
  if (p > kThinMaxPieces) p = kThinMaxPieces;
  return p < 1 ? 1 : p;
}

hipError_t launch_thin_out(const uint16_t* cat, const uint16_t* w_out, int M, int D, int F,
                           const uint16_t* x, const uint16_t* mod, uint16_t* y, int e0, int e1,
                           uint32_t flags, float* partial, size_t partial_bytes, int* counters,
                           int n_counters, hipStream_t stream) {
  ThinArgs g{};
  g.A = cat;
  g.W = w_out;
  g.M = M;
  g.K = D + F;
  g.KT = (D + F) / TBK;
  g.D = D;
  g.F = F;
  g.H = D / 128;
  g.n_cb = D / kOutRows;
  g.pieces = thin_out_pieces(D, F);
  while (g.pieces > 1 &&
         (thin_partial_bytes(M, D, g.pieces) > partial_bytes || g.n_cb > n_counters))
    --g.pieces;
  g.x = x;
  g.mod = mod;
  g.y = y;
  g.e0 = e0;
  g.e1 = e1;
  g.flags = flags;
  g.partial = partial;
  g.counters = counters;
  return launch_thin<TH_OUT, kOutRows / 32>(g, stream);
}

}  // namespace dit
