// Full joint attention, o = softmax(q k^T * scale) v per head, flash style.
//
// Source: "Welcome FLUX.3 Image Klein in Diffusers", section "How it works"
// (the 28 joint blocks run full attention over the concatenated streams,
// prompt padding included) and the miles page "FLUX 3 Image Klein", section 3
// (the DiT takes no padding mask).  No mask is applied.
//
// Design (gfx950, 64-wide waves, 32x32x16 bf16 MFMA, 64-bank LDS):
//  * A workgroup is one head x 256 queries; each of its 8 waves owns 32
//    queries for the whole key loop.  Keys stream through LDS in tiles of 64;
//    K and V go from HBM/L2 straight into LDS with the 16-byte direct-to-LDS
//    loads, no staging registers.  A workgroup serves as many queries as 2
//    waves per SIMD allow, so one K/V tile feeds 256 queries (measured
//    faster than 128).
//  * Scores are computed transposed, S^T = K Q^T (A = K from LDS, B = Q held
//    in registers).  In the 32x32 MFMA result a lane holds one column, so
//    each lane owns one query: row max and row sum are in-lane reductions
//    plus one exchange with the other half-wave.
//  * The K rows fed to the A operand are permuted (key_slot) so that the 16
//    scores a lane holds are exactly the 16 keys it supplies as the B operand
//    of O^T = V^T P^T.  P never leaves registers.
//  * V stays row-major [key][dim] in LDS; the A operand V^T of the PV MFMA is
//    read with gfx950's transposing LDS read (ds_read_b64_tr_b16): each lane
//    fetches 4 dims of one key and the hardware hands every lane 4 keys of one
//    dim.
//  * Online softmax in fp32 with the hardware exp2 (v_exp_f32; results below
//    2^-126 flush to zero, far under bf16 resolution of P), scale * log2 e
//    folded into one FMA.
//    The running max is only moved (and O, l rescaled) when a row's max grows
//    by more than 2^8; otherwise the stale max is kept, which bounds P by 2^8
//    and leaves the result unchanged (P and l share the same reference).  P is
//    rounded to bf16 for the MFMA; one division by the row sum at the end.
//  * Fixed reference: inside the block, q and k leave the QK RMSNorm with
//    known scales, which bound every score, and q is stored already
//    multiplied by the softmax scale times log2 e.  When the bound is small
//    (at most 40 in log2 units, as for scales near one) the weights are
//    exp2 of the raw scores with no reference: the row max, the rescale
//    checks and the FMA before each exp drop out of the loop.  Each tile's
//    softmax is then split in halves over both MFMA steps (see run_fixed).
//    Together about 20% of the kernel's time at 4,256 tokens.
//  * Work split.  The work is the grid of (head, 256-query tile, 64-key
//    tile) iterations, heads outermost.  When there are more (head, query
//    tile) items than CUs, one workgroup per CU takes an equal contiguous
//    share of the iterations, so no last round of whole items leaves CUs
//    idle (at 4,256 tokens the 408 items are 1.59 rounds of 256 CUs).  A
//    share can end part-way through an item; since every share is at least
//    one item long, an item is cut at most once, between two neighbouring
//    workgroups.  Each part stores its unnormalized output, row sums and row
//    max (fp32) to a scratch slot of the workspace and counts itself in on
//    the slot's counter; whichever part arrives second reads the other's
//    partial, merges it (the two parts' weights share no reference, so the
//    merge rescales by exp2 of their max differences; with the fixed
//    reference below it is a plain sum) and stores o.  No workgroup ever
//    waits for another, and the merge is symmetric in the two parts, so the
//    result does not depend on which arrives first.  With at most as many
//    items as CUs (or no scratch) each workgroup runs one whole item.
//  * Whole-item rounds.  With at least two rounds of items, only the last
//    round and the remainder (between one and two rounds) are split into
//    shares; before that every workgroup runs whole items round by round,
//    workgroup w taking item round * G + w.  Shares that start part-way
//    through an item put each CU at its own key position, so on a long
//    sequence every CU streamed its head's K and V on its own (52 GB from
//    behind L2 per launch at 32,928 tokens, where one head's K and V are
//    17 MB against a 4 MB L2); in whole-item rounds the 32 CUs of an XCD
//    start together on consecutive query tiles of one head and read each
//    key tile at about the same time.  Sequences of at most two rounds
//    (4,256 tokens: 1.59) are split as before.
//  * Shares of neighbouring workgroups sit on one XCD (and so do the items of
//    one head), so K and V and the split partials stay in that XCD's L2.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace dit {

namespace {

constexpr int NWAVE = 8;  // waves per workgroup (32 queries each)
constexpr int BQ = 32 * NWAVE;  // queries per workgroup
constexpr int BKEY = 64;  // keys per tile
constexpr int LPW = BKEY / 4 / NWAVE;  // 1 KB loads per wave per K (or V) tile
constexpr int HD = 128;   // head dim
constexpr float RESCALE_LOG2 = 8.f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4;

// gfx950's LDS has 64 banks of 4 B; a 16-byte access serves 16 lanes per
// cycle (256 B), an 8-byte one 32 lanes.
// K tile [64 keys][128 dims], rows of 256 B = 16 chunks of 16 B: the 16 lanes
// of an A read hit 16 different rows at one logical chunk, so the chunk is
// xor-ed with the row's low 4 bits.
__device__ __forceinline__ int kswz(int row) { return row & 15; }
// V tile [64 keys][128 dims], rows of 256 B = 4 segments of 64 B (32 dims):
// a 32-lane half of a transposing read touches 4 consecutive rows at one
// segment, so the segment is xor-ed with the row's low 2 bits.
__device__ __forceinline__ int vswz(int row) { return row & 3; }

// Key held by A-operand row m of a 32-key block (m = 8r + 4h + j maps to
// 16(r/2) + 8h + 4(r%2) + j): with this order the MFMA output register
// 4r + j of half-wave h is the key the PV MFMA wants in B slot 8(r%2) + j
// of k-step r/2.
__device__ __forceinline__ int key_slot(int m) {
  const int r = m >> 3, h = (m >> 2) & 1, j = m & 3;
  return 16 * (r >> 1) + 8 * h + 4 * (r & 1) + j;
}

// s_waitcnt immediates: vmcnt(4) / vmcnt(0), expcnt and lgkmcnt left alone
constexpr int vmcnt_imm_lpw() { return LPW | 0x0F70; }
constexpr int vmcnt_imm0() { return 0x0F70; }

// Workgroup barrier that does not wait for outstanding vector-memory loads
// (__syncthreads() waits for all of them, the whole prefetch ring); LDS
// reads are completed first so a slot can be refilled after it.  The empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_keep_loads() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Split partials: a part is NWAVE waves x PGROUPS 16-byte groups x 64 lanes
// (a lane's 64 accumulators, then its row sum l and row max m), group-major
// per wave so each wave store or load moves 1 KB contiguously.  Slot s (the
// boundary between shares s - 1 and s) holds the two parts of the item cut
// there: part 0 the keys before the cut, part 1 the keys after it.
constexpr int PGROUPS = 17;
// cache-policy bits of the buffer loads and stores: device scope (sc1)
constexpr int kScopeDevice = 16;
typedef int i32x4 __attribute__((ext_vector_type(4)));

}  // namespace

__global__ __launch_bounds__(64 * NWAVE, 1) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, int N, int H, int ld_qkv,
    int ld_o, float c, float c_bound, const uint16_t* __restrict__ q_scale,
    const uint16_t* __restrict__ k_scale, int prescaled, void* __restrict__ part,
    int part_bytes, int* __restrict__ cnt) {
  // distinct arrays per stage: reads of one stage never wait on the
  // direct-to-LDS loads in flight into the other
  __shared__ __attribute__((aligned(16))) uint16_t s_k0[BKEY * HD];
  __shared__ __attribute__((aligned(16))) uint16_t s_v0[BKEY * HD];
  __shared__ __attribute__((aligned(16))) uint16_t s_k1[BKEY * HD];
  __shared__ __attribute__((aligned(16))) uint16_t s_v1[BKEY * HD];
  __shared__ int s_arrival;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, hl = lane >> 5;
  const int nqt = (N + BQ - 1) / BQ;
  const int ntiles = (N + BKEY - 1) / BKEY;
  // This workgroup's share [b0, b1) of the nqt * H * ntiles iterations
  // (item = head * nqt + query tile, then key tile).  With one share per item
  // (gridDim.x == nqt * H) every share is exactly one whole item.
  const int G = gridDim.x;
  const int r = xcd_remap(blockIdx.x, G);
  const int items = nqt * H;
  // R whole-item rounds first (none with one workgroup per item, G = items),
  // then the share [b0, b1) of the iterations after them
  const int R = items >= 2 * G ? items / G - 1 : 0;
  const long long split_from = (long long)R * G * ntiles;
  const long long total = (long long)items * ntiles;
  const long long b0 = split_from + (total - split_from) * r / G;
  const long long b1 = split_from + (total - split_from) * (r + 1) / G;
  const long long whole = (long long)R * ntiles;  // iterations of the whole-item rounds

  // Per-segment state read by the loops below: the head's K and V, the first
  // key tile kt0 and tile count nt of the segment, and the number of keys
  // that count in its last tile (lim_seg < 64 only in the last tile of a
  // ragged N).
  const char* kbase;
  const char* vbase;
  int kt0 = 0, nt = 0, lim_seg = BKEY;
  bf16x8 qf[8];

  // Direct-to-LDS loads: a wave instruction fills 1 KB = 4 rows of 256 B;
  // lane i lands in row 4 j' + i / 16 at physical chunk i % 16.  Wave w
  // fills rows [4 LPW w, 4 LPW (w + 1)) of a tile.
  const int prow = lane >> 4, pch = lane & 15;
  // byte offsets of the chunk this lane fetches for slab j (recomputed per
  // load: a few integer ops instead of 8 live registers)
  auto kch = [&](int j) __attribute__((always_inline)) {
    return (uint32_t)((pch ^ kswz(wave * 4 * LPW + 4 * j + prow)) * 16);
  };
  auto vch = [&](int j) __attribute__((always_inline)) {
    return (uint32_t)(((((pch >> 2) ^ vswz(wave * 4 * LPW + 4 * j + prow)) << 2) | (pch & 3)) * 16);
  };
  const uint32_t row_bytes = (uint32_t)ld_qkv * 2u;
  // tile t of the segment (key tile kt0 + t); tiles past the end of the
  // sequence reload the last one into an idle slot (never read), tiles past
  // the segment's end load real keys that are never read either
  auto dma_k = [&](int t, uint16_t* sk) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int rw = wave * 4 * LPW + 4 * j + prow;
      const uint32_t key = (uint32_t)min(min(kt0 + t, ntiles - 1) * BKEY + rw, N - 1);
      __builtin_amdgcn_global_load_lds(kbase + (key * row_bytes + kch(j)),
                                       (lds_ptr)(sk + (wave * 4 * LPW + 4 * j) * HD), 16, 0, 0);
    }
  };
  auto dma_v = [&](int t, uint16_t* sv) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int rw = wave * 4 * LPW + 4 * j + prow;
      const uint32_t key = (uint32_t)min(min(kt0 + t, ntiles - 1) * BKEY + rw, N - 1);
      __builtin_amdgcn_global_load_lds(vbase + (key * row_bytes + vch(j)),
                                       (lds_ptr)(sv + (wave * 4 * LPW + 4 * j) * HD), 16, 0, 0);
    }
  };

  // per-lane LDS read offsets (bytes) that do not change from tile to tile
  const int krow = key_slot(ln);  // + 32 kb
  uint32_t koff[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) koff[st] = krow * 256 + (((2 * st + hl) ^ kswz(krow)) << 4);
  // transposing V read: 16-lane group g covers dims 16 (g & 1) .. + 15 of the
  // 32-dim block and keys 8 (g >> 1) + 4 u .. + 3 of the 16-key step (u = 0, 1);
  // lane i of the group reads key (i >> 2), dims 4 (i & 3) .. + 3
  const int g = lane >> 4, gi = lane & 15;
  const int vrow = 8 * (g >> 1) + (gi >> 2);
  uint32_t voff[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
    voff[d] = vrow * 256 + ((d ^ vswz(vrow)) << 6) + (16 * (g & 1) + 4 * (gi & 3)) * 2;

  f32x16 acc[4];
  float m_run;  // running max, already multiplied by c
  float l_run;

  // Fixed reference.  When q and k come out of the block's QK RMSNorm with
  // scales g_q, g_k, every row has |q| <= sqrt(128) max|g_q| (and likewise
  // for k; RoPE keeps norms, the bf16 rounding adds under 1%), so every
  // scaled score S c lies within +-B, B = c 128 max|g_q| max|g_k| (1.01 for
  // the rounding; c = c_bound, the softmax scale times log2 e).  The block
  // stores q already multiplied by c (prescaled; then c = 1 here), and with
  // B <= 40 the kernel takes P = exp2(S) with no reference at all: the
  // weights lie in [2^-40, 2^40], far inside fp32 and bf16 range, the row
  // sums stay below 2^57, and the normalization at the end cancels the
  // common factor.  The FMA before each exp, the row max and the rescale
  // checks drop out of the loop.  Larger bounds, and attention without
  // scales, use the running max.
  bool fixed = false;
  if (q_scale != nullptr && prescaled) {
    float gq = fmaxf(fabsf(bf2f(q_scale[lane])), fabsf(bf2f(q_scale[lane + 64])));
    float gk = fmaxf(fabsf(bf2f(k_scale[lane])), fabsf(bf2f(k_scale[lane + 64])));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      gq = fmaxf(gq, __shfl_xor(gq, off, 64));
      gk = fmaxf(gk, __shfl_xor(gk, off, 64));
    }
    const float bound = c_bound * 128.0f * gq * gk * 1.01f;
    // uniform over the workgroup (a wave-wide max); read as a scalar so the
    // branch on it is a scalar branch
    fixed = __builtin_amdgcn_readfirstlane(bound <= 40.0f ? 1 : 0) != 0;  // NaN: running max
  }

  // S^T = K Q^T for one key tile: 2 key blocks of 32, 8 k steps of 16 dims.
  // MFMA i (st = i / 2, kb = i % 2) alternates the two blocks' chains so
  // neither waits on itself; its K fragment was read one MFMA earlier.
  auto kfrag = [&](const char* skb, int i) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(skb + (i & 1) * 32 * 256 + koff[i >> 1]);
  };
  auto qk = [&](const uint16_t* sk, f32x16 (&sc)[2]) __attribute__((always_inline)) {
    const char* skb = reinterpret_cast<const char*>(sk);
    bf16x8 fk[2];
    fk[0] = kfrag(skb, 0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sc[kb][rr] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 1 < 16) fk[(i + 1) & 1] = kfrag(skb, i + 1);
      sc[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[i & 1], qf[i >> 1], sc[i & 1], 0, 0, 0);
    }
  };
  // row max of a tile's scores, times c.  In the last tile of a ragged N the
  // keys past N are copies of key N - 1 (the loads clamp), so they do not
  // change the max and need no mask here.
  auto row_max = [&](const f32x16 (&sc)[2]) __attribute__((always_inline)) {
    float mx = sc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, sc[kb][rr]);
    return fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
  };
  auto rescale = [&](float mx) __attribute__((always_inline)) {
    if (__any(mx > m_run + RESCALE_LOG2)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) acc[d][rr] *= alpha;
    }
  };
  // P = exp2(S c - m) in bf16 for the PV MFMA; with `lim` < 64 keys at local
  // index >= lim get no weight (the last tile of a ragged N)
  auto softmax = [&](const f32x16 (&sc)[2], bf16x8 (&pb)[4], int lim)
      __attribute__((always_inline)) {
    float psum = 0.f;
    // key index 32 kb + 16 (rr / 8) + 8 hl + rr % 8 against lim, with the
    // lane's part moved to the bound (no per-lane index constants)
    const int lim_l = lim - 8 * hl;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float p = __builtin_amdgcn_exp2f(fmaf(sc[kb][rr], c, -m_run));
        if (lim < BKEY && 32 * kb + 16 * (rr >> 3) + (rr & 7) >= lim_l) p = 0.f;
        psum += p;
        pb[2 * kb + (rr >> 3)][rr & 7] = (__bf16)p;
      }
    l_run += psum;
  };
  // O^T += V^T P^T.  The A operand of MFMA i (ks = i / 4, d = i % 4), 8 keys
  // of one dim per lane, is two transposing reads issued one MFMA earlier.
  auto vfrag = [&](const char* svb, int i) __attribute__((always_inline)) {
    const char* base = svb + (i >> 2) * 16 * 256 + voff[i & 3];
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(base));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(base + 4 * 256));
    const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, both);
  };
  auto pv = [&](const uint16_t* sv, const bf16x8 (&pb)[4]) __attribute__((always_inline)) {
    const char* svb = reinterpret_cast<const char*>(sv);
    bf16x8 fv[2];
    fv[0] = vfrag(svb, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 1 < 16) fv[(i + 1) & 1] = vfrag(svb, i + 1);
      acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv[i & 1], pb[i >> 2], acc[i & 3], 0, 0, 0);
    }
  };

  // the key loop of one segment with the running max
  auto run_online = [&]() __attribute__((always_inline)) {
    // Software pipeline over key tiles.  Iteration t holds S(t) and its row
    // max; it computes S(t + 1) = K(t + 1) Q^T while the softmax of S(t) runs
    // (MFMA and VALU of one wave overlap), then O += V(t) P(t) while the row
    // max of S(t + 1) runs.  K and V have separate 2-slot LDS rings: K(t + 3)
    // is loaded once every wave has read K(t + 1) (barrier B1), V(t + 2) once
    // every wave has read V(t) (barrier B2), so each load has about 1.5
    // iterations to land.  Before B2 a wave waits for K(t + 2) and V(t + 1);
    // only its K(t + 3) loads (the youngest LPW) may still fly.  The last tile
    // (softmax with the ragged-N mask, then PV) is peeled off the loop.
    uint16_t* const ring_k[2] = {s_k0, s_k1};
    uint16_t* const ring_v[2] = {s_v0, s_v1};
    f32x16 sa[2], sb[2];
    bf16x8 pb[4];
    float mx_a, mx_b;

    dma_k(0, s_k0);
    dma_v(0, s_v0);
    dma_k(1, s_k1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm_lpw());
    barrier_keep_loads();
    qk(s_k0, sa);
    mx_a = row_max(sa);
    dma_v(1, s_v1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm_lpw());
    barrier_keep_loads();
    dma_k(2, s_k0);

    // `slot` is t % 2 as a compile-time constant, so every LDS access names
    // its array statically (the compiler then never waits on the loads in
    // flight into the other slots)
    auto iter = [&](auto slot, int t, f32x16 (&cur)[2], float mx_cur, f32x16 (&nxt)[2],
                    float& mx_nxt) __attribute__((always_inline)) {
      constexpr int sl = decltype(slot)::value;
      rescale(mx_cur);
      // step 1: S(t + 1) MFMAs with softmax(t) VALU
      qk(ring_k[sl ^ 1], nxt);
      softmax(cur, pb, BKEY);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // first K fragment
  #pragma unroll
      for (int q = 0; q < 16; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // next K fragment
        __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);  // 7 VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      barrier_keep_loads();  // B1
      dma_k(t + 3, ring_k[sl ^ 1]);
      // step 2: O += V(t) P(t) with the row max of S(t + 1)
      pv(ring_v[sl], pb);
      mx_nxt = row_max(nxt);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // first V fragment
  #pragma unroll
      for (int q = 0; q < 16; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // next V fragment
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // 1 VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm_lpw());
      barrier_keep_loads();  // B2
      dma_v(t + 2, ring_v[sl]);
    };
    auto last = [&](auto slot, f32x16 (&cur)[2], float mx_cur) __attribute__((always_inline)) {
      constexpr int sl = decltype(slot)::value;
      rescale(mx_cur);
      softmax(cur, pb, lim_seg);
      pv(ring_v[sl], pb);
    };
    int t = 0;
    for (; t + 2 < nt; t += 2) {
      iter(std::integral_constant<int, 0>{}, t, sa, mx_a, sb, mx_b);
      iter(std::integral_constant<int, 1>{}, t + 1, sb, mx_b, sa, mx_a);
    }
    if (t + 1 < nt) {
      iter(std::integral_constant<int, 0>{}, t, sa, mx_a, sb, mx_b);
      last(std::integral_constant<int, 1>{}, sb, mx_b);
    } else {
      last(std::integral_constant<int, 0>{}, sa, mx_a);
    }
  };
  // The loop with the fixed reference.  With no running max a tile's
  // weights need nothing but its own scores, so the softmax of each tile is
  // split in its two 32-key halves: the second half of P(t) is computed in
  // step 1 beside the QK MFMAs of tile t + 1, the first half of P(t + 1) in
  // step 2 beside the PV MFMAs of tile t (which read the other register set
  // of first halves).  Both steps then carry VALU work under their MFMAs.
  // The first half of the last tile takes the ragged-N mask in the iteration
  // before it (MASK0), its second half in the peeled last step.
  auto run_fixed = [&]() __attribute__((always_inline)) {
    uint16_t* const ring_k[2] = {s_k0, s_k1};
    uint16_t* const ring_v[2] = {s_v0, s_v1};
    const int lim = lim_seg;
    // weights of one 32-key half (kb) of a tile into its two B fragments;
    // keys at tile index >= lim get none.  Returns the half's row sum.
    auto half = [&](const f32x16& sv, int kb, bf16x8 (&ph)[2], int lm)
        __attribute__((always_inline)) {
      float sum = 0.f;
      const int lm_l = lm - 8 * hl;  // the lane's part of the key index moved to the bound
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float p = __builtin_amdgcn_exp2f(sv[rr]);
        if (lm < BKEY && 32 * kb + 16 * (rr >> 3) + (rr & 7) >= lm_l) p = 0.f;
        sum += p;
        ph[rr >> 3][rr & 7] = (__bf16)p;
      }
      return sum;
    };
    auto pv2 = [&](const uint16_t* sv, const bf16x8 (&p0)[2], const bf16x8 (&p1)[2])
        __attribute__((always_inline)) {
      const char* svb = reinterpret_cast<const char*>(sv);
      bf16x8 fv[2];
      fv[0] = vfrag(svb, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + 1 < 16) fv[(i + 1) & 1] = vfrag(svb, i + 1);
        const bf16x8& pf = (i >> 3) ? p1[(i >> 2) & 1] : p0[(i >> 2) & 1];
        acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv[i & 1], pf, acc[i & 3], 0, 0, 0);
      }
    };
    f32x16 sa[2], sb[2];
    bf16x8 pa0[2], pb0[2], p1[2];

    dma_k(0, s_k0);
    dma_v(0, s_v0);
    dma_k(1, s_k1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm_lpw());
    barrier_keep_loads();
    qk(s_k0, sa);
    l_run = half(sa[0], 0, pa0, nt == 1 ? lim : BKEY);
    dma_v(1, s_v1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm_lpw());
    barrier_keep_loads();
    dma_k(2, s_k0);

    auto iter = [&](auto slot, auto mask0, int t, f32x16 (&cur)[2], f32x16 (&nxt)[2],
                    bf16x8 (&p0_cur)[2], bf16x8 (&p0_nxt)[2]) __attribute__((always_inline)) {
      constexpr int sl = decltype(slot)::value;
      constexpr bool MASK0 = decltype(mask0)::value;
      // step 1: S(t + 1) MFMAs with the second half of P(t)
      qk(ring_k[sl ^ 1], nxt);
      l_run += half(cur[1], 1, p1, BKEY);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // first K fragment
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // next K fragment
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // 3 VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      barrier_keep_loads();  // B1
      dma_k(t + 3, ring_k[sl ^ 1]);
      // step 2: O += V(t) P(t) with the first half of P(t + 1)
      pv2(ring_v[sl], p0_cur, p1);
      l_run += half(nxt[0], 0, p0_nxt, MASK0 ? lim : BKEY);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // first V fragment
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // next V fragment
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // 3 VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm_lpw());
      barrier_keep_loads();  // B2
      dma_v(t + 2, ring_v[sl]);
    };
    auto last = [&](auto slot, f32x16 (&cur)[2], bf16x8 (&p0_cur)[2])
        __attribute__((always_inline)) {
      constexpr int sl = decltype(slot)::value;
      l_run += half(cur[1], 1, p1, lim);
      pv2(ring_v[sl], p0_cur, p1);
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using NoMask = std::false_type;
    using Mask = std::true_type;
    int t = 0;
    for (; t + 3 < nt; t += 2) {
      iter(S0{}, NoMask{}, t, sa, sb, pa0, pb0);
      iter(S1{}, NoMask{}, t + 1, sb, sa, pb0, pa0);
    }
    if (t + 3 == nt) {
      iter(S0{}, NoMask{}, t, sa, sb, pa0, pb0);
      iter(S1{}, Mask{}, t + 1, sb, sa, pb0, pa0);
      last(S0{}, sa, pa0);
    } else if (t + 2 == nt) {
      iter(S0{}, Mask{}, t, sa, sb, pa0, pb0);
      last(S1{}, sb, pb0);
    } else {
      last(S0{}, sa, pa0);
    }
  };

  // The whole-item rounds, then the share, one segment (an item or the part
  // of one inside the share) at a time.  `done` counts this workgroup's
  // iterations: [0, whole) the whole-item rounds, then the share.
  for (long long done = 0; done < whole + (b1 - b0);) {
    const long long seg_start = done;
    int item, k0, k1;
    if (done < whole) {
      item = (int)(done / ntiles) * G + r;
      k0 = 0;
      k1 = ntiles;
    } else {
      const long long at = b0 + (done - whole);
      item = (int)(at / ntiles);
      k0 = (int)(at - (long long)item * ntiles);
      k1 = (int)min((long long)ntiles, b1 - (long long)item * ntiles);
    }
    done += k1 - k0;
    const int h = item / nqt, qt = item % nqt;
    const int q0 = qt * BQ + wave * 32;
    // every wave is done with the previous segment's LDS tiles before the
    // rings are refilled
    if (seg_start != 0) __syncthreads();
    kbase = reinterpret_cast<const char*>(k + (size_t)h * HD);
    vbase = reinterpret_cast<const char*>(v + (size_t)h * HD);
    kt0 = k0;
    nt = k1 - k0;
    lim_seg = k1 == ntiles ? N - (ntiles - 1) * BKEY : BKEY;

    // Q fragments (B operand of S^T = K Q^T): lane holds q[q0 + ln][16 s + 8 hl .. + 8]
    {
      const int qi = min(q0 + ln, N - 1);
      const uint4* qp = reinterpret_cast<const uint4*>(q + (size_t)qi * ld_qkv + (size_t)h * HD);
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[s] = __builtin_bit_cast(bf16x8, qp[2 * s + hl]);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) acc[d][rr] = 0.f;
    m_run = -INFINITY;
    l_run = 0.f;

    if (fixed)
      run_fixed();
    else
      run_online();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm0());

    if (k0 != 0 || k1 != ntiles) {
      // A part of a cut item: store it, count it in, and if the other part is
      // already in, merge it and finish the item here.
      const int slot = k0 != 0 ? r : r + 1;
      const int half_id = k0 != 0 ? 1 : 0;
      // The two parts may run on different XCDs, whose L2s are not
      // coherent, so the partials are stored and loaded with 16-byte
      // device-scope (sc1) buffer accesses, which write through to and read
      // from the device's coherence point; every wave's stores are complete
      // (vmcnt(0)) before the workgroup barrier that precedes the count, and
      // the other part's were before its count.  No cache-wide write-back or
      // invalidation is needed (per-wave fences that do both took attention
      // from 207 to 423 us).
      const __amdgpu_buffer_rsrc_t rsrc =
          __builtin_amdgcn_make_buffer_rsrc(part, 0, part_bytes, 0x00020000);
      auto group_off = [&](int hid, int gi) __attribute__((always_inline)) {
        return (int)(((((2 * slot + hid) * NWAVE + wave) * PGROUPS + gi) * 64 + lane) * 16);
      };
      auto st16 = [&](int gi, float a0, float a1, float a2, float a3)
          __attribute__((always_inline)) {
        const f32x4 w = {a0, a1, a2, a3};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, w), rsrc,
                                               group_off(half_id, gi), 0, kScopeDevice);
      };
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
          st16(4 * d + gq, acc[d][4 * gq], acc[d][4 * gq + 1], acc[d][4 * gq + 2],
               acc[d][4 * gq + 3]);
      st16(16, l_run, m_run, 0.f, 0.f);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm0());
      __syncthreads();
      if (tid == 0)
        s_arrival = __hip_atomic_fetch_add(&cnt[slot], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      // first in: the other part finishes the item
      if (__builtin_amdgcn_readfirstlane(s_arrival) == 0) continue;
      if (tid == 0)  // ready for the next launch
        __hip_atomic_store(&cnt[slot], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      auto ld16 = [&](int gi) __attribute__((always_inline)) {
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rsrc, group_off(half_id ^ 1, gi), 0, kScopeDevice));
      };
      const f32x4 lm = ld16(16);
      float sa = 1.f, sb = 1.f;
      if (!fixed) {
        // both parts' weights relative to the larger of their references;
        // the same expression for either order of arrival
        const float mm = fmaxf(m_run, lm[1]);
        sa = __builtin_amdgcn_exp2f(m_run - mm);
        sb = __builtin_amdgcn_exp2f(lm[1] - mm);
      }
      l_run = l_run * sa + lm[0] * sb;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const f32x4 w = ld16(4 * d + gq);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[d][4 * gq + e] = acc[d][4 * gq + e] * sa + w[e] * sb;
        }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.0f / l_tot;
    const int qi = q0 + ln;
    if (qi < N) {
      uint16_t* op = o + (size_t)qi * ld_o + (size_t)h * HD;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int dim = 32 * d + 8 * rr + 4 * hl;
          const uint32_t lo = pack2(acc[d][4 * rr] * inv, acc[d][4 * rr + 1] * inv);
          const uint32_t hi = pack2(acc[d][4 * rr + 2] * inv, acc[d][4 * rr + 3] * inv);
          *reinterpret_cast<uint2*>(op + dim) = make_uint2(lo, hi);
        }
    }
  }
}

__global__ void attn_clear_kernel(int* __restrict__ cnt, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    cnt[i] = 0;
}

size_t attn_split_bytes(int n_slots) {
  return (size_t)n_slots * 2 * NWAVE * PGROUPS * 64 * sizeof(float4);
}

hipError_t launch_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                       int N, int H, int ld_qkv, int ld_o, float softmax_scale,
                       const uint16_t* q_scale, const uint16_t* k_scale, int q_prescaled,
                       const AttnSplit* split, hipStream_t stream) {
  const int nqt = (N + BQ - 1) / BQ;
  const int items = nqt * H;
  int grid = items;
  void* part = nullptr;
  int part_bytes = 0;
  int* cnt = nullptr;
  if (split != nullptr) {
    // one share per CU, as many as the scratch has slots for
    int cap = device_cus();
    while (cap > 1 && (attn_split_bytes(cap) > split->part_bytes || cap > split->n_counters))
      --cap;
    if (items > cap && cap > 1) {
      grid = cap;
      part = split->part;
      part_bytes = (int)attn_split_bytes(grid);
      cnt = split->counters;
      if (split->clear) {
        hipLaunchKernelGGL(attn_clear_kernel, dim3(1), dim3(256), 0, stream, cnt, grid);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
    }
  }
  const float c = softmax_scale * DIT_LOG2E;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(grid), dim3(64 * NWAVE), 0, stream, q, k, v, o, N, H,
                     ld_qkv, ld_o, q_prescaled ? 1.0f : c, c, q_scale, k_scale, q_prescaled,
                     part, part_bytes, cnt);
  return hipGetLastError();
}

}  // namespace dit
