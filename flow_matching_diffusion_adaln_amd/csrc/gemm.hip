// bf16 MFMA GEMMs of the block, C = A W^T with both operands K-contiguous,
// with the block's epilogues fused in.
//
//  * Input projection: u [N, D] x W_in [3D + 2F, D]^T.  The to_q / to_k /
//    to_v / ff.linear_in projections (NeMo AutoModel page, section
//    "Image-Editing LoRA") read the same normalized input ("Welcome FLUX.3
//    Image Klein in Diffusers", section "How it works": attention and the MLP
//    run in parallel on it), so they are one GEMM.  Tiles over the q / k / v
//    rows store bf16 q, k, v; tiles over the MLP rows load gate and up rows
//    interleaved in 32-row groups, so one wave holds gate and up of the same
//    hidden units and writes m = silu(gate) * up straight into the [o | m]
//    buffer.  z = [q | k | v | gate | up] is never stored.
//  * Output projection: [o | m] [N, D + F] x W_out [D, D + F]^T, i.e. to_out.0
//    and ff.linear_out summed, with y = x + gate_s * r in the epilogue (one
//    gate per stream, "How it works": scale, shift and gate per stream).
//
// Tiling for gfx950: BM x 256 workgroup tiles with BM = 256 (4 waves in
// 2 x 2, 128 x 128 each) or BM = 224 (4 waves in 1 x 4, 224 x 64 each), and
// BM = 128 (1 x 4, 128 x 64) for split launches of at most 128 rows, built
// from v_mfma_f32_32x32x16_bf16 blocks with the fp32 accumulators in AGPRs.
// The host picks the tile height: fewest rounds of tiles over the CUs, then
// the shorter tile (224 divides the 4,256-token sequence into 19 tiles, 256
// leaves a 160-row remainder).  The K loop streams k tiles of 128 bytes per
// row (64 bf16) from L2/HBM straight into LDS with 16-byte direct-to-LDS
// loads: W in a double buffer, A in a triple buffer when the K loop's period
// allows it (loads of tile kt + 2 start during tile kt).  The 16-byte chunk
// index is xor-swizzled by the row so fragment reads are bank-conflict free.
// Tiles are ordered XCD-aware: each XCD takes one contiguous range of tiles,
// walked in groups of 4 N-tiles so the A and W panels in flight on one XCD
// stay few.
//
// FP8 mode (F8): the same kernel on OCP e4m3 operands with rowwise scales,
// the analogue of the rowwise-scaled FP8 ("fp8r") projections the SGLang
// FLUX.3 page ships.  A k tile is then 128 one-byte elements: the same
// 128-byte LDS rows, ring and swizzle, but 2 k steps of
// v_mfma_scale_f32_32x32x64_f8f6f4 (64 k, unit block scale) instead of 4 of
// the bf16 MFMA, so the MFMA time, LDS traffic and fragment reads per k tile
// are unchanged and the k tile carries twice the FLOPs.  The accumulators
// are multiplied by the A row's scale and the W row's scale before the
// epilogue, which is otherwise the bf16 one.
#include "common.h"
#include "kernels.h"

#include <atomic>
#include <type_traits>

namespace dit {

namespace {

constexpr int BN = 256, BK = 64;  // BK in bf16 elements: 128 bytes per tile row
constexpr int NW = 2;                // LDS slots for W k tiles (double buffer)
constexpr int CH = BK / 8;           // 16-byte chunks per tile row (8 = one 128-byte cache line)
constexpr int RPI = 64 / CH;         // tile rows filled by one 1 KB wave load (8)
constexpr int GROUP_N = 4;
constexpr int kMaxPieces = GEMM_MAX_SPLIT_PIECES;  // split pieces per launch (kernels.h)

enum { EPI_IN = 0, EPI_OUT = 1 };

struct GemmArgs {
  const uint16_t* A;  // [M, K]
  const uint16_t* W;  // weight rows, [*, K]
  int M, K, num_n;
  int D, F;           // width, mlp hidden
  // input projection outputs
  uint16_t* q;
  uint16_t* k;
  uint16_t* v;
  uint16_t* cat;      // [M, D + F]; m goes to columns [D, D + F)
  // per-head QK RMSNorm + 4-axis RoPE applied to q and k in the epilogue
  const int32_t* pos;      // [M, 4] (t, h, w, l)
  const uint16_t* q_scale;  // [128] bf16
  const uint16_t* k_scale;  // [128] bf16
  float qk_eps;
  float theta;
  float q_mul;             // multiplies the normalized, rotated q before it is stored
  // theta^(-2j / 32) / (2 pi), the turns per position step of pair j, as
  // hi + lo: hi keeps 8 significant bits, so pos * hi is exact in fp32 for
  // |pos| < 2^16 and the turn count's fraction costs no fp64 work
  float rope_hi[16], rope_lo[16];
  // output projection
  const uint16_t* x;  // residual [M, D]
  const uint16_t* mod;  // [S, 3, D]
  uint16_t* y;        // [M, D]
  int e0, e1;         // stream boundaries
  uint32_t flags;
  // Split of the last, partial round of tiles (see launch()): tiles
  // [0, n_dp) run whole, one per workgroup; the n_tail tiles after them are
  // cut along K into n_pieces equal runs of whole units, one per
  // workgroup, whose fp32 partial tiles go to `partial` and are summed by the
  // fix-up kernel.
  int n_dp, n_tail, n_pieces;
  int unit;           // k tiles per split unit (the K loop's unroll period)
  float* partial;     // 2 * n_pieces slots of BM * BN floats
  int KT;             // k tiles of 128 bytes per row
  // FP8 mode: A = q_a diag(s_a)^-1 row scales [M], W row scales [W rows]
  const float* sa;
  const float* sw;
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Tile geometry: BM rows, WM x WN waves, MB x NB blocks of 32 x 32 per wave.
template <int BM_>
struct Tile {
  static constexpr int BM = BM_;
  static constexpr int WM = BM_ == 256 ? 2 : 1;
  static constexpr int WN = 4 / WM;
  static constexpr int MB = BM_ / (32 * WM);
  static constexpr int NB = BN / (32 * WN);
  static constexpr int A_SLABS = BM_ / RPI;  // 1 KB loads that fill the A tile
  static constexpr int NLD_A = A_SLABS / 4;  // per wave per k tile
  static constexpr int NLD_B = BN / RPI / 4;
  static_assert(MB * 32 * WM == BM_ && NB * 32 * WN == BN, "tile geometry");
  static_assert(NB % 2 == 0, "gate and up blocks pair up inside a wave");
  static_assert(NLD_A * 4 == A_SLABS, "A tile loads");
};

// Weight row feeding row r (0..255) of N-tile tn.
template <int EPI, int NB>
__device__ __forceinline__ int weight_row(const GemmArgs& g, int tn, int r) {
  if (EPI == EPI_IN) {
    const int n_qkv = 3 * g.D / BN;
    if (tn < n_qkv) return tn * BN + r;
    // MLP tile: 128 hidden units.  Wave wn owns rows [32 NB wn, 32 NB (wn + 1));
    // its 32-row blocks alternate gate, up, gate, up over the wave's NB / 2
    // groups of 32 hidden units.
    const int wn = r / (32 * NB), blk = (r >> 5) % NB, i = r & 31;
    const int hidden = (tn - n_qkv) * 128 + wn * (NB / 2) * 32 + (blk >> 1) * 32 + i;
    return 3 * g.D + (blk & 1) * g.F + hidden;
  }
  return tn * BN + r;
}

// LDS tiles are rows of 64 bf16 (128 B = 8 chunks of 16 B).  gfx950's LDS
// has 64 banks of 4 B, so 16 lanes of a 16-byte read are served per cycle:
// the 16 consecutive rows one MFMA fragment read touches must land on 16
// distinct 16-byte bank slots.  Row r covers slots 8 (r % 2) .. + 7, so the
// chunk is xor-ed with (r >> 1) & 7, a bijection on the 8 rows of each parity.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// s_waitcnt immediate: vmcnt(n), expcnt and lgkmcnt left alone
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int LGKMCNT0 = 0xC07F;

// Workgroup barrier for the K loop.  __syncthreads() would also wait for every
// outstanding vector-memory operation (the whole prefetch ring); here the
// caller waits only for the tile about to be read, plus its own LDS reads.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// silu(a) = a / (1 + e^-a) with the hardware reciprocal (about 1 ulp; the
// result is rounded to bf16), not the IEEE division sequence
__device__ __forceinline__ float silu(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  return make_uint2(pack2(a, b), pack2(c, d));
}

// Logical tile id -> (tm, tn): groups of GROUP_N N-tiles, M fastest inside
// a group, so the tiles one XCD runs together share few A and W panels.
template <int BM>
__device__ __forceinline__ void tile_coords(const GemmArgs& g, int id, int& tm, int& tn) {
  const int num_m = (g.M + BM - 1) / BM;
  const int grp = id / (GROUP_N * num_m);
  const int rem = id - grp * GROUP_N * num_m;
  const int gw = min(GROUP_N, g.num_n - grp * GROUP_N);
  tm = rem / gw;
  tn = grp * GROUP_N + rem % gw;
}

// Epilogue of one accumulator pair.  The MFMAs compute C^T, so in block
// (i, j) of wave (wm, wn), lane (ln, hl) holds output row (wm MB + i) 32 + ln
// and the 4 consecutive columns (wn NB + j) 32 + 8 rr + 4 hl .. + 3 in
// registers 4 rr .. 4 rr + 3: every store, residual load and gate load is 8
// contiguous bytes.  Blocks are taken in pairs j = 2 jp, 2 jp + 1 because the
// SwiGLU tiles interleave them as (gate, up) of the same hidden units; `a` and
// `b` are the two blocks' 4 values for one rr.
template <int EPI, int BM>
__device__ __forceinline__ void epilogue_pair(const GemmArgs& g, int tm, int tn, int wm, int wn,
                                              int lane, int i, int jp, int rr, const float (&a)[4],
                                              const float (&b)[4]) {
  constexpr int MB = Tile<BM>::MB, NB = Tile<BM>::NB;
  const int ln = lane & 31, hl = lane >> 5;
  const int row = tm * BM + (wm * MB + i) * 32 + ln;
  if (row >= g.M) return;
  const int col = tn * BN + wn * NB * 32 + 4 * hl + 2 * jp * 32 + 8 * rr;  // block 2 jp
  if (EPI == EPI_IN) {
    const int n_qkv = 3 * g.D / BN;
    if (tn < n_qkv) {
      // q | k | v: D is a multiple of the 256-wide N tile, so the whole tile
      // falls in one of the three
      const int which = tn * BN / g.D;
      uint16_t* const dr = (which == 0 ? g.q : which == 1 ? g.k : g.v) + (size_t)row * g.D +
                           (col - which * g.D);
      *reinterpret_cast<uint2*>(dr) = pack4(a[0], a[1], a[2], a[3]);
      *reinterpret_cast<uint2*>(dr + 32) = pack4(b[0], b[1], b[2], b[3]);
    } else {
      const int hid = (tn - n_qkv) * 128 + wn * (NB / 2) * 32 + 4 * hl + jp * 32 + 8 * rr;
      uint16_t* const dr = g.cat + (size_t)row * (g.D + g.F) + g.D + hid;
      *reinterpret_cast<uint2*>(dr) = pack4(silu(a[0]) * b[0], silu(a[1]) * b[1],
                                            silu(a[2]) * b[2], silu(a[3]) * b[3]);
    }
  } else {
    const bool use_gate = !(g.flags & 2u), use_res = !(g.flags & 1u);
    const uint16_t* gate = g.mod + (size_t)stream_of(row, g.e0, g.e1) * 3 * g.D + 2 * g.D + col;
    const uint16_t* xr = g.x + (size_t)row * g.D + col;
    uint16_t* yr = g.y + (size_t)row * g.D + col;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float(&v)[4] = h ? b : a;
      const uint2 gv = use_gate ? *reinterpret_cast<const uint2*>(gate + 32 * h)
                                : make_uint2(0x3f803f80u, 0x3f803f80u);
      const uint2 xv = use_res ? *reinterpret_cast<const uint2*>(xr + 32 * h) : make_uint2(0u, 0u);
      *reinterpret_cast<uint2*>(yr + 32 * h) =
          pack4(fmaf(lo2f(gv.x), v[0], lo2f(xv.x)), fmaf(hi2f(gv.x), v[1], hi2f(xv.x)),
                fmaf(lo2f(gv.y), v[2], lo2f(xv.y)), fmaf(hi2f(gv.y), v[3], hi2f(xv.y)));
    }
  }
}

// Whole-tile epilogues stage each wave's outputs in LDS (the ring is free
// once the K loop is done) and then store rows: 16 contiguous bytes per lane,
// whole cache lines per 8 or 16 lanes, where the accumulator layout (one row
// per lane) would touch 32 rows per store instruction.  Each wave stages its
// own sub-tile in its own ring array, so after one workgroup barrier the
// waves proceed independently.  A staged row is ROW_CHUNKS 16-byte chunks;
// chunk c of row r sits at chunk c ^ (r & mask) so the 32 rows one
// accumulator write touches spread over the LDS banks, while a row read back
// stays whole.
template <int ROW_CHUNKS>
__device__ __forceinline__ int st_off(int r, int c) {
  constexpr int MASK = ROW_CHUNKS < 16 ? ROW_CHUNKS - 1 : 15;
  return (r * ROW_CHUNKS + (c ^ (r & MASK))) * 16;
}

// LDS writes of this wave are complete and visible to its own later reads;
// the compiler keeps LDS accesses on either side of it in order
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(LGKMCNT0);
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// Stores n_rows staged bf16 rows of ROW_CHUNKS * 8 elements to dst (row r at
// dst + (row0 + r) * ld), rows at or past M skipped.
template <int ROW_CHUNKS>
__device__ __forceinline__ void store_staged(const char* st, int n_rows, uint16_t* dst,
                                             size_t ld, int row0, int M, int lane) {
  constexpr int RPI = 64 / ROW_CHUNKS;  // rows per store instruction
  const int c = lane % ROW_CHUNKS;
  for (int r = lane / ROW_CHUNKS; r < n_rows; r += RPI) {
    if (row0 + r >= M) break;
    *reinterpret_cast<uint4*>(dst + (size_t)(row0 + r) * ld + c * 8) =
        *reinterpret_cast<const uint4*>(st + st_off<ROW_CHUNKS>(r, c));
  }
}

// Fraction of pos * (hi + lo) turns: pos * hi is exact (hi has 8
// significant bits, |pos| < 2^16), so its fraction is exact too, and one fma
// adds pos * lo before the second reduction; the result is within about 2^-24
// (|pos lo| + 1) of the exact fraction.
__device__ __forceinline__ float turn_fraction(float pos, float hi, float lo) {
  const float a = __builtin_amdgcn_fractf(pos * hi);
  return __builtin_amdgcn_fractf(fmaf(pos, lo, a));
}

// q / k tile epilogue of the 256-row layout: per-head RMSNorm with the
// learnable scale, then 4-axis RoPE, straight from the fp32 accumulators
// (the same operations the standalone rope4 kernel applies to stored q, k).
// Wave (wm, wn) holds columns [128 wn, 128 wn + 128) of the tile, i.e. one
// whole head, and in block j = 0..3 the 32 dims of axis j; lane (ln, hl)
// holds, for each row, dims 8 rr + 4 hl + e of every axis, the other half
// sits in lane ln ^ 32.  Pair p of an axis is dims (2 p, 2 p + 1), turned by
// pos_axis * theta^(-2 p / 32) radians.
__device__ __forceinline__ void epilogue_qk(const GemmArgs& g, const f32x16 (&acc)[4][4], int tm,
                                            int tn, int wm, int wn, int lane, char* st) {
  constexpr int BM = 256, MB = 4, NB = 4;
  const int ln = lane & 31, hl = lane >> 5;
  const int which = tn * BN / g.D;  // 0: q, 1: k
  uint16_t* const dst = which ? g.k : g.q;
  const uint16_t* const scale = which ? g.k_scale : g.q_scale;
  const int c0 = tn * BN - which * g.D + wn * NB * 32;  // first dim of the head
  const float qmul = which ? 1.0f : g.q_mul;
  // Per-lane inputs, all loads issued before the first use: the scale of
  // this lane's 64 dims, the turn rate of its 8 pairs per axis, and the
  // positions of its 4 rows.
  uint2 gsc[NB][4];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      gsc[j][rr] = *reinterpret_cast<const uint2*>(scale + j * 32 + 8 * rr + 4 * hl);
  float fh[4][2], fl[4][2];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      fh[rr][pr] = hl ? g.rope_hi[4 * rr + 2 + pr] : g.rope_hi[4 * rr + pr];
      fl[rr][pr] = hl ? g.rope_lo[4 * rr + 2 + pr] : g.rope_lo[4 * rr + pr];
    }
  int4 p4[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int row = tm * BM + (wm * MB + i) * 32 + ln;
    p4[i] = reinterpret_cast<const int4*>(g.pos)[min(row, g.M - 1)];
  }
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int row = tm * BM + (wm * MB + i) * 32 + ln;
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) ss = fmaf(acc[i][j][r], acc[i][j][r], ss);
    ss += __shfl_xor(ss, 32, 64);
    const float rstd = rsqrtf(ss * (1.0f / 128.0f) + g.qk_eps) * qmul;
    if (row >= g.M) continue;
    const int pa[4] = {p4[i].x, p4[i].y, p4[i].z, p4[i].w};
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float pj = (float)pa[j];
      // position 0 on this axis in every lane of the wave (t and l of image
      // tokens, h, w and l of text tokens): nothing turns, no angles needed
      const bool turn = __ballot(pa[j] != 0) != 0;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const uint2 gs = gsc[j][rr];
        const float x[4] = {acc[i][j][4 * rr] * rstd * lo2f(gs.x),
                            acc[i][j][4 * rr + 1] * rstd * hi2f(gs.x),
                            acc[i][j][4 * rr + 2] * rstd * lo2f(gs.y),
                            acc[i][j][4 * rr + 3] * rstd * hi2f(gs.y)};
        float y[4] = {x[0], x[1], x[2], x[3]};
        if (turn) {
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            // pair 4 rr + 2 hl + pr of axis j: the turn count reduced to
            // [0, 1), then sin / cos of 2 pi r in hardware
            const float r = turn_fraction(pj, fh[rr][pr], fl[rr][pr]);
            const float sn = __builtin_amdgcn_sinf(r), cs = __builtin_amdgcn_cosf(r);
            y[2 * pr] = x[2 * pr] * cs - x[2 * pr + 1] * sn;
            y[2 * pr + 1] = x[2 * pr] * sn + x[2 * pr + 1] * cs;
          }
        }
        // staged at row i 32 + ln, columns j 32 + 8 rr + 4 hl .. + 3
        *reinterpret_cast<uint2*>(st + st_off<16>(i * 32 + ln, 4 * j + rr) + 8 * hl) =
            pack4(y[0], y[1], y[2], y[3]);
      }
    }
  }
  wave_lds_sync();
  store_staged<16>(st, MB * 32, dst + c0, g.D, tm * BM + wm * MB * 32, g.M, lane);
}

// q / k tile epilogue of the 1 x 4 layouts (224 or 128 rows; waves of
// BM x 64): a head's 128 dims are split over waves wn and wn ^ 1, 64 each, so
// the two halves of each row's sum of squares meet in LDS (s_rs, BM floats per
// wave).  Wave wn holds axes 2 (wn & 1) and 2 (wn & 1) + 1 in its blocks 0
// and 1; the rest is the 256-row epilogue's norm and rotation.
template <int BM>
__device__ __forceinline__ void epilogue_qk224(const GemmArgs& g,
                                               const f32x16 (&acc)[BM / 32][2], int tm, int tn,
                                               int wn, int lane, char* st, float* s_rs) {
  constexpr int MB = BM / 32, NB = 2;
  const int ln = lane & 31, hl = lane >> 5;
  const int which = tn * BN / g.D;  // 0: q, 1: k
  uint16_t* const dst = which ? g.k : g.q;
  const uint16_t* const scale = which ? g.k_scale : g.q_scale;
  const int hh = wn & 1;                                  // half of the head
  const int c0 = tn * BN - which * g.D + wn * NB * 32;    // first dim of this wave
  const float qmul = which ? 1.0f : g.q_mul;
  uint2 gsc[NB][4];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      gsc[j][rr] = *reinterpret_cast<const uint2*>(scale + (2 * hh + j) * 32 + 8 * rr + 4 * hl);
  float fh[4][2], fl[4][2];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      fh[rr][pr] = hl ? g.rope_hi[4 * rr + 2 + pr] : g.rope_hi[4 * rr + pr];
      fl[rr][pr] = hl ? g.rope_lo[4 * rr + 2 + pr] : g.rope_lo[4 * rr + pr];
    }
  int4 p4[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int row = tm * BM + i * 32 + ln;
    p4[i] = reinterpret_cast<const int4*>(g.pos)[min(row, g.M - 1)];
  }
  float ss[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) a = fmaf(acc[i][j][r], acc[i][j][r], a);
    ss[i] = a + __shfl_xor(a, 32, 64);
    // both half-waves hold the same sum and store it to the same address: a
    // store predicated on one half-wave let the compiler place a register
    // copy inside its exec mask, which the other half then read stale
    s_rs[wn * BM + i * 32 + ln] = ss[i];
  }
  __syncthreads();  // every wave of the tile is a q or k wave
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int row = tm * BM + i * 32 + ln;
    const float tot = ss[i] + s_rs[(wn ^ 1) * BM + i * 32 + ln];
    const float rstd = rsqrtf(tot * (1.0f / 128.0f) + g.qk_eps) * qmul;
    if (row >= g.M) continue;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int pax = hh ? (j ? p4[i].w : p4[i].z) : (j ? p4[i].y : p4[i].x);
      const float pj = (float)pax;
      const bool turn = __ballot(pax != 0) != 0;  // as in epilogue_qk
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const uint2 gs = gsc[j][rr];
        const float x[4] = {acc[i][j][4 * rr] * rstd * lo2f(gs.x),
                            acc[i][j][4 * rr + 1] * rstd * hi2f(gs.x),
                            acc[i][j][4 * rr + 2] * rstd * lo2f(gs.y),
                            acc[i][j][4 * rr + 3] * rstd * hi2f(gs.y)};
        float y[4] = {x[0], x[1], x[2], x[3]};
        if (turn) {
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const float r = turn_fraction(pj, fh[rr][pr], fl[rr][pr]);
            const float sn = __builtin_amdgcn_sinf(r), cs = __builtin_amdgcn_cosf(r);
            y[2 * pr] = x[2 * pr] * cs - x[2 * pr + 1] * sn;
            y[2 * pr + 1] = x[2 * pr] * sn + x[2 * pr + 1] * cs;
          }
        }
        // staged at row i 32 + ln, columns j 32 + 8 rr + 4 hl .. + 3
        *reinterpret_cast<uint2*>(st + st_off<8>(i * 32 + ln, 4 * j + rr) + 8 * hl) =
            pack4(y[0], y[1], y[2], y[3]);
      }
    }
  }
  wave_lds_sync();
  store_staged<8>(st, MB * 32, dst + c0, g.D, tm * BM, g.M, lane);
}

// Output projection of a whole tile: y = x + gate * r, staged in passes of
// PASS_RB 32-row blocks of the wave's fp32 r (24 KB for the 224-row layout's
// 64 columns, 32 KB for the 256-row layout's 128), with every residual and
// gate load of a pass issued before its staging writes.  x may be y (in
// place): each element is read before it is written, by the same lane.
template <int BM>
__device__ __forceinline__ void epilogue_out(const GemmArgs& g,
                                             const f32x16 (&acc)[Tile<BM>::MB][Tile<BM>::NB],
                                             int tm, int tn, int wm, int wn, int lane, char* st) {
  constexpr int MB = Tile<BM>::MB, NB = Tile<BM>::NB;
  constexpr int RC = NB * 32 / 4;         // fp32 16-byte chunks per staged row (16 or 32)
  constexpr int OC = NB * 32 / 8;         // bf16 16-byte chunks per output row (8 or 16)
  constexpr int RPI = 64 / OC;            // output rows per wave instruction
  constexpr int PASS_RB = BM == 224 ? 3 : 2;
  constexpr int ITERS = PASS_RB * 32 / RPI;
  const int ln = lane & 31, hl = lane >> 5;
  const bool use_gate = !(g.flags & 2u), use_res = !(g.flags & 1u);
  const int c = lane % OC;
  const int col = tn * BN + wn * NB * 32 + c * 8;  // this lane's 8 output columns
#pragma unroll
  for (int p = 0; p * PASS_RB < MB; ++p) {
    const int rb0 = p * PASS_RB;
    const int row0 = tm * BM + (wm * MB + rb0) * 32;
    uint4 xv[ITERS], gv[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int row = min(row0 + it * RPI + lane / OC, g.M - 1);
      xv[it] = use_res ? *reinterpret_cast<const uint4*>(g.x + (size_t)row * g.D + col)
                       : make_uint4(0u, 0u, 0u, 0u);
      gv[it] = use_gate ? *reinterpret_cast<const uint4*>(
                              g.mod + (size_t)stream_of(row, g.e0, g.e1) * 3 * g.D + 2 * g.D + col)
                        : make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
    }
#pragma unroll
    for (int i = rb0; i < rb0 + PASS_RB && i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const f32x16& a = acc[i][j];
          // row (i - rb0) 32 + ln, columns j 32 + 8 rr + 4 hl .. + 3
          *reinterpret_cast<float4*>(st + st_off<RC>((i - rb0) * 32 + ln, 8 * j + 2 * rr + hl)) =
              make_float4(a[4 * rr], a[4 * rr + 1], a[4 * rr + 2], a[4 * rr + 3]);
        }
    wave_lds_sync();
    const int n_rows = (min(MB, rb0 + PASS_RB) - rb0) * 32;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int r = it * RPI + lane / OC;
      if (r >= n_rows || row0 + r >= g.M) continue;
      const float4 r0 = *reinterpret_cast<const float4*>(st + st_off<RC>(r, 2 * c));
      const float4 r1 = *reinterpret_cast<const float4*>(st + st_off<RC>(r, 2 * c + 1));
      const float rv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
      const uint32_t xw[4] = {xv[it].x, xv[it].y, xv[it].z, xv[it].w};
      const uint32_t gw[4] = {gv[it].x, gv[it].y, gv[it].z, gv[it].w};
      uint32_t o[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        o[t] = pack2(fmaf(lo2f(gw[t]), rv[2 * t], lo2f(xw[t])),
                     fmaf(hi2f(gw[t]), rv[2 * t + 1], hi2f(xw[t])));
      *reinterpret_cast<uint4*>(g.y + (size_t)(row0 + r) * g.D + col) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
    wave_lds_sync();  // the next pass rewrites the staging rows
  }
  (void)ln;
  (void)hl;
}

// Input projection of a whole tile: q / k heads through the norm + RoPE
// epilogue, v heads and the SwiGLU product m, each staged and stored by rows.
// A wave holds NB * 32 columns: 128 (256-row layout) or 64 (224-row layout).
template <int BM>
__device__ __forceinline__ void epilogue_in(const GemmArgs& g,
                                            const f32x16 (&acc)[Tile<BM>::MB][Tile<BM>::NB],
                                            int tm, int tn, int wm, int wn, int lane, char* st,
                                            float* s_rs) {
  constexpr int MB = Tile<BM>::MB, NB = Tile<BM>::NB;
  const int ln = lane & 31, hl = lane >> 5;
  const int n_qkv = 3 * g.D / BN;
  if (tn < 2 * g.D / BN) {  // q or k
    if constexpr (BM == 256)
      epilogue_qk(g, acc, tm, tn, wm, wn, lane, st);
    else
      epilogue_qk224<BM>(g, acc, tm, tn, wn, lane, st, s_rs);
    return;
  }
  const int row0 = tm * BM + wm * MB * 32;
  if (tn < n_qkv) {  // v
    constexpr int RC = NB * 4;  // 16-byte chunks per staged row
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const f32x16& a = acc[i][j];
          *reinterpret_cast<uint2*>(st + st_off<RC>(i * 32 + ln, 4 * j + rr) + 8 * hl) =
              pack4(a[4 * rr], a[4 * rr + 1], a[4 * rr + 2], a[4 * rr + 3]);
        }
    wave_lds_sync();
    store_staged<RC>(st, MB * 32, g.v + (tn * BN - 2 * g.D + wn * NB * 32), g.D, row0, g.M,
                     lane);
    return;
  }
  // MLP tile: blocks 2 jp (gate) and 2 jp + 1 (up) of the same 32 hidden
  // units; the wave's NB / 2 groups of 32 units are staged as 2 NB chunks
  // per row
  constexpr int MC = NB * 2;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int jp = 0; jp < NB / 2; ++jp)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const f32x16& a = acc[i][2 * jp];
        const f32x16& b = acc[i][2 * jp + 1];
        *reinterpret_cast<uint2*>(st + st_off<MC>(i * 32 + ln, 4 * jp + rr) + 8 * hl) =
            pack4(silu(a[4 * rr]) * b[4 * rr], silu(a[4 * rr + 1]) * b[4 * rr + 1],
                  silu(a[4 * rr + 2]) * b[4 * rr + 2], silu(a[4 * rr + 3]) * b[4 * rr + 3]);
      }
  wave_lds_sync();
  const int hid0 = (tn - n_qkv) * 128 + wn * (NB / 2) * 32;
  store_staged<MC>(st, MB * 32, g.cat + g.D + hid0, (size_t)(g.D + g.F), row0, g.M, lane);
}

template <int EPI, int BM>
__device__ __forceinline__ void epilogue(const GemmArgs& g,
                                         const f32x16 (&acc)[Tile<BM>::MB][Tile<BM>::NB], int tm,
                                         int tn, int wm, int wn, int lane, char* st, float* s_rs) {
  if constexpr (EPI == EPI_IN) {
    epilogue_in<BM>(g, acc, tm, tn, wm, wn, lane, st, s_rs);
  } else {
    (void)s_rs;
    epilogue_out<BM>(g, acc, tm, tn, wm, wn, lane, st);
  }
}

// FP8 mode: multiplies a whole tile's accumulators by the rowwise scales,
// s_a of the output row times s_w of the weight row of each column.
template <int EPI, int BM>
__device__ __forceinline__ void scale_acc(const GemmArgs& g,
                                          f32x16 (&acc)[Tile<BM>::MB][Tile<BM>::NB], int tm,
                                          int tn, int wm, int wn, int lane) {
  constexpr int MB = Tile<BM>::MB, NB = Tile<BM>::NB;
  const int ln = lane & 31, hl = lane >> 5;
  float4 ws[NB][4];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      ws[j][rr] = *reinterpret_cast<const float4*>(
          g.sw + weight_row<EPI, NB>(g, tn, (wn * NB + j) * 32 + 8 * rr + 4 * hl));
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const float sr = g.sa[min(tm * BM + (wm * MB + i) * 32 + ln, g.M - 1)];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        acc[i][j][4 * rr] *= sr * ws[j][rr].x;
        acc[i][j][4 * rr + 1] *= sr * ws[j][rr].y;
        acc[i][j][4 * rr + 2] *= sr * ws[j][rr].z;
        acc[i][j][4 * rr + 3] *= sr * ws[j][rr].w;
      }
  }
}

// A partial tile in fp32: wave w's accumulators as consecutive 16-byte
// groups, group-major, so each wave store / load moves 1 KB contiguously.
template <int BM>
__device__ __forceinline__ float4* partial_slot(const GemmArgs& g, int slot, int wave, int lane) {
  constexpr int G4 = Tile<BM>::MB * Tile<BM>::NB * 4;  // 16-byte groups per lane
  return reinterpret_cast<float4*>(g.partial + (size_t)slot * BM * BN) + (size_t)wave * G4 * 64 + lane;
}

// First unit of piece p when `units` 4-k-tile units are cut into `pieces` runs.
__device__ __forceinline__ int piece_start(int p, int units, int pieces) {
  return (int)(((long long)p * units) / pieces);
}

// NA: LDS slots for A k tiles.  NA = 3 lets the A loads of tile kt + 2 start
// during the first k steps of tile kt (A is the operand that misses L2 more:
// each A panel is shared by fewer concurrent tiles than a W panel), spread
// over them instead of bursting after the barrier; the K loop's unroll period
// is then lcm(3, 2) = 6 k tiles.  NA = 2 serves K that is not a multiple of
// 6 k tiles; then both operands load right after the barrier.
template <int EPI, int BM, int NA, bool F8>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs g) {
  using T = Tile<BM>;
  constexpr int MB = T::MB, NB = T::NB;
  constexpr int PERIOD = NA == 3 ? 6 : 2;
  constexpr int ES = F8 ? 1 : 2;    // bytes per element
  constexpr int KSTEPS = F8 ? 2 : 4;  // MFMA k steps per k tile
  using Frag = std::conditional_t<F8, i32x8, bf16x8>;
  // One LDS array per slot, not one indexed array: the compiler tracks
  // direct-to-LDS stores per LDS variable, so it can see that fragment reads
  // of one slot never alias the loads in flight into the others and does not
  // wait on them.  NA = 3 and BM = 256 use all 160 KB.
  __shared__ __attribute__((aligned(16))) uint16_t s_a0[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t s_a1[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t s_a2[NA == 3 ? BM * BK : 8];
  __shared__ __attribute__((aligned(16))) uint16_t s_w0[BN * BK];
  __shared__ __attribute__((aligned(16))) uint16_t s_w1[BN * BK];
  // row sums of squares exchanged by the q / k epilogue of the 1 x 4 layout
  __shared__ float s_rs[EPI == EPI_IN && BM != 256 ? 4 * BM : 1];
  uint16_t* const ring_a[3] = {s_a0, s_a1, s_a2};
  uint16_t* const ring_w[NW] = {s_w0, s_w1};

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar: LDS addresses of the direct loads (M0) then come
  // from scalar arithmetic instead of a v_readfirstlane per load
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WN, wn = wave % T::WN;
  const int ln = lane & 31, hl = lane >> 5;

  const int KT = g.KT;          // a multiple of PERIOD (the host picks NA so)
  const int upt = KT / PERIOD;  // split units per tile

  // Work items: one whole tile, or the one or two tail tiles a split piece
  // covers (pieces are shorter than a tile).  Split piece p covers units [u0, u1) of the tail tiles, laid end to end.
  const bool dp = (int)blockIdx.x < g.n_dp;
  const int p = blockIdx.x - g.n_dp;
  const int units = g.n_tail * upt;
  const int u0 = dp ? 0 : piece_start(p, units, g.n_pieces);
  const int u1 = dp ? 0 : piece_start(p + 1, units, g.n_pieces);
  const int t0 = u0 / upt;
  const int end0 = min(u1, (t0 + 1) * upt);

  const char* abase = reinterpret_cast<const char*>(g.A);
  const char* bbase = reinterpret_cast<const char*>(g.W);
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const int lrow = lane / CH;

  // One work item: tile `id` over k tiles [k0, k1).  A whole tile (SPLIT
  // false) ends in the epilogue, a split piece stores its fp32 partial tile in
  // `slot`.  The two kinds are separate instances so neither carries the
  // other's registers.
  auto item = [&](auto split, int id, int k0, int k1, int slot) __attribute__((always_inline)) {
    constexpr bool SPLIT = decltype(split)::value;
    constexpr int NLD_A = T::NLD_A, NLD_B = T::NLD_B;
    // fixed bounds (not NLD_A): an array of template-dependent type would make
    // the direct-load builtins below dependent, and the host pass, which
    // cannot check them, would then drop the kernel's host stub
    uint32_t aoff[8], boff[8];
    static_assert(NLD_A <= 8 && NLD_B <= 8, "load offsets");
    f32x16 acc[MB][NB];
    Frag fa[2][MB], fb[2][NB];
    int tm, tn;
    tile_coords<BM>(g, id, tm, tn);

    // Global -> LDS with gfx950's 16-byte direct loads (no staging registers).
    // One wave instruction fills 1 KB of LDS = 8 tile rows of 128 B (a slab),
    // so it reads 8 whole cache lines: the vector L1 delivers twice the bytes
    // per cycle that it does for half lines.  Lane i lands in row 8 s + i / 8
    // at physical chunk i % 8, which holds logical chunk (i % 8) ^ swz(row), so
    // that is the chunk the lane fetches.  Wave w loads A slabs
    // NLD_A w .. NLD_A (w + 1) - 1 and W slabs likewise.  Byte offsets are
    // 32-bit: the loads use the scalar-base + vector-offset form.
#pragma unroll
    for (int j = 0; j < NLD_A; ++j) {
      const int ra = (wave * NLD_A + j) * RPI + lrow;
      const int arow = min(tm * BM + ra, g.M - 1);
      aoff[j] = (uint32_t)arow * (uint32_t)(g.K * ES) + (((lane % CH) ^ swz(ra)) * 16u);
    }
#pragma unroll
    for (int j = 0; j < NLD_B; ++j) {
      const int rb = (wave * NLD_B + j) * RPI + lrow;
      boff[j] = (uint32_t)weight_row<EPI, NB>(g, tn, rb) * (uint32_t)(g.K * ES) +
                (((lane % CH) ^ swz(rb)) * 16u);
    }
    // Past k1 the last tile is reloaded into an idle slot (never read), so
    // the loop needs no branches.  gload_a issues A loads j0 .. j1 - 1 of k
    // tile kt, so they can be spread over several k steps.
    auto gload_a = [&](int kt, uint16_t* st, int j0, int j1) __attribute__((always_inline)) {
      const uint32_t ko = (uint32_t)min(kt, k1 - 1) * (BK * 2);
#pragma unroll
      for (int j = j0; j < j1; ++j)
        __builtin_amdgcn_global_load_lds(abase + (aoff[j] + ko),
                                         (lds_ptr)(st + (wave * NLD_A + j) * RPI * BK), 16, 0, 0);
    };
    auto gload_w = [&](int kt, uint16_t* st) __attribute__((always_inline)) {
      const uint32_t ko = (uint32_t)min(kt, k1 - 1) * (BK * 2);
#pragma unroll
      for (int j = 0; j < NLD_B; ++j)
        __builtin_amdgcn_global_load_lds(bbase + (boff[j] + ko),
                                         (lds_ptr)(st + (wave * NLD_B + j) * RPI * BK), 16, 0, 0);
    };

#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // MFMA fragments, double-buffered in registers: while the MFMAs of one
    // k step run, the next step's fragment reads are in flight.  A bf16
    // fragment is the 16-byte chunk 2 ks + hl of the lane's row (8 k); an FP8
    // fragment is chunks 4 ks + 2 hl and 4 ks + 2 hl + 1 (32 k): both operands
    // use the same chunks, so the k order inside the MFMA does not matter.
    auto lds16 = [&](const uint16_t* base, int r, int c) __attribute__((always_inline)) {
      return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + r * 128 +
                                             ((c ^ swz(r)) << 4));
    };
    auto read_frags = [&](const uint16_t* sa, const uint16_t* sw, int ks, int slot)
                          __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int r = (wm * MB + i) * 32 + ln;
        if constexpr (F8) {
          const uint4 x = lds16(sa, r, 4 * ks + 2 * hl), y = lds16(sa, r, 4 * ks + 2 * hl + 1);
          fa[slot][i] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                              (int)y.x, (int)y.y, (int)y.z, (int)y.w};
        } else {
          fa[slot][i] = __builtin_bit_cast(bf16x8, lds16(sa, r, 2 * ks + hl));
        }
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int r = (wn * NB + j) * 32 + ln;
        if constexpr (F8) {
          const uint4 x = lds16(sw, r, 4 * ks + 2 * hl), y = lds16(sw, r, 4 * ks + 2 * hl + 1);
          fb[slot][j] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w,
                              (int)y.x, (int)y.y, (int)y.z, (int)y.w};
        } else {
          fb[slot][j] = __builtin_bit_cast(bf16x8, lds16(sw, r, 2 * ks + hl));
        }
      }
    };
    // C^T = W A^T: the weights are the A operand, so each lane ends up owning
    // an output row (see the epilogue)
    auto mfmas = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if constexpr (F8)
            // formats 0 / 0: e4m3 for both operands; scale exponents 127: 2^0
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fb[slot][j], fa[slot][i], acc[i][j], 0, 0, 0, 127, 0, 127);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[slot][j], fa[slot][i],
                                                                acc[i][j], 0, 0, 0);
        }
    };
    // One k tile (KSTEPS k steps) from A slot i % NA and W slot i % 2, while
    // tile kt + 1 lands in the other slots.  The instruction order is pinned
    // (the compiler would otherwise sink the loads next to the waits and pair
    // each fragment read with its first use).  Each k step's MFMAs run while
    // the next step's fragment reads are in flight.  With NA = 3 the A loads
    // of tile kt + 2 go to the slot tile kt - 1 used, free since the previous
    // barrier, and are spread over k steps 0..2.  The barrier comes before the
    // last k step, whose fragments are already in registers: every read of
    // this tile's slots is then complete (lgkmcnt(0)), so right after the
    // barrier the W slot (and with NA = 2 the A slot) is refilled with tile
    // kt + 2 and the first fragments of tile kt + 1 are read, all overlapping
    // the last k step's MFMAs.
    auto ktile = [&](int kt, int i) __attribute__((always_inline)) {
      uint16_t* const sa = ring_a[i % NA];
      uint16_t* const sw = ring_w[i % NW];
      constexpr int KS1 = KSTEPS - 1;  // k steps before the barrier
      // one A load of tile kt + 2 after every GL_EVERY MFMAs: NLD_A of them
      // fit in KS1 k steps of MB x NB MFMAs
      constexpr int GL_EVERY = F8 ? 2 : 4;
#pragma unroll
      for (int ks = 0; ks < KS1; ++ks) {
        if constexpr (NA == 3) {
          // A loads of tile kt + 2: NLD_A split as evenly as possible
          gload_a(kt + 2, ring_a[(i + 2) % 3], ks * NLD_A / KS1, (ks + 1) * NLD_A / KS1);
        }
        read_frags(sa, sw, ks + 1, (ks + 1) & 1);
        mfmas(ks & 1);
#pragma unroll
        for (int q = 0; q < MB * NB; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
          if (NA == 3 && q % GL_EVERY == 1)
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
          __builtin_amdgcn_sched_group_barrier(0x100, F8 ? 2 : 1, 0);  // LDS reads
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // tile kt + 1 has landed; with NA = 3 the A loads of tile kt + 2 (the
      // youngest NLD_A) may still fly
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(NA == 3 ? NLD_A : 0));
      __builtin_amdgcn_s_waitcnt(LGKMCNT0);
      ring_barrier();
      if constexpr (NA == 2) gload_a(kt + 2, sa, 0, NLD_A);
      gload_w(kt + 2, sw);
      read_frags(ring_a[(i + 1) % NA], ring_w[(i + 1) % NW], 0, 0);
      mfmas(KS1 & 1);
#pragma unroll
      for (int q = 0; q < MB * NB; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 global load
        __builtin_amdgcn_sched_group_barrier(0x100, F8 ? 2 : 1, 0);  // LDS reads
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: tiles k0 and k0 + 1 in flight, wait for k0
    gload_a(k0, ring_a[0], 0, NLD_A);
    gload_w(k0, ring_w[0]);
    gload_a(k0 + 1, ring_a[1], 0, NLD_A);
    gload_w(k0 + 1, ring_w[1]);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(NLD_A + NLD_B));
    ring_barrier();
    read_frags(ring_a[0], ring_w[0], 0, 0);
    for (int kt = k0; kt < k1; kt += PERIOD) {
#pragma unroll
      for (int i = 0; i < PERIOD; ++i) ktile(kt + i, i);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

    if constexpr (!SPLIT) {
      if constexpr (F8) scale_acc<EPI, BM>(g, acc, tm, tn, wm, wn, lane);
      // every wave is past its last fragment read of the ring before any
      // wave stages into it; wave w stages into ring array w (>= 16 KB, as
      // much as a wave stages)
      __syncthreads();
      char* const st = reinterpret_cast<char*>(wave == 0   ? s_a0
                                               : wave == 1 ? s_a1
                                               : wave == 2 ? s_w0
                                                           : s_w1);
      epilogue<EPI, BM>(g, acc, tm, tn, wm, wn, lane, st, s_rs);
    } else {
      float4* dst = partial_slot<BM>(g, slot, wave, lane);
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        // 32-row blocks wholly past M are neither stored nor read back
        if (tm * BM + (wm * MB + i) * 32 >= g.M) continue;
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const f32x16& a = acc[i][j];
            dst[((i * NB + j) * 4 + rr) * 64] =
                make_float4(a[4 * rr], a[4 * rr + 1], a[4 * rr + 2], a[4 * rr + 3]);
          }
      }
    }
  };

  if (dp) {
    item(std::false_type{}, xcd_remap(blockIdx.x, g.n_dp), 0, KT, -1);
  } else {
    const int n_items = end0 < u1 ? 2 : 1;
    for (int it = 0; it < n_items; ++it) {
      // the ring is refilled for the next tile only after every wave is done
      if (it) __syncthreads();
      item(std::true_type{}, g.n_dp + t0 + it, it ? 0 : (u0 - t0 * upt) * PERIOD,
           it ? (u1 - (t0 + 1) * upt) * PERIOD : (end0 - t0 * upt) * PERIOD, 2 * p + it);
    }
  }
}

// Sums the partial tiles of the split tiles in K order (fixed, so results are
// bitwise reproducible) and applies the epilogue.  One thread per pair of
// 16-byte accumulator groups (blocks 2 jp and 2 jp + 1 of one wave, one rr,
// one lane), so each wave load reads 1 KB contiguously and every thread has
// two independent loads per partial in flight.
template <int EPI, int BM, bool F8>
__global__ __launch_bounds__(256) void gemm_fixup_kernel(GemmArgs g) {
  using T = Tile<BM>;
  constexpr int MB = T::MB, NB = T::NB;
  constexpr int PER_TILE = BM * BN / 8;  // threads per tile
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int t_rel = t / PER_TILE;
  int rem = t - t_rel * PER_TILE;
  const int lane = rem & 63;
  rem >>= 6;
  const int rr = rem & 3;
  rem >>= 2;
  const int jp = rem % (NB / 2);
  rem /= NB / 2;
  const int i = rem % MB;
  const int wave = rem / MB;
  const int wm = wave / T::WN, wn = wave % T::WN;
  int tm, tn;
  tile_coords<BM>(g, g.n_dp + t_rel, tm, tn);
  // the split items store no 32-row block that lies wholly past M
  if (tm * BM + (wm * MB + i) * 32 >= g.M) return;
  const int upt = g.KT / g.unit;
  const int units = g.n_tail * upt;
  const int ua = t_rel * upt, ub = ua + upt;  // this tile's units
  // first and last pieces that touch the tile
  int pa = (int)(((long long)ua * g.n_pieces) / units);
  while (pa > 0 && piece_start(pa, units, g.n_pieces) > ua) --pa;
  while (piece_start(pa + 1, units, g.n_pieces) <= ua) ++pa;
  int pb = pa;
  while (pb + 1 < g.n_pieces && piece_start(pb + 1, units, g.n_pieces) < ub) ++pb;

  const int g0 = ((i * NB + 2 * jp) * 4 + rr) * 64;  // group offsets in float4
  const int g1 = g0 + 4 * 64;
  float a[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f};
  // The pieces' partials are independent loads: up to FIX_BATCH of them are
  // issued before they are summed (one at a time, the sum would wait one L2
  // round trip per piece).  They are added in piece order, as one at a time.
  constexpr int FIX_BATCH = 8;
  const int pa_second = piece_start(pa, units, g.n_pieces) < ua ? 1 : 0;
  for (int p0 = pa; p0 <= pb; p0 += FIX_BATCH) {
    float4 va[FIX_BATCH], vb[FIX_BATCH];
#pragma unroll
    for (int u = 0; u < FIX_BATCH; ++u) {
      const int p = p0 + u;
      va[u] = vb[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (p <= pb) {
        // the tile is a piece's second item when the piece began in an
        // earlier tile, which only the first piece pa can have done
        const int slot = 2 * p + (p == pa ? pa_second : 0);
        const float4* src = partial_slot<BM>(g, slot, wave, lane);
        va[u] = src[g0];
        vb[u] = src[g1];
      }
    }
#pragma unroll
    for (int u = 0; u < FIX_BATCH; ++u) {
      if (p0 + u > pb) break;
      a[0] += va[u].x; a[1] += va[u].y; a[2] += va[u].z; a[3] += va[u].w;
      b[0] += vb[u].x; b[1] += vb[u].y; b[2] += vb[u].z; b[3] += vb[u].w;
    }
  }
  if constexpr (F8) {
    const int ln = lane & 31, hl = lane >> 5;
    const float sr = g.sa[min(tm * BM + (wm * MB + i) * 32 + ln, g.M - 1)];
    const int r0 = (wn * NB + 2 * jp) * 32 + 8 * rr + 4 * hl;
    const float4 wa = *reinterpret_cast<const float4*>(g.sw + weight_row<EPI, NB>(g, tn, r0));
    const float4 wb = *reinterpret_cast<const float4*>(g.sw + weight_row<EPI, NB>(g, tn, r0 + 32));
    a[0] *= sr * wa.x; a[1] *= sr * wa.y; a[2] *= sr * wa.z; a[3] *= sr * wa.w;
    b[0] *= sr * wb.x; b[1] *= sr * wb.y; b[2] *= sr * wb.z; b[3] *= sr * wb.w;
  }
  epilogue_pair<EPI, BM>(g, tm, tn, wm, wn, lane, i, jp, rr, a, b);
}

}  // namespace

// Compute units of the current device (queried once per device).
int device_cus() {
  // several host threads may fill an entry at once; they store the same value
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

namespace {

// Work plan of one GEMM launch.  With one workgroup per CU at a time, tiles
// run in rounds of `cus`.  A last round holding only a few tiles would leave
// most CUs idle for a whole tile time, so when at least one full round exists
// and the last round is at most half full, its tail tiles are cut along K
// into pieces of whole units (the K loop's unroll period of 6 or 2 k tiles),
// one piece per CU (or per unit when there are fewer units than CUs); the
// fix-up kernel then sums each tile's fp32 partials in K order and runs the
// epilogue.
// K loop unroll period in k tiles: 6 (3 A slots) when it divides K / BK,
// else 2 (K is a multiple of 128 for every supported shape).
int unroll_period(int KT) { return KT % 6 == 0 ? 6 : 2; }

struct Plan {
  int bm, tiles, n_dp, n_tail, n_pieces;
  float cost;  // estimated time in tile times
};

Plan make_plan(int bm, int M, int KT, int num_n, bool can_split, float fix_per_tile) {
  const int cus = device_cus();
  Plan p{};
  p.bm = bm;
  p.tiles = ((M + bm - 1) / bm) * num_n;
  const int full = p.tiles / cus, tail = p.tiles - full * cus;
  const int upt = KT / unroll_period(KT);
  // cost is counted in rounds of tiles, a tile's time in units of a 256-row
  // tile's: a 224-row tile has 7/8 of its MFMAs, plus an epilogue, prologue
  // and workgroup turnover of about an eighth of a 256-row tile that do not
  // shrink (measured per tile with cycle counters)
  const float tile_time = bm == 256 ? 1.0f : bm == 224 ? 0.89f : 0.56f;
  // a last round at most half full is split; so is a launch with at most
  // half as many tiles as CUs (a short sequence, e.g. an 80- or 160-token
  // text stage): then every tile is cut, so all CUs share the weight stream
  const bool split_tail = full >= 1 && tail > 0 && 2 * tail <= cus;
  const bool split_all = full == 0 && tail > 0 && 2 * tail <= cus;
  if (can_split && (split_tail || split_all)) {
    p.n_dp = full * cus;
    p.n_tail = tail;
    p.n_pieces = min(min(cus, kMaxPieces), tail * upt);
    // the longest piece, plus partial stores and the fix-up pass, which
    // grows with the tiles it sums by fix_per_tile tile times each
    const int units = tail * upt;
    const int longest = (units + p.n_pieces - 1) / p.n_pieces;
    p.cost = tile_time * (full + (float)longest / upt + 0.1f + fix_per_tile * tail);
  } else {
    p.n_dp = p.tiles;
    p.n_tail = 0;
    p.n_pieces = 0;
    p.cost = tile_time * ((p.tiles + cus - 1) / cus);
  }
  return p;
}

// The 224-row layout (1 x 4 waves) gives a better round count for some M
// (4,256 tokens x 12 output tiles: 228 tiles in one round, where 256-row tiles
// need 204 but each is slower; the 4,256-token input projection: 19 full
// 224-row tiles against 17 256-row ones with a 160-row remainder); the
// cheaper plan wins, ties going to the shorter tile.  `ok` rejects a plan
// (falling back to the same height without a split) whose split tail would
// hold q or k tiles: the fix-up's epilogue does not normalize or rotate.
//
// 128-row tiles (1 x 4 waves of 128 x 64) serve sequences of at most 128
// tokens when every tile is split and the weight-streaming kernels of
// thin.hip do not take the shape (an 80-token block: one row of tiles, where
// a 224-row tile would run 2.8 times the MFMAs the 80 rows need).
// Their whole-tile epilogues are then never used; bf16 only.  For longer
// sequences they were measured slower than 224-row tiles (336 tokens, output
// projection: more tiles with the same fixed costs each).
template <class Ok>
Plan pick_plan(int M, int KT, int num_n, bool can_split, bool allow128, float fix_per_tile, Ok ok) {
  auto plan = [&](int bm) {
    const Plan p = make_plan(bm, M, KT, num_n, can_split, fix_per_tile);
    return ok(p) ? p : make_plan(bm, M, KT, num_n, false, fix_per_tile);
  };
  const Plan a = plan(224), b = plan(256);
  Plan best = a.cost <= b.cost ? a : b;
  if (allow128 && can_split && M <= 128) {
    const Plan c = make_plan(128, M, KT, num_n, true, fix_per_tile);
    if (c.n_dp == 0 && c.n_tail > 0 && ok(c) && c.cost < best.cost) best = c;
  }
  return best;
}

// Fix-up cost per split tail tile, in tile times.  FP8: 14.4 us for the 44
// tail tiles of the 4,256-token input projection with 256-row tiles, about
// 0.3 of its tile time; with it that projection takes 224-row tiles (4 tail
// tiles), measured 350 against 363 us.  bf16: the plans were tuned and
// measured with the fix-up as a flat 0.1 (its per-tile cost, about 0.003,
// would only flip near-ties that were not measured).
template <bool F8>
constexpr float kFixPerTile = F8 ? 0.007f : 0.0f;

template <int EPI, bool F8>
hipError_t launch(GemmArgs g, hipStream_t stream) {
  const bool can_split = g.partial != nullptr;
  bool qk_after = false;
  g.KT = g.K * (F8 ? 1 : 2) / 128;
  Plan p;
  if constexpr (EPI == EPI_IN) {
    // Split tail tiles end in the fix-up kernel, whose epilogue does not
    // normalize or rotate, so a tail must hold no q or k tile (tail tiles are
    // the last in tile order, i.e. the highest N tiles: MLP ones).
    const int num_qk = 2 * g.D / BN;
    p = pick_plan(g.M, g.KT, g.num_n, can_split, !F8, kFixPerTile<F8>, [&](const Plan& q) {
      const int num_m = (g.M + q.bm - 1) / q.bm;
      return !(q.n_tail && q.n_dp > 0 && (q.n_dp / (GROUP_N * num_m)) * GROUP_N < num_qk);
    });
    // with every tile split, the fix-up stores q and k as summed, and the
    // norm + RoPE pass runs on them afterwards
    qk_after = p.n_tail > 0 && p.n_dp == 0;
  } else {
    p = pick_plan(g.M, g.KT, g.num_n, can_split, !F8, kFixPerTile<F8>,
                  [](const Plan&) { return true; });
  }
  g.n_dp = p.n_dp;
  g.n_tail = p.n_tail;
  g.n_pieces = p.n_pieces;
  g.unit = unroll_period(g.KT);
  const int grid = g.n_dp + (g.n_tail ? g.n_pieces : 0);
  if (p.bm == 256) {
    if (g.unit == 6)
      hipLaunchKernelGGL((gemm_kernel<EPI, 256, 3, F8>), dim3(grid), dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL((gemm_kernel<EPI, 256, 2, F8>), dim3(grid), dim3(256), 0, stream, g);
    if (g.n_tail)
      hipLaunchKernelGGL((gemm_fixup_kernel<EPI, 256, F8>), dim3(g.n_tail * 256 * BN / 8 / 256),
                         dim3(256), 0, stream, g);
  } else if (p.bm == 128) {
    if constexpr (!F8) {
      if (g.unit == 6)
        hipLaunchKernelGGL((gemm_kernel<EPI, 128, 3, false>), dim3(grid), dim3(256), 0, stream, g);
      else
        hipLaunchKernelGGL((gemm_kernel<EPI, 128, 2, false>), dim3(grid), dim3(256), 0, stream, g);
      hipLaunchKernelGGL((gemm_fixup_kernel<EPI, 128, false>), dim3(g.n_tail * 128 * BN / 8 / 256),
                         dim3(256), 0, stream, g);
    }
  } else {
    if (g.unit == 6)
      hipLaunchKernelGGL((gemm_kernel<EPI, 224, 3, F8>), dim3(grid), dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL((gemm_kernel<EPI, 224, 2, F8>), dim3(grid), dim3(256), 0, stream, g);
    if (g.n_tail)
      hipLaunchKernelGGL((gemm_fixup_kernel<EPI, 224, F8>), dim3(g.n_tail * 224 * BN / 8 / 256),
                         dim3(256), 0, stream, g);
  }
  if (qk_after) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_rope4(g.q, g.k, g.pos, g.q_scale, g.k_scale, g.M, g.D / 128, g.theta,
                        g.qk_eps, g.q_mul, stream);
  }
  return hipGetLastError();
}

}  // namespace

namespace {

GemmArgs in_args(const void* u, const void* w_in, int M, int D, int F, uint16_t* q, uint16_t* k,
                 uint16_t* v, uint16_t* cat, const int32_t* pos, const uint16_t* q_scale,
                 const uint16_t* k_scale, float theta, float qk_eps, float* partial) {
  GemmArgs g{};
  g.pos = pos;
  g.q_scale = q_scale;
  g.k_scale = k_scale;
  g.qk_eps = qk_eps;
  g.q_mul = 1.0f;
  g.theta = theta;
  const double two_pi = 6.283185307179586;
  for (int j = 0; j < 16; ++j) {
    const double rev = pow((double)theta, -2.0 * j / 32.0) / two_pi;
    int e;
    frexp(rev, &e);  // rev = m 2^e, 0.5 <= m < 1
    const double hi = ldexp(nearbyint(ldexp(rev, 8 - e)), e - 8);
    g.rope_hi[j] = (float)hi;  // exact: 8 significant bits
    g.rope_lo[j] = (float)(rev - hi);
  }
  g.partial = partial;
  g.A = static_cast<const uint16_t*>(u);
  g.W = static_cast<const uint16_t*>(w_in);
  g.M = M;
  g.K = D;
  g.num_n = 3 * D / BN + F / 128;
  g.D = D;
  g.F = F;
  g.q = q;
  g.k = k;
  g.v = v;
  g.cat = cat;
  return g;
}

GemmArgs out_args(const void* cat, const void* w_out, int M, int D, int F, const uint16_t* x,
                  const uint16_t* mod, uint16_t* y, int e0, int e1, uint32_t flags,
                  float* partial) {
  GemmArgs g{};
  g.partial = partial;
  g.A = static_cast<const uint16_t*>(cat);
  g.W = static_cast<const uint16_t*>(w_out);
  g.M = M;
  g.K = D + F;
  g.num_n = D / BN;
  g.D = D;
  g.F = F;
  g.x = x;
  g.mod = mod;
  g.y = y;
  g.e0 = e0;
  g.e1 = e1;
  g.flags = flags;
  return g;
}

}  // namespace

hipError_t launch_gemm_in(const uint16_t* u, const uint16_t* w_in, int M, int D, int F,
                          uint16_t* q, uint16_t* k, uint16_t* v, uint16_t* cat,
                          const int32_t* pos, const uint16_t* q_scale, const uint16_t* k_scale,
                          float theta, float qk_eps, float q_mul, float* partial,
                          hipStream_t stream) {
  if (thin_fits(M, D, F))
    return launch_thin_in(u, w_in, M, D, F, q, k, v, cat, pos, q_scale, k_scale, theta, qk_eps,
                          q_mul, stream);
  GemmArgs g = in_args(u, w_in, M, D, F, q, k, v, cat, pos, q_scale, k_scale, theta, qk_eps,
                       partial);
  g.q_mul = q_mul;
  return launch<EPI_IN, false>(g, stream);
}

hipError_t launch_gemm_out(const uint16_t* cat, const uint16_t* w_out, int M, int D, int F,
                           const uint16_t* x, const uint16_t* mod, uint16_t* y, int e0, int e1,
                           uint32_t flags, float* partial, hipStream_t stream, int* counters,
                           int n_counters) {
  if (thin_fits(M, D, F))
    return launch_thin_out(cat, w_out, M, D, F, x, mod, y, e0, e1, flags, partial,
                           partial ? kGemmPartialBytes : 0, counters, n_counters, stream);
  return launch<EPI_OUT, false>(out_args(cat, w_out, M, D, F, x, mod, y, e0, e1, flags, partial),
                                stream);
}

hipError_t launch_gemm_in_fp8(const uint8_t* u8, const float* u_scale, const uint8_t* w_in8,
                              const float* w_in_scale, int M, int D, int F, uint16_t* q,
                              uint16_t* k, uint16_t* v, uint16_t* cat, const int32_t* pos,
                              const uint16_t* q_scale, const uint16_t* k_scale, float theta,
                              float qk_eps, float q_mul, float* partial, hipStream_t stream) {
  GemmArgs g = in_args(u8, w_in8, M, D, F, q, k, v, cat, pos, q_scale, k_scale, theta, qk_eps,
                       partial);
  g.q_mul = q_mul;
  g.sa = u_scale;
  g.sw = w_in_scale;
  return launch<EPI_IN, true>(g, stream);
}

hipError_t launch_gemm_out_fp8(const uint8_t* cat8, const float* cat_scale,
                               const uint8_t* w_out8, const float* w_out_scale, int M, int D,
                               int F, const uint16_t* x, const uint16_t* mod, uint16_t* y,
                               int e0, int e1, uint32_t flags, float* partial,
                               hipStream_t stream) {
  GemmArgs g = out_args(cat8, w_out8, M, D, F, x, mod, y, e0, e1, flags, partial);
  g.sa = cat_scale;
  g.sw = w_out_scale;
  return launch<EPI_OUT, true>(g, stream);
}

}  // namespace dit
