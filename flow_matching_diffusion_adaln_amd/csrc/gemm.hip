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
// 2 x 2, 128 x 128 each) or BM = 224 (4 waves in 1 x 4, 224 x 64 each), built
// from v_mfma_f32_32x32x16_bf16 blocks with the fp32 accumulators in AGPRs.
// The host picks the tile height: fewest rounds of tiles over the CUs, then
// the shorter tile (224 divides the 4,256-token sequence into 19 tiles, 256
// leaves a 160-row remainder).  The K loop streams 32-wide k
// tiles from L2/HBM straight into LDS with 16-byte direct-to-LDS loads
// through a 4-stage ring: loads run three tiles ahead of the MFMAs, which
// hides the L2-miss latency that a double buffer exposes.  The 16-byte chunk
// index is xor-swizzled by the row so fragment reads are bank-conflict free.
// Tiles are ordered XCD-aware: each XCD takes one contiguous range of tiles,
// walked in groups of 4 N-tiles so the A and W panels in flight on one XCD
// stay few and L2-resident.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int BN = 256, BK = 32;
constexpr int STAGES = 4;            // LDS ring depth; loads run STAGES - 1 tiles ahead
constexpr int CH = BK / 8;           // 16-byte chunks per tile row (4)
constexpr int RPI = 64 / CH;         // tile rows filled by one 1 KB wave load (16)
constexpr int NLD = 4;               // loads per wave per k tile, for each of A and W
constexpr int GROUP_N = 4;

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
  // output projection
  const uint16_t* x;  // residual [M, D]
  const uint16_t* mod;  // [S, 3, D]
  uint16_t* y;        // [M, D]
  int e0, e1;         // stream boundaries
  uint32_t flags;
};

// Tile geometry: BM rows, WM x WN waves, MB x NB blocks of 32 x 32 per wave.
template <int BM_>
struct Tile {
  static constexpr int BM = BM_;
  static constexpr int WM = BM_ == 256 ? 2 : 1;
  static constexpr int WN = 4 / WM;
  static constexpr int MB = BM_ / (32 * WM);
  static constexpr int NB = BN / (32 * WN);
  static constexpr int A_SLABS = BM_ / RPI;  // 1 KB loads that fill the A tile
  static_assert(MB * 32 * WM == BM_ && NB * 32 * WN == BN, "tile geometry");
  static_assert(NB % 2 == 0, "gate and up blocks pair up inside a wave");
  static_assert(A_SLABS <= 4 * NLD && A_SLABS > 4 * (NLD - 1), "A tile loads");
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

// LDS tiles are rows of 32 bf16 (64 B = 4 chunks of 16 B).  gfx950's LDS has
// 64 banks of 4 B, so 16 lanes of a 16-byte read are served per cycle: the
// 16 consecutive rows one MFMA fragment read touches must land on 16
// distinct 16-byte bank slots.  Row r covers slots 4 (r % 4) .. + 3, so the
// chunk is xor-ed with (r >> 2) & 3, a bijection on the 4 rows of each class.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

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

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
  return make_uint2(pack2(a, b), pack2(c, d));
}

template <int EPI, int BM>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs g) {
  using T = Tile<BM>;
  constexpr int MB = T::MB, NB = T::NB;
  // One LDS array per ring stage (A tile, then W tile), not one indexed array:
  // the compiler tracks direct-to-LDS stores per LDS variable, so it can see
  // that fragment reads of one stage never alias the loads in flight into the
  // others and does not wait on them.  (It tracks only a few variables, hence
  // A and W share one array per stage.)
  __shared__ __attribute__((aligned(16))) uint16_t s_st0[(BM + BN) * BK];
  __shared__ __attribute__((aligned(16))) uint16_t s_st1[(BM + BN) * BK];
  __shared__ __attribute__((aligned(16))) uint16_t s_st2[(BM + BN) * BK];
  __shared__ __attribute__((aligned(16))) uint16_t s_st3[(BM + BN) * BK];
  uint16_t* const ring[STAGES] = {s_st0, s_st1, s_st2, s_st3};

  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar: LDS addresses of the direct loads (M0) then come
  // from scalar arithmetic instead of a v_readfirstlane per load
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WN, wn = wave % T::WN;
  const int ln = lane & 31, hl = lane >> 5;

  const int num_m = (g.M + BM - 1) / BM;
  const int id = xcd_remap(blockIdx.x, num_m * g.num_n);
  const int grp = id / (GROUP_N * num_m);
  const int rem = id - grp * GROUP_N * num_m;
  const int gw = min(GROUP_N, g.num_n - grp * GROUP_N);
  const int tm = rem / gw;
  const int tn = grp * GROUP_N + rem % gw;

  // Global -> LDS with gfx950's 16-byte direct loads (no staging registers).
  // One wave instruction fills 1 KB of LDS = 16 tile rows of 64 B (a slab);
  // lane i lands in row 16 s + i / 4 at physical chunk i % 4, which holds
  // logical chunk (i % 4) ^ swz(row), so that is the chunk the lane fetches.
  // Wave w loads slabs 4 w .. 4 w + 3 of both tiles; when the A tile has
  // fewer slabs (BM = 224) the last wave reloads its last slab, writing the
  // same bytes to the same place, so every wave issues the same count.
  const int lrow = lane / CH;
  // byte offsets in 32 bits: the loads then use the scalar-base + vector-offset form
  uint32_t aoff[NLD], boff[NLD];
  int aslab[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    aslab[j] = min(wave * NLD + j, T::A_SLABS - 1);
    const int ra = aslab[j] * RPI + lrow;
    const int rb = (wave * NLD + j) * RPI + lrow;
    const int arow = min(tm * BM + ra, g.M - 1);
    aoff[j] = ((uint32_t)arow * (uint32_t)g.K + (((lane % CH) ^ swz(ra)) * 8)) * 2u;
    boff[j] = ((uint32_t)weight_row<EPI, NB>(g, tn, rb) * (uint32_t)g.K +
               (((lane % CH) ^ swz(rb)) * 8)) * 2u;
  }
  const char* abase = reinterpret_cast<const char*>(g.A);
  const char* bbase = reinterpret_cast<const char*>(g.W);
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const int KT = g.K / BK;  // a multiple of STAGES for every supported shape
  // tile kt -> ring stage st; past the end the last tile is reloaded into the
  // idle stage (never read), so the loop needs no branches
  auto gload = [&](int kt, uint16_t* st) __attribute__((always_inline)) {
    const uint32_t ko = (uint32_t)min(kt, KT - 1) * (BK * 2);
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      __builtin_amdgcn_global_load_lds(abase + (aoff[j] + ko),
                                       (lds_ptr)(st + aslab[j] * RPI * BK), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(bbase + (boff[j] + ko),
                                       (lds_ptr)(st + BM * BK + (wave * NLD + j) * RPI * BK),
                                       16, 0, 0);
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // MFMA fragments, double-buffered in registers: while the MFMAs of one
  // 16-wide k step run, the fragment reads of the next step are in flight.
  bf16x8 fa[2][MB], fb[2][NB];
  auto read_frags = [&](const uint16_t* st, int ks, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int r = (wm * MB + i) * 32 + ln;
      fa[slot][i] = *reinterpret_cast<const bf16x8*>(&st[r * BK + (((2 * ks + hl) ^ swz(r)) << 3)]);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int r = (wn * NB + j) * 32 + ln;
      fb[slot][j] = *reinterpret_cast<const bf16x8*>(&st[BM * BK + r * BK + (((2 * ks + hl) ^ swz(r)) << 3)]);
    }
  };
  // C^T = W A^T: the weights are the A operand, so each lane ends up owning
  // an output row (see the epilogue)
  auto mfmas = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[slot][j], fa[slot][i], acc[i][j], 0, 0, 0);
  };
  // One k tile from ring stage s.  The instruction order is pinned (the
  // compiler would otherwise sink the loads next to the waits and pair each
  // fragment read with its first use).  The first k step interleaves its
  // MFMAs with the loads of the tile STAGES - 1 ahead and the fragment reads
  // of the second step.  The barrier then comes before the second k step,
  // whose fragments are already in registers: the next tile's first fragment
  // reads overlap those MFMAs instead of stalling after the barrier.  That is
  // safe because every read of stage s has completed before the barrier
  // (lgkmcnt(0)), and stage s is refilled only after it.
  auto ktile = [&](int kt, int s) __attribute__((always_inline)) {
    gload(kt + STAGES - 1, ring[(s + STAGES - 1) % STAGES]);
    read_frags(ring[s], 1, 1);
    mfmas(0);
#pragma unroll
    for (int i = 0; i < MB * NB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 global load
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
    // tile kt + 1 must have landed; the STAGES - 2 younger tiles may still fly
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NLD * (STAGES - 2)));
    __builtin_amdgcn_s_waitcnt(LGKMCNT0);
    ring_barrier();
    read_frags(ring[(s + 1) % STAGES], 0, 0);
    mfmas(1);
#pragma unroll
    for (int i = 0; i < MB * NB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) gload(s, ring[s]);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NLD * (STAGES - 2)));
  ring_barrier();
  read_frags(ring[0], 0, 0);
  for (int kt = 0; kt < KT; kt += STAGES) {
#pragma unroll
    for (int s = 0; s < STAGES; ++s) ktile(kt + s, s);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // Epilogue.  The MFMAs compute C^T, so in block (i, j) lane (ln, hl) holds
  // output row (wm MB + i) 32 + ln and the 4 consecutive columns
  // (wn NB + j) 32 + 8 rr + 4 hl .. + 3 in registers 4 rr .. 4 rr + 3: every
  // store, residual load and gate load is 8 contiguous bytes.
  const int row_base = tm * BM + wm * MB * 32 + ln;
  const int col_base = tn * BN + wn * NB * 32 + 4 * hl;
  if (EPI == EPI_IN) {
    const int n_qkv = 3 * g.D / BN;
    if (tn < n_qkv) {
      // q | k | v: 4 consecutive columns never straddle a D boundary
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int row = row_base + i * 32;
        if (row >= g.M) continue;
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int col = col_base + j * 32 + 8 * rr;
            const int which = col / g.D;
            uint16_t* dst = which == 0 ? g.q : which == 1 ? g.k : g.v;
            const f32x16& a = acc[i][j];
            *reinterpret_cast<uint2*>(dst + (size_t)row * g.D + (col - which * g.D)) =
                pack4(a[4 * rr], a[4 * rr + 1], a[4 * rr + 2], a[4 * rr + 3]);
          }
      }
    } else {
      // SwiGLU: block 2p holds gate, block 2p + 1 up, of the same hidden units
      const int ldc = g.D + g.F;
      const int hid_base = (tn - n_qkv) * 128 + wn * (NB / 2) * 32 + 4 * hl;
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int row = row_base + i * 32;
        if (row >= g.M) continue;
        uint16_t* dst = g.cat + (size_t)row * ldc + g.D;
#pragma unroll
        for (int p = 0; p < NB / 2; ++p)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const f32x16& ga = acc[i][2 * p];
            const f32x16& up = acc[i][2 * p + 1];
            float m[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) m[e] = silu(ga[4 * rr + e]) * up[4 * rr + e];
            *reinterpret_cast<uint2*>(dst + hid_base + p * 32 + 8 * rr) = pack4(m[0], m[1], m[2], m[3]);
          }
      }
    }
  } else {
    const bool use_gate = !(g.flags & 2u), use_res = !(g.flags & 1u);
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int row = row_base + i * 32;
      if (row >= g.M) continue;
      const uint16_t* gate = g.mod + (size_t)stream_of(row, g.e0, g.e1) * 3 * g.D + 2 * g.D;
      const uint16_t* xr = g.x + (size_t)row * g.D;
      uint16_t* yr = g.y + (size_t)row * g.D;
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int col = col_base + j * 32 + 8 * rr;
          const uint2 gv = use_gate ? *reinterpret_cast<const uint2*>(gate + col)
                                    : make_uint2(0x3f803f80u, 0x3f803f80u);
          const uint2 xv = use_res ? *reinterpret_cast<const uint2*>(xr + col) : make_uint2(0u, 0u);
          const f32x16& a = acc[i][j];
          *reinterpret_cast<uint2*>(yr + col) =
              pack4(fmaf(lo2f(gv.x), a[4 * rr], lo2f(xv.x)), fmaf(hi2f(gv.x), a[4 * rr + 1], hi2f(xv.x)),
                    fmaf(lo2f(gv.y), a[4 * rr + 2], lo2f(xv.y)), fmaf(hi2f(gv.y), a[4 * rr + 3], hi2f(xv.y)));
        }
    }
  }
}

// Compute units of the current device (queried once per device).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Tile height for M rows: fewest rounds of tiles over the CUs (one workgroup
// per CU at a time), then the shorter tile.  The 224-row layout moves more
// LDS data per MFMA than the 256-row one, so it only pays when it does not
// add a round (4,256 tokens x 12 output tiles: 228 tiles in one round
// instead of 204 taller ones).
int pick_bm(int M, int num_n) {
  const int cus = device_cus();
  auto rounds = [&](int bm) {
    const long tiles = (long)((M + bm - 1) / bm) * num_n;
    return (tiles + cus - 1) / cus;
  };
  return rounds(224) <= rounds(256) ? 224 : 256;
}

template <int EPI>
hipError_t launch(const GemmArgs& g, hipStream_t stream) {
  const int bm = pick_bm(g.M, g.num_n);
  const int tiles = ((g.M + bm - 1) / bm) * g.num_n;
  if (bm == 224)
    hipLaunchKernelGGL((gemm_kernel<EPI, 224>), dim3(tiles), dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL((gemm_kernel<EPI, 256>), dim3(tiles), dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_in(const uint16_t* u, const uint16_t* w_in, int M, int D, int F,
                          uint16_t* q, uint16_t* k, uint16_t* v, uint16_t* cat,
                          hipStream_t stream) {
  GemmArgs g{};
  g.A = u;
  g.W = w_in;
  g.M = M;
  g.K = D;
  g.num_n = 3 * D / BN + F / 128;
  g.D = D;
  g.F = F;
  g.q = q;
  g.k = k;
  g.v = v;
  g.cat = cat;
  return launch<EPI_IN>(g, stream);
}

hipError_t launch_gemm_out(const uint16_t* cat, const uint16_t* w_out, int M, int D, int F,
                           const uint16_t* x, const uint16_t* mod, uint16_t* y, int e0, int e1,
                           uint32_t flags, hipStream_t stream) {
  GemmArgs g{};
  g.A = cat;
  g.W = w_out;
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
  return launch<EPI_OUT>(g, stream);
}

}  // namespace dit
