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
// Tiling for gfx950: 256 x 256 x 64 workgroup tile, 4 waves in 2 x 2, each
// wave 128 x 128 as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 (256 fp32
// accumulators per lane).  A and W tiles are staged through LDS, double
// buffered (2 x 64 KB), with the 16-byte chunk index xor-swizzled by the row
// so the MFMA fragment reads are bank-conflict free.  Tiles are ordered XCD-aware: each XCD takes one contiguous range of
// tiles, walked in groups of 4 N-tiles so the A and W panels in flight on one
// XCD stay few and L2-resident.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
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

// Weight row feeding row r (0..255) of N-tile tn.
template <int EPI>
__device__ __forceinline__ int weight_row(const GemmArgs& g, int tn, int r) {
  if (EPI == EPI_IN) {
    const int n_qkv = 3 * g.D / BN;
    if (tn < n_qkv) return tn * BN + r;
    // MLP tile: 128 hidden units; within a wave's 128 rows the 32-row groups
    // alternate gate, up, gate, up
    const int wn = r >> 7, grp = (r >> 5) & 3, i = r & 31;
    const int hidden = (tn - n_qkv) * 128 + wn * 64 + (grp >> 1) * 32 + i;
    return 3 * g.D + (grp & 1) * g.F + hidden;
  }
  return tn * BN + r;
}

// LDS tiles are rows of 64 bf16 (128 B = 8 chunks of 16 B).  gfx950's LDS has
// 64 banks of 4 B, so 16 lanes of a 16-byte read are served per cycle: the
// 16 consecutive rows one MFMA fragment read touches must land on 16
// distinct 16-byte bank slots.  Row r covers slots 8 (r % 2) .. + 7, so the
// chunk is xor-ed with (r >> 1) & 7, a bijection on the 8 rows of each parity.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Wait for this wave's outstanding vector-memory operations, including the
// direct-to-LDS loads, before the barrier that publishes the tile.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs g) {
  // Four distinct LDS arrays (not one indexed array) so the compiler can see
  // that fragment reads of one stage never alias the direct-to-LDS loads in
  // flight into the other, and does not wait on those loads before reading.
  __shared__ __attribute__((aligned(16))) uint16_t s_a0[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t s_b0[BN * BK];
  __shared__ __attribute__((aligned(16))) uint16_t s_a1[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t s_b1[BN * BK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ln = lane & 31, hl = lane >> 5;

  const int num_m = (g.M + BM - 1) / BM;
  const int id = xcd_remap(blockIdx.x, num_m * g.num_n);
  const int grp = id / (GROUP_N * num_m);
  const int rem = id - grp * GROUP_N * num_m;
  const int gw = min(GROUP_N, g.num_n - grp * GROUP_N);
  const int tm = rem / gw;
  const int tn = grp * GROUP_N + rem % gw;

  // Global -> LDS with gfx950's 16-byte direct loads (no staging registers).
  // One wave instruction fills 1 KB of LDS = 8 tile rows of 128 B; lane i
  // lands in row 8 j' + i / 8 at physical chunk i % 8, which holds logical
  // chunk (i % 8) ^ swz(row) of the swizzled layout, so that is the chunk
  // the lane fetches.  Wave w fills rows [64 w, 64 w + 64) of both tiles.
  const int lrow = lane >> 3;                  // row inside the 8-row slab
  // byte offsets in 32 bits: the loads then use the scalar-base + vector-offset form
  uint32_t aoff[8], boff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = wave * 64 + 8 * j + lrow;
    const int lch = (lane & 7) ^ swz(r);       // logical chunk this lane fetches
    const int arow = min(tm * BM + r, g.M - 1);
    aoff[j] = ((uint32_t)arow * (uint32_t)g.K + lch * 8) * 2u;
    boff[j] = ((uint32_t)weight_row<EPI>(g, tn, r) * (uint32_t)g.K + lch * 8) * 2u;
  }
  const char* abase = reinterpret_cast<const char*>(g.A);
  const char* bbase = reinterpret_cast<const char*>(g.W);
  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto gload = [&](int kt, uint16_t* sa, uint16_t* sb) {
    const uint32_t ko = (uint32_t)kt * (BK * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int slab = (wave * 64 + 8 * j) * BK;
      __builtin_amdgcn_global_load_lds(abase + (aoff[j] + ko), (lds_ptr)(sa + slab), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(bbase + (boff[j] + ko), (lds_ptr)(sb + slab), 16, 0, 0);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = g.K / BK;  // even for every supported shape
  // MFMA fragments, double-buffered in registers: while the 16 MFMAs of one
  // 16-wide k step run, the 8 fragment reads of the next step are in flight.
  bf16x8 fa[2][4], fb[2][4];
  auto read_frags = [&](const uint16_t* sa, const uint16_t* sb, int ks, int slot) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + i * 32 + ln;
      fa[slot][i] = *reinterpret_cast<const bf16x8*>(&sa[r * BK + (((2 * ks + hl) ^ swz(r)) << 3)]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 128 + j * 32 + ln;
      fb[slot][j] = *reinterpret_cast<const bf16x8*>(&sb[r * BK + (((2 * ks + hl) ^ swz(r)) << 3)]);
    }
  };
  auto mfmas = [&](int slot) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
  };
  // One k tile: compute from (ca, cb) while the next tile streams into (na, nb).
  // The last tile reloads itself into the idle buffer, which is never read;
  // that keeps the body free of branches.  The instruction order is pinned:
  // the compiler would otherwise sink the global loads next to the wait at
  // the end of the tile (no overlap) and pair each fragment read with its
  // first use.  Each 16-wide k step issues its 16 MFMAs (512 cycles)
  // interleaved with the next step's 8 fragment reads; the first step also
  // carries the 16 direct-to-LDS loads of the next tile.
  auto ktile = [&](int kt, const uint16_t* ca, const uint16_t* cb, uint16_t* na, uint16_t* nb) {
    gload(min(kt + 1, KT - 1), na, nb);
    read_frags(ca, cb, 1, 1);
    mfmas(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // 2 VMEM loads
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 DS read
    }
    __builtin_amdgcn_sched_barrier(0);
    read_frags(ca, cb, 2, 0);
    mfmas(1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(ca, cb, 3, 1);
    mfmas(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(1);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm();
    __syncthreads();
    read_frags(na, nb, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  gload(0, s_a0, s_b0);
  wait_vm();
  __syncthreads();
  read_frags(s_a0, s_b0, 0, 0);
  for (int kt = 0; kt < KT; kt += 2) {
    ktile(kt, s_a0, s_b0, s_a1, s_b1);
    ktile(kt + 1, s_a1, s_b1, s_a0, s_b0);
  }

  // Epilogue.  Lane holds C[8 rr + 4 hl + j][ln] of each 32 x 32 block in
  // register 4 rr + j.
  const int row_base = tm * BM + wm * 128;
  if (EPI == EPI_IN) {
    const int n_qkv = 3 * g.D / BN;
    if (tn < n_qkv) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = tn * BN + wn * 128 + j * 32 + ln;
        const int which = col / g.D;
        const int cc = col - which * g.D;
        uint16_t* dst = which == 0 ? g.q : which == 1 ? g.k : g.v;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = row_base + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            if (row < g.M)
              dst[(size_t)row * g.D + cc] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][j][r]);
          }
      }
    } else {
      const int ldc = g.D + g.F;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int hidden = (tn - n_qkv) * 128 + wn * 64 + p * 32 + ln;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = row_base + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            const float mval = silu(acc[i][2 * p][r]) * acc[i][2 * p + 1][r];
            if (row < g.M)
              g.cat[(size_t)row * ldc + g.D + hidden] = __builtin_bit_cast(uint16_t, (__bf16)mval);
          }
      }
    }
  } else {
    const bool use_gate = !(g.flags & 2u), use_res = !(g.flags & 1u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = tn * BN + wn * 128 + j * 32 + ln;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row_base + i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (row < g.M) {
            const int s = stream_of(row, g.e0, g.e1);
            const float gate = use_gate ? bf2f(g.mod[(size_t)s * 3 * g.D + 2 * g.D + col]) : 1.f;
            const float res = use_res ? bf2f(g.x[(size_t)row * g.D + col]) : 0.f;
            g.y[(size_t)row * g.D + col] =
                __builtin_bit_cast(uint16_t, (__bf16)fmaf(gate, acc[i][j][r], res));
          }
        }
    }
  }
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
  const int num_m = (M + BM - 1) / BM;
  hipLaunchKernelGGL(gemm_kernel<EPI_IN>, dim3(num_m * g.num_n), dim3(256), 0, stream, g);
  return hipGetLastError();
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
  const int num_m = (M + BM - 1) / BM;
  hipLaunchKernelGGL(gemm_kernel<EPI_OUT>, dim3(num_m * g.num_n), dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace dit
