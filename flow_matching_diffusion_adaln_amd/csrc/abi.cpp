// C ABI of the DiT block library: host-side validation, workspace layouts and
// the launch sequences of the block (bf16 and FP8), the two-stage stack with
// classifier-free guidance and the flow-matching sampler.  Every check runs
// before the first launch, so an error leaves all outputs untouched.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "dit.h"
#include "kernels.h"

namespace {

// The block stores q multiplied by its softmax scale times log2 e (1 /
// sqrt(128) * log2 e), so attention's fixed-reference path can take exp2 of
// the raw scores; see launch_attn.
const float kQMul = (1.0f / sqrtf((float)DIT_HEAD_DIM)) * 1.4426950408889634f;

constexpr size_t kAlign = 256;
constexpr long long kMaxBytes = 1ll << 32;

constexpr size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool bad_float(float v, bool positive) { return !isfinite(v) || (positive ? v <= 0.f : v < 0.f); }

// Shapes derived from a validated descriptor.
struct Shape {
  int N, D, H, F, S, e0, e1;
};

int check_desc(const dit_block_desc* d, Shape* sh) {
  if (!d) return DIT_ERR_NULL;
  if (d->n_streams < 1 || d->n_streams > DIT_MAX_STREAMS) return DIT_ERR_SHAPE;
  long long n = 0;
  for (int i = 0; i < d->n_streams; ++i) {
    if (d->n_tokens[i] < 0) return DIT_ERR_SHAPE;
    n += d->n_tokens[i];
  }
  if (n > DIT_MAX_TOKENS) return DIT_ERR_SHAPE;
  if (d->n_heads <= 0 || d->head_dim <= 0 || d->width <= 0 || d->mlp_hidden <= 0)
    return DIT_ERR_SHAPE;
  if ((long long)d->n_heads * d->head_dim != d->width) return DIT_ERR_SHAPE;
  if (d->head_dim != DIT_HEAD_DIM) return DIT_ERR_UNSUPPORTED;
  // GEMM N-tiles are 256 wide and the modulation kernel works in 512-wide rows
  if (d->n_heads % 4 != 0 || d->width > 8192) return DIT_ERR_UNSUPPORTED;
  if (d->mlp_hidden % 128 != 0 || d->mlp_hidden > 65536) return DIT_ERR_UNSUPPORTED;
  // kernels address tensors with 32-bit byte offsets
  const long long width = d->width, hidden = d->mlp_hidden;
  if (n * (width + hidden) * 2 >= kMaxBytes || (3 * width + 2 * hidden) * width * 2 >= kMaxBytes)
    return DIT_ERR_UNSUPPORTED;
  if (bad_float(d->rope_theta, true) || bad_float(d->ln_eps, false) || bad_float(d->qk_eps, false))
    return DIT_ERR_ARG;
  if (d->flags & ~(DIT_F_NO_RESIDUAL | DIT_F_NO_GATE)) return DIT_ERR_ARG;
  sh->N = (int)n;
  sh->D = d->width;
  sh->H = d->n_heads;
  sh->F = d->mlp_hidden;
  sh->S = d->n_streams;
  sh->e0 = d->n_tokens[0];
  sh->e1 = sh->e0 + (d->n_streams > 1 ? d->n_tokens[1] : 0);
  if (d->n_streams == 1) sh->e0 = sh->e1 = (int)n;
  if (d->n_streams == 2) sh->e1 = (int)n;
  return DIT_OK;
}

struct Workspace {
  uint16_t *u, *q, *k, *v, *cat;
  float* partial;  // GEMM split-K partial tiles; attention's split partials
  int* attn_cnt;   // kCounters ints, zeroed by the AdaLN launch: attention's split
                   // counters, then the short-sequence output projection's
  size_t bytes;
};

// Counters in the block workspace: attention's (one per cut between two CU
// shares; more than any GPU has CUs), then one per 128 output columns of the
// short-sequence output projection.
constexpr int kAttnCounters = 512;
constexpr int kThinCounters = 512;
constexpr int kCounters = kAttnCounters + kThinCounters;

// Bytes of the block workspace for N tokens of width D and MLP hidden F (the
// sum of the regions `layout` places).
constexpr size_t block_ws_bytes(size_t N, size_t D, size_t F) {
  return 4 * round_up(N * D * 2) + round_up(N * (D + F) * 2) + round_up(dit::kGemmPartialBytes) +
         round_up(kCounters * sizeof(int));
}

Workspace layout(const Shape& s, void* base) {
  const size_t nd = (size_t)s.N * s.D * 2;
  const size_t ncat = (size_t)s.N * (s.D + s.F) * 2;
  char* p = static_cast<char*>(base);
  Workspace w;
  size_t off = 0;
  w.u = reinterpret_cast<uint16_t*>(p + off);
  off += round_up(nd);
  w.q = reinterpret_cast<uint16_t*>(p + off);
  off += round_up(nd);
  w.k = reinterpret_cast<uint16_t*>(p + off);
  off += round_up(nd);
  w.v = reinterpret_cast<uint16_t*>(p + off);
  off += round_up(nd);
  w.cat = reinterpret_cast<uint16_t*>(p + off);
  off += round_up(ncat);
  w.partial = reinterpret_cast<float*>(p + off);
  off += round_up(dit::kGemmPartialBytes);
  w.attn_cnt = reinterpret_cast<int*>(p + off);
  off += round_up(kCounters * sizeof(int));
  w.bytes = off;
  return w;
}

// The attention split of a block: the GEMM partial region is free between
// the input projection's fix-up and the output projection, and the counters
// were zeroed by the block's AdaLN launch.
dit::AttnSplit block_attn_split(const Workspace& w) {
  return dit::AttnSplit{w.partial, dit::kGemmPartialBytes, w.attn_cnt, kAttnCounters, false};
}

// ---- the block with a file-scope scratch (no allocation by the caller) -----
//
// Every GPU the library runs on holds one copy of `scratch` until the process
// ends.  In host code the array's name is only a stand-in for the device
// symbol: the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device (with that device current) and
// kept in `g_scratch`; only that pointer is ever handed to kernels.
constexpr size_t kScratchBytes =
    block_ws_bytes(DIT_NOALLOC_MAX_TOKENS, DIT_NOALLOC_WIDTH, DIT_NOALLOC_MLP_HIDDEN);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of the current device's scratch, or null with *rc set.
void* scratch_ptr(int* rc) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *rc = DIT_ERR_HIP;
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // two threads may both get here on first use; they store the same address
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      *rc = DIT_ERR_HIP;
      return nullptr;
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DIT_OK : DIT_ERR_HIP; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Null and alignment checks of the block's tensor arguments.
int check_block_ptrs(const void* x, const void* mod, const int32_t* pos, const void* w_in,
                     const void* w_out, const void* q_scale, const void* k_scale, const void* y) {
  if (!x || !mod || !pos || !w_in || !w_out || !q_scale || !k_scale || !y) return DIT_ERR_NULL;
  if (misaligned(x) || misaligned(mod) || misaligned(pos) || misaligned(w_in) ||
      misaligned(w_out) || misaligned(q_scale) || misaligned(k_scale) || misaligned(y))
    return DIT_ERR_ALIGN;
  return DIT_OK;
}

int block_fwd(const dit_block_desc* desc, const void* x, const void* mod, const int32_t* pos,
              const void* w_in, const void* w_out, const void* q_scale, const void* k_scale,
              void* y, void* workspace, size_t ws_bytes, hipStream_t stream,
              void* const* events) {
  Shape s;
  int rc = check_desc(desc, &s);
  if (rc != DIT_OK) return rc;
  if (s.N == 0) return DIT_OK;
  if ((rc = check_block_ptrs(x, mod, pos, w_in, w_out, q_scale, k_scale, y)) != DIT_OK) return rc;
  if (!workspace) return DIT_ERR_NULL;
  if (misaligned(workspace)) return DIT_ERR_ALIGN;
  Workspace w = layout(s, workspace);
  if (ws_bytes < w.bytes) return DIT_ERR_WORKSPACE;
  if (overlaps(y, (size_t)s.N * s.D * 2, workspace, w.bytes)) return DIT_ERR_ARG;
  if (events) {
    for (int i = 0; i <= DIT_N_STAGES; ++i)
      if (!events[i]) return DIT_ERR_NULL;
  }
  auto mark = [&](int i) -> int {
    if (!events) return DIT_OK;
    return hip_status(hipEventRecord(static_cast<hipEvent_t>(events[i]), stream));
  };

  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* mb = static_cast<const uint16_t*>(mod);
  if ((rc = mark(DIT_STAGE_ADALN))) return rc;
  if ((rc = hip_status(dit::launch_adaln(xb, mb, w.u, s.N, s.D, s.e0, s.e1, desc->ln_eps,
                                         stream, w.attn_cnt, kCounters))))
    return rc;
  if ((rc = mark(DIT_STAGE_GEMM_IN))) return rc;
  // the input projection applies the QK RMSNorm and RoPE in its epilogue, so
  // the rope stage is empty here (its events bracket no work)
  if ((rc = hip_status(dit::launch_gemm_in(
           w.u, static_cast<const uint16_t*>(w_in), s.N, s.D, s.F, w.q, w.k, w.v, w.cat, pos,
           static_cast<const uint16_t*>(q_scale), static_cast<const uint16_t*>(k_scale),
           desc->rope_theta, desc->qk_eps, kQMul, w.partial, stream))))
    return rc;
  if ((rc = mark(DIT_STAGE_ROPE))) return rc;
  if ((rc = mark(DIT_STAGE_ATTN))) return rc;
  const dit::AttnSplit split = block_attn_split(w);
  if ((rc = hip_status(dit::launch_attn(w.q, w.k, w.v, w.cat, s.N, s.H, s.D, s.D + s.F,
                                        1.0f / sqrtf((float)DIT_HEAD_DIM),
                                        static_cast<const uint16_t*>(q_scale),
                                        static_cast<const uint16_t*>(k_scale), 1, &split,
                                        stream))))
    return rc;
  if ((rc = mark(DIT_STAGE_GEMM_OUT))) return rc;
  if ((rc = hip_status(dit::launch_gemm_out(w.cat, static_cast<const uint16_t*>(w_out), s.N,
                                            s.D, s.F, xb, mb, static_cast<uint16_t*>(y), s.e0,
                                            s.e1, desc->flags, w.partial, stream,
                                            w.attn_cnt + kAttnCounters, kThinCounters))))
    return rc;
  return mark(DIT_N_STAGES);
}

// Workspace of the FP8 block: the bf16 block's, then the e4m3 codes and
// rowwise scales of the two projections' inputs.
struct WorkspaceF8 {
  Workspace base;
  uint8_t *u8, *cat8;
  float *u_scale, *cat_scale;
  size_t bytes;
};

WorkspaceF8 layout_fp8(const Shape& s, void* base) {
  WorkspaceF8 w;
  w.base = layout(s, base);
  char* p = static_cast<char*>(base);
  size_t off = w.base.bytes;
  w.u8 = reinterpret_cast<uint8_t*>(p + off);
  off += round_up((size_t)s.N * s.D);
  w.cat8 = reinterpret_cast<uint8_t*>(p + off);
  off += round_up((size_t)s.N * (s.D + s.F));
  w.u_scale = reinterpret_cast<float*>(p + off);
  off += round_up((size_t)s.N * 4);
  w.cat_scale = reinterpret_cast<float*>(p + off);
  off += round_up((size_t)s.N * 4);
  w.bytes = off;
  return w;
}

int block_fwd_fp8(const dit_block_desc* desc, const void* x, const void* mod, const int32_t* pos,
                  const void* w_in8, const float* w_in_scale, const void* w_out8,
                  const float* w_out_scale, const void* q_scale, const void* k_scale, void* y,
                  void* workspace, size_t ws_bytes, hipStream_t stream, void* const* events) {
  Shape s;
  int rc = check_desc(desc, &s);
  if (rc != DIT_OK) return rc;
  if (s.N == 0) return DIT_OK;
  if (!x || !mod || !pos || !w_in8 || !w_in_scale || !w_out8 || !w_out_scale || !q_scale ||
      !k_scale || !y || !workspace)
    return DIT_ERR_NULL;
  if (misaligned(x) || misaligned(mod) || misaligned(pos) || misaligned(w_in8) ||
      misaligned(w_in_scale) || misaligned(w_out8) || misaligned(w_out_scale) ||
      misaligned(q_scale) || misaligned(k_scale) || misaligned(y) || misaligned(workspace))
    return DIT_ERR_ALIGN;
  const WorkspaceF8 w = layout_fp8(s, workspace);
  if (ws_bytes < w.bytes) return DIT_ERR_WORKSPACE;
  if (overlaps(y, (size_t)s.N * s.D * 2, workspace, w.bytes)) return DIT_ERR_ARG;
  if (events) {
    for (int i = 0; i <= DIT_N_STAGES; ++i)
      if (!events[i]) return DIT_ERR_NULL;
  }
  auto mark = [&](int i) -> int {
    if (!events) return DIT_OK;
    return hip_status(hipEventRecord(static_cast<hipEvent_t>(events[i]), stream));
  };
  const Workspace& b = w.base;
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* mb = static_cast<const uint16_t*>(mod);
  if ((rc = mark(DIT_STAGE_ADALN))) return rc;
  if ((rc = hip_status(dit::launch_adaln_fp8(xb, mb, w.u8, w.u_scale, s.N, s.D, s.e0, s.e1,
                                             desc->ln_eps, stream, w.base.attn_cnt,
                                             kCounters))))
    return rc;
  if ((rc = mark(DIT_STAGE_GEMM_IN))) return rc;
  if ((rc = hip_status(dit::launch_gemm_in_fp8(
           w.u8, w.u_scale, static_cast<const uint8_t*>(w_in8), w_in_scale, s.N, s.D, s.F, b.q,
           b.k, b.v, b.cat, pos, static_cast<const uint16_t*>(q_scale),
           static_cast<const uint16_t*>(k_scale), desc->rope_theta, desc->qk_eps, kQMul,
           b.partial, stream))))
    return rc;
  if ((rc = mark(DIT_STAGE_ROPE))) return rc;
  if ((rc = mark(DIT_STAGE_ATTN))) return rc;
  const dit::AttnSplit split = block_attn_split(b);
  if ((rc = hip_status(dit::launch_attn(b.q, b.k, b.v, b.cat, s.N, s.H, s.D, s.D + s.F,
                                        1.0f / sqrtf((float)DIT_HEAD_DIM),
                                        static_cast<const uint16_t*>(q_scale),
                                        static_cast<const uint16_t*>(k_scale), 1, &split,
                                        stream))))
    return rc;
  if ((rc = mark(DIT_STAGE_GEMM_OUT))) return rc;
  // the output projection's input [o | m] is quantized rowwise first
  if ((rc = hip_status(dit::launch_quant_rows(b.cat, w.cat8, w.cat_scale, s.N, s.D + s.F,
                                              stream))) ||
      (rc = hip_status(dit::launch_gemm_out_fp8(
           w.cat8, w.cat_scale, static_cast<const uint8_t*>(w_out8), w_out_scale, s.N, s.D, s.F,
           xb, mb, static_cast<uint16_t*>(y), s.e0, s.e1, desc->flags, b.partial, stream))))
    return rc;
  return mark(DIT_N_STAGES);
}

// Block descriptor of one stage of the stack: 1 stream of n tokens, or the
// joint [image | reference | text] sequence (the reference segment only when
// there are reference tokens).
dit_block_desc stack_block_desc(const dit_stack_desc* d, int n_streams, int n0, int n1 = 0,
                                int n2 = 0) {
  dit_block_desc b{};
  b.n_streams = n_streams;
  b.n_tokens[0] = n0;
  b.n_tokens[1] = n1;
  b.n_tokens[2] = n2;
  b.width = d->width;
  b.n_heads = d->n_heads;
  b.head_dim = d->head_dim;
  b.mlp_hidden = d->mlp_hidden;
  b.rope_theta = d->rope_theta;
  b.ln_eps = d->ln_eps;
  b.qk_eps = d->qk_eps;
  b.flags = 0;
  return b;
}

dit_block_desc joint_desc(const dit_stack_desc* d) {
  return d->n_ref > 0 ? stack_block_desc(d, 3, d->n_img, d->n_ref, d->n_txt)
                      : stack_block_desc(d, 2, d->n_img, d->n_txt);
}

constexpr int kMaxStackBlocks = 1024;

// Validates the stack descriptor; on success `joint` is the joint block's
// shape and *bytes the workspace the stack needs.
int check_stack(const dit_stack_desc* d, Shape* joint, size_t* bytes) {
  if (!d) return DIT_ERR_NULL;
  if (d->n_img <= 0 || d->n_ref < 0 || d->n_txt <= 0 || d->n_img_blocks < 0 ||
      d->n_ref_blocks < 0 || d->n_txt_blocks < 0 || d->n_joint_blocks < 0)
    return DIT_ERR_SHAPE;
  if (d->n_ref == 0 && d->n_ref_blocks != 0) return DIT_ERR_SHAPE;
  if ((long long)d->n_img_blocks + d->n_ref_blocks + d->n_txt_blocks + d->n_joint_blocks >
      kMaxStackBlocks)
    return DIT_ERR_SHAPE;
  if (!isfinite(d->cfg_scale)) return DIT_ERR_ARG;
  if (d->flags & ~DIT_STACK_TEXT_SIDE_STREAM) return DIT_ERR_ARG;
  const dit_block_desc jd = joint_desc(d);
  const int rc = check_desc(&jd, joint);
  if (rc != DIT_OK) return rc;
  const size_t act = round_up((size_t)joint->N * joint->D * 2);
  *bytes = layout(*joint, nullptr).bytes + 2 * act;
  if (d->flags & DIT_STACK_TEXT_SIDE_STREAM) {
    Shape ts = *joint;
    ts.N = d->n_txt;
    *bytes += layout(ts, nullptr).bytes;
  }
  return DIT_OK;
}

// The side stream of DIT_STACK_TEXT_SIDE_STREAM and its fork / join events,
// one set per device, created on first use and kept until the process ends.
// A call holds `use` from recording the fork to enqueuing the wait on the
// join, so calls from several host threads cannot re-record the shared
// events between another call's record and wait.
struct SideStream {
  hipStream_t stream;
  hipEvent_t fork, join;
  std::mutex* use;
};
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];
bool g_side_ok[kMaxDevices];

// The current device's set, or null with *rc set.
const SideStream* side_stream(int* rc) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *rc = DIT_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_side_mu);
  if (!g_side_ok[dev]) {
    SideStream s{};
    if (hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&s.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&s.join, hipEventDisableTiming) != hipSuccess) {
      *rc = DIT_ERR_HIP;
      return nullptr;
    }
    s.use = new std::mutex();  // kept until the process ends, like the stream
    g_side[dev] = s;
    g_side_ok[dev] = true;
  }
  return &g_side[dev];
}

int check_params(const dit_block_params& p) {
  if (!p.mod || !p.w_in || !p.w_out || !p.q_scale || !p.k_scale) return DIT_ERR_NULL;
  if (misaligned(p.mod) || misaligned(p.w_in) || misaligned(p.w_out) || misaligned(p.q_scale) ||
      misaligned(p.k_scale))
    return DIT_ERR_ALIGN;
  return DIT_OK;
}


// ---- sampler ---------------------------------------------------------------

constexpr int kMaxSteps = 100000;
constexpr int kGroupImg = 0, kGroupRef = 1, kGroupTxt = 2, kGroupJoint = 3;

// Workspace of the sampler: the stack's (block workspace + one activation
// buffer per branch) first, then the rows prepared once per generation, the
// timestep path and the two branches' velocities.
struct SamplerWs {
  char* stack;                 // block workspace, then xc, xn
  size_t block_ws;             // bytes of the block workspace
  char* xc;                    // [N, D] prompt branch
  char* xn;                    // [N, D] negative branch
  uint16_t *txt_c, *txt_n;     // [n_txt, D] prepared text rows
  uint16_t* ref;               // [n_ref, D] prepared reference rows
  uint16_t* phi;               // [4, 256] timestep sinusoids
  uint16_t *th, *te;           // [2, D] timestep MLP hidden and output (rows: t, 0)
  uint16_t *mod_img, *mod_ref, *mod_txt;  // [3, D]
  uint16_t* mod_joint;         // [3, 3, D]
  uint16_t* out_mod;           // [2, D]
  uint16_t* u;                 // [n_img, D] normalized image rows
  uint16_t *v_c, *v_n;         // [n_img, C]
  size_t bytes;
};

SamplerWs sampler_layout(const dit_model_desc* d, const Shape& js, void* base) {
  const dit_stack_desc& st = d->stack;
  const size_t D = js.D, row = D * 2, C = d->latent_ch;
  char* p = static_cast<char*>(base);
  SamplerWs w;
  size_t off = 0;
  auto take = [&](size_t n) -> char* {
    char* q = p + off;
    off += round_up(n);
    return q;
  };
  w.block_ws = layout(js, nullptr).bytes;
  w.stack = take(w.block_ws);
  w.xc = take((size_t)js.N * row);
  w.xn = take((size_t)js.N * row);
  w.txt_c = reinterpret_cast<uint16_t*>(take((size_t)st.n_txt * row));
  w.txt_n = reinterpret_cast<uint16_t*>(take((size_t)st.n_txt * row));
  w.ref = reinterpret_cast<uint16_t*>(take((size_t)st.n_ref * row));
  w.phi = reinterpret_cast<uint16_t*>(take(4 * DIT_TIME_DIM * 2));
  w.th = reinterpret_cast<uint16_t*>(take(2 * row));
  w.te = reinterpret_cast<uint16_t*>(take(2 * row));
  w.mod_img = reinterpret_cast<uint16_t*>(take(3 * row));
  w.mod_ref = reinterpret_cast<uint16_t*>(take(3 * row));
  w.mod_txt = reinterpret_cast<uint16_t*>(take(3 * row));
  w.mod_joint = reinterpret_cast<uint16_t*>(take(9 * row));
  w.out_mod = reinterpret_cast<uint16_t*>(take(2 * row));
  w.u = reinterpret_cast<uint16_t*>(take((size_t)st.n_img * row));
  w.v_c = reinterpret_cast<uint16_t*>(take((size_t)st.n_img * C * 2));
  w.v_n = reinterpret_cast<uint16_t*>(take((size_t)st.n_img * C * 2));
  w.bytes = off;
  return w;
}

int check_model(const dit_model_desc* d, Shape* js, size_t* bytes) {
  if (!d) return DIT_ERR_NULL;
  size_t stack_bytes = 0;
  int rc = check_stack(&d->stack, js, &stack_bytes);
  if (rc != DIT_OK) return rc;
  if (d->stack.flags != 0) return DIT_ERR_ARG;  // text blocks run once, in prepare
  if (d->latent_ch <= 0 || d->text_dim <= 0) return DIT_ERR_SHAPE;
  if (d->latent_ch % 32 != 0 || d->latent_ch > 8192 || d->text_dim % 16 != 0 ||
      d->text_dim > (1 << 20))
    return DIT_ERR_UNSUPPORTED;
  *bytes = sampler_layout(d, *js, nullptr).bytes;
  return DIT_OK;
}

bool bad_ptr(const void* p) { return p == nullptr; }

int check_weights(const dit_model_desc* d, const dit_model_weights* w) {
  if (!w) return DIT_ERR_NULL;
  const bool refs = d->stack.n_ref > 0;
  const void* need[] = {w->img_in_w, w->img_in_b, w->txt_in_w,  w->txt_in_b,  w->t_w1,
                        w->t_b1,     w->t_w2,     w->t_b2,      w->out_mod_w, w->out_mod_b,
                        w->out_w,    w->out_b};
  for (const void* p : need)
    if (bad_ptr(p)) return DIT_ERR_NULL;
  for (int g = 0; g < DIT_N_GROUPS; ++g) {
    if (g == kGroupRef && !refs) continue;
    if (bad_ptr(w->mod_w[g]) || bad_ptr(w->mod_b[g])) return DIT_ERR_NULL;
    if (misaligned(w->mod_w[g]) || misaligned(w->mod_b[g])) return DIT_ERR_ALIGN;
  }
  if (refs && (bad_ptr(w->ref_in_w) || bad_ptr(w->ref_in_b))) return DIT_ERR_NULL;
  for (const void* p : need)
    if (misaligned(p)) return DIT_ERR_ALIGN;
  if (refs && (misaligned(w->ref_in_w) || misaligned(w->ref_in_b))) return DIT_ERR_ALIGN;
  const dit_stack_desc& st = d->stack;
  const int n_blocks = st.n_img_blocks + st.n_ref_blocks + st.n_txt_blocks + st.n_joint_blocks;
  if (n_blocks > 0 && !w->blocks) return DIT_ERR_NULL;
  for (int i = 0; i < n_blocks; ++i) {
    const dit_block_weights& b = w->blocks[i];
    if (!b.w_in || !b.w_out || !b.q_scale || !b.k_scale) return DIT_ERR_NULL;
    if (misaligned(b.w_in) || misaligned(b.w_out) || misaligned(b.q_scale) ||
        misaligned(b.k_scale))
      return DIT_ERR_ALIGN;
  }
  return DIT_OK;
}

int lin(const void* x, const void* w, const void* b, void* y, int M, int N, int K, int ldy,
        int act, hipStream_t stream) {
  return hip_status(dit::launch_linear(static_cast<const uint16_t*>(x),
                                       static_cast<const uint16_t*>(w),
                                       static_cast<const uint16_t*>(b), static_cast<uint16_t*>(y),
                                       M, N, K, K, ldy, act, stream));
}

// e (rows: the given timesteps) = SiLU(W2 SiLU(W1 phi(t) + b1) + b2) into ws.te
int time_embedding(const dit_model_weights* w, const SamplerWs& ws, const double* t, int n_t,
                   int D, hipStream_t stream) {
  int rc = hip_status(dit::launch_sinusoid(t, n_t, DIT_TIME_DIM, 1000.0, 10000.0, ws.phi, stream));
  if (rc == DIT_OK) rc = lin(ws.phi, w->t_w1, w->t_b1, ws.th, n_t, D, DIT_TIME_DIM, D, 1, stream);
  if (rc == DIT_OK) rc = lin(ws.th, w->t_w2, w->t_b2, ws.te, n_t, D, D, D, 1, stream);
  return rc;
}

// Runs blocks [first, first + n) of the model on rows h with one modulation.
int run_blocks(const dit_model_weights* w, const SamplerWs& ws, const dit_block_desc& d,
               int first, int n, const uint16_t* mod, char* h, const int32_t* pos,
               hipStream_t stream) {
  for (int i = 0; i < n; ++i) {
    const dit_block_weights& b = w->blocks[first + i];
    const int rc = block_fwd(&d, h, mod, pos, b.w_in, b.w_out, b.q_scale, b.k_scale, h, ws.stack,
                             ws.block_ws, stream, nullptr);
    if (rc != DIT_OK) return rc;
  }
  return DIT_OK;
}

int dcopy(void* dst, const void* src, size_t n, hipStream_t stream) {
  return hip_status(hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, stream));
}

// ---- attention on its own -----------------------------------------------

int check_attn(int32_t n_tokens, int32_t n_heads, int32_t head_dim, float softmax_scale) {
  if (n_tokens < 0 || n_tokens > DIT_MAX_TOKENS || n_heads <= 0 || head_dim <= 0)
    return DIT_ERR_SHAPE;
  if (head_dim != DIT_HEAD_DIM) return DIT_ERR_UNSUPPORTED;
  if ((long long)n_heads * head_dim > 65536) return DIT_ERR_UNSUPPORTED;
  if ((long long)n_tokens * n_heads * head_dim * 2 >= kMaxBytes) return DIT_ERR_UNSUPPORTED;
  if (bad_float(softmax_scale, true)) return DIT_ERR_ARG;
  return DIT_OK;
}

// Workspace of dit_attn_fwd_ws: the split partials for up to kAttnMaxShares
// shares (one per CU), then their counters.
constexpr int kAttnMaxShares = 256;
const size_t kAttnPartBytes = dit::attn_split_bytes(kAttnMaxShares);
const size_t kAttnWsBytes = round_up(kAttnPartBytes) + round_up(kAttnMaxShares * sizeof(int));

int attn_fwd(int32_t n_tokens, int32_t n_heads, int32_t head_dim, const void* q, const void* k,
             const void* v, void* o, float softmax_scale, void* workspace, size_t ws_bytes,
             bool use_ws, hipStream_t stream) {
  int rc = check_attn(n_tokens, n_heads, head_dim, softmax_scale);
  if (rc != DIT_OK) return rc;
  if (n_tokens == 0) return DIT_OK;
  if (!q || !k || !v || !o || (use_ws && !workspace)) return DIT_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) ||
      (use_ws && misaligned(workspace)))
    return DIT_ERR_ALIGN;
  if (use_ws && ws_bytes < kAttnWsBytes) return DIT_ERR_WORKSPACE;
  const size_t bytes = (size_t)n_tokens * n_heads * head_dim * 2;
  if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, k, bytes) || overlaps(o, bytes, v, bytes))
    return DIT_ERR_ARG;
  if (use_ws && (overlaps(workspace, kAttnWsBytes, o, bytes) ||
                 overlaps(workspace, kAttnWsBytes, q, bytes) ||
                 overlaps(workspace, kAttnWsBytes, k, bytes) ||
                 overlaps(workspace, kAttnWsBytes, v, bytes)))
    return DIT_ERR_ARG;
  const int ld = n_heads * head_dim;
  char* wsp = static_cast<char*>(workspace);
  const dit::AttnSplit split{wsp, kAttnPartBytes,
                             reinterpret_cast<int*>(wsp + round_up(kAttnPartBytes)),
                             kAttnMaxShares, true};
  return hip_status(dit::launch_attn(static_cast<const uint16_t*>(q),
                                     static_cast<const uint16_t*>(k),
                                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o),
                                     n_tokens, n_heads, ld, ld, softmax_scale, nullptr, nullptr,
                                     0, use_ws ? &split : nullptr, stream));
}

}  // namespace

extern "C" {

int dit_block_workspace_bytes(const dit_block_desc* desc, size_t* bytes) {
  Shape s;
  const int rc = check_desc(desc, &s);
  if (rc != DIT_OK) return rc;
  if (!bytes) return DIT_ERR_NULL;
  *bytes = layout(s, nullptr).bytes;
  return DIT_OK;
}

int dit_block_fwd(const dit_block_desc* desc, const void* x, const void* mod, const int32_t* pos,
                  const void* w_in, const void* w_out, const void* q_scale, const void* k_scale,
                  void* y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return block_fwd(desc, x, mod, pos, w_in, w_out, q_scale, k_scale, y, workspace,
                   workspace_bytes, stream, nullptr);
}

int dit_block_fwd_events(const dit_block_desc* desc, const void* x, const void* mod,
                         const int32_t* pos, const void* w_in, const void* w_out,
                         const void* q_scale, const void* k_scale, void* y, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, void* const* events) {
  if (!events) return DIT_ERR_NULL;
  return block_fwd(desc, x, mod, pos, w_in, w_out, q_scale, k_scale, y, workspace,
                   workspace_bytes, stream, events);
}

int dit_block_fwd_noalloc(const dit_block_desc* desc, const void* x, const void* mod,
                          const int32_t* pos, const void* w_in, const void* w_out,
                          const void* q_scale, const void* k_scale, void* y, hipStream_t stream) {
  Shape s;
  int rc = check_desc(desc, &s);
  if (rc != DIT_OK) return rc;
  if (s.N == 0) return DIT_OK;
  // sizes beyond the scratch, and bad pointers, are refused before anything
  // touches the device
  if (layout(s, nullptr).bytes > kScratchBytes) return DIT_ERR_WORKSPACE;
  if ((rc = check_block_ptrs(x, mod, pos, w_in, w_out, q_scale, k_scale, y)) != DIT_OK) return rc;
  void* ws = scratch_ptr(&rc);
  if (!ws) return rc;
  return block_fwd(desc, x, mod, pos, w_in, w_out, q_scale, k_scale, y, ws, kScratchBytes, stream,
                   nullptr);
}

int dit_block_noalloc_scratch_bytes(size_t* bytes) {
  if (!bytes) return DIT_ERR_NULL;
  *bytes = kScratchBytes;
  return DIT_OK;
}

int dit_attn_fwd(int32_t n_tokens, int32_t n_heads, int32_t head_dim, const void* q,
                 const void* k, const void* v, void* o, float softmax_scale, hipStream_t stream) {
  return attn_fwd(n_tokens, n_heads, head_dim, q, k, v, o, softmax_scale, nullptr, 0, false,
                  stream);
}

int dit_attn_workspace_bytes(int32_t n_tokens, int32_t n_heads, int32_t head_dim,
                             size_t* bytes) {
  const int rc = check_attn(n_tokens, n_heads, head_dim, 1.0f);
  if (rc != DIT_OK) return rc;
  if (!bytes) return DIT_ERR_NULL;
  *bytes = kAttnWsBytes;
  return DIT_OK;
}

int dit_attn_fwd_ws(int32_t n_tokens, int32_t n_heads, int32_t head_dim, const void* q,
                    const void* k, const void* v, void* o, float softmax_scale, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  return attn_fwd(n_tokens, n_heads, head_dim, q, k, v, o, softmax_scale, workspace,
                  workspace_bytes, true, stream);
}

int rope4_apply(int32_t n_tokens, int32_t n_heads, int32_t head_dim, void* q, void* k,
                const int32_t* pos, float theta, const void* q_scale, const void* k_scale,
                float qk_eps, hipStream_t stream) {
  if (n_tokens < 0 || n_tokens > DIT_MAX_TOKENS || n_heads <= 0 || head_dim <= 0)
    return DIT_ERR_SHAPE;
  if (head_dim != DIT_HEAD_DIM) return DIT_ERR_UNSUPPORTED;
  if ((long long)n_heads * head_dim > 65536) return DIT_ERR_UNSUPPORTED;
  if (bad_float(theta, true) || bad_float(qk_eps, false)) return DIT_ERR_ARG;
  if ((q_scale == nullptr) != (k_scale == nullptr)) return DIT_ERR_ARG;
  if (n_tokens == 0) return DIT_OK;
  if (!q || !k || !pos) return DIT_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(pos) || misaligned(q_scale) ||
      misaligned(k_scale))
    return DIT_ERR_ALIGN;
  return hip_status(dit::launch_rope4(static_cast<uint16_t*>(q), static_cast<uint16_t*>(k), pos,
                                      static_cast<const uint16_t*>(q_scale),
                                      static_cast<const uint16_t*>(k_scale), n_tokens, n_heads,
                                      theta, qk_eps, 1.0f, stream));
}

int adaln_mod(int32_t n_streams, const int32_t* n_tokens, int32_t width, const void* x,
              const void* mod, void* out, float eps, hipStream_t stream) {
  if (n_streams < 1 || n_streams > DIT_MAX_STREAMS) return DIT_ERR_SHAPE;
  if (!n_tokens) return DIT_ERR_NULL;
  long long n = 0;
  for (int i = 0; i < n_streams; ++i) {
    if (n_tokens[i] < 0) return DIT_ERR_SHAPE;
    n += n_tokens[i];
  }
  if (n > DIT_MAX_TOKENS || width <= 0) return DIT_ERR_SHAPE;
  if (width % 512 != 0 || width > 8192) return DIT_ERR_UNSUPPORTED;
  if (bad_float(eps, false)) return DIT_ERR_ARG;
  if (n == 0) return DIT_OK;
  if (!x || !mod || !out) return DIT_ERR_NULL;
  if (misaligned(x) || misaligned(mod) || misaligned(out)) return DIT_ERR_ALIGN;
  int e0 = n_tokens[0];
  int e1 = e0 + (n_streams > 1 ? n_tokens[1] : 0);
  if (n_streams == 1) e0 = e1 = (int)n;
  if (n_streams == 2) e1 = (int)n;
  return hip_status(dit::launch_adaln(static_cast<const uint16_t*>(x),
                                      static_cast<const uint16_t*>(mod),
                                      static_cast<uint16_t*>(out), (int)n, width, e0, e1, eps,
                                      stream));
}

int dit_stack_workspace_bytes(const dit_stack_desc* desc, size_t* bytes) {
  Shape js;
  size_t need = 0;
  const int rc = check_stack(desc, &js, &need);
  if (rc != DIT_OK) return rc;
  if (!bytes) return DIT_ERR_NULL;
  *bytes = need;
  return DIT_OK;
}

int dit_stack_fwd(const dit_stack_desc* desc, const void* x_img, const void* x_ref,
                  const void* x_txt_cond, const void* x_txt_neg, const int32_t* pos,
                  const dit_block_params* blocks, void* v_img, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  Shape js;
  size_t need = 0;
  int rc = check_stack(desc, &js, &need);
  if (rc != DIT_OK) return rc;
  const bool guided = desc->cfg_scale != 1.0f;
  const bool refs = desc->n_ref > 0;
  const int n_blocks =
      desc->n_img_blocks + desc->n_ref_blocks + desc->n_txt_blocks + desc->n_joint_blocks;
  if (!x_img || (refs && !x_ref) || !x_txt_cond || (guided && !x_txt_neg) || !pos || !v_img ||
      !workspace || (n_blocks > 0 && !blocks))
    return DIT_ERR_NULL;
  if (misaligned(x_img) || (refs && misaligned(x_ref)) || misaligned(x_txt_cond) ||
      (guided && misaligned(x_txt_neg)) || misaligned(pos) || misaligned(v_img) ||
      misaligned(workspace))
    return DIT_ERR_ALIGN;
  // every block is checked before anything is launched
  for (int i = 0; i < n_blocks; ++i)
    if ((rc = check_params(blocks[i])) != DIT_OK) return rc;
  if (workspace_bytes < need) return DIT_ERR_WORKSPACE;
  const size_t row = (size_t)js.D * 2;  // bytes per token row
  const size_t img_bytes = (size_t)desc->n_img * row, ref_bytes = (size_t)desc->n_ref * row,
               txt_bytes = (size_t)desc->n_txt * row;
  const size_t pre_bytes = img_bytes + ref_bytes;  // the rows both branches share
  if (overlaps(v_img, img_bytes, workspace, need)) return DIT_ERR_ARG;

  char* wsp = static_cast<char*>(workspace);
  const size_t block_ws = layout(js, nullptr).bytes;
  const size_t act = round_up((size_t)js.N * row);
  char* xc = wsp + block_ws;        // [N, D] activations of the prompt branch
  char* xn = xc + act;              // [N, D] activations of the negative branch
  const dit_block_desc di = stack_block_desc(desc, 1, desc->n_img);
  const dit_block_desc dr = stack_block_desc(desc, 1, desc->n_ref);
  const dit_block_desc dt = stack_block_desc(desc, 1, desc->n_txt);
  const dit_block_desc dj = joint_desc(desc);
  const int32_t* pos_ref = pos + (size_t)desc->n_img * 4;
  const int32_t* pos_txt = pos_ref + (size_t)desc->n_ref * 4;
  const dit_block_params* bi = blocks;
  const dit_block_params* br = bi + desc->n_img_blocks;
  const dit_block_params* bt = br + desc->n_ref_blocks;
  const dit_block_params* bj = bt + desc->n_txt_blocks;
  auto run_on = [&](const dit_block_desc& d, const dit_block_params& p, char* h,
                    const int32_t* ps, char* ws, size_t ws_bytes, hipStream_t st) -> int {
    return block_fwd(&d, h, p.mod, ps, p.w_in, p.w_out, p.q_scale, p.k_scale, h, ws, ws_bytes, st,
                     nullptr);
  };
  auto run = [&](const dit_block_desc& d, const dit_block_params& p, char* h,
                 const int32_t* ps) -> int {
    return run_on(d, p, h, ps, wsp, block_ws, stream);
  };
  auto copy = [&](void* dst, const void* src, size_t n) -> int {
    return hip_status(hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, stream));
  };
  auto joint = [&](char* h) -> int {
    for (int i = 0; i < desc->n_joint_blocks; ++i)
      if ((rc = run(dj, bj[i], h, pos)) != DIT_OK) return rc;
    return DIT_OK;
  };
  auto finish = [&]() -> int {
    if ((rc = joint(xc)) != DIT_OK) return rc;
    if (!guided) return copy(v_img, xc, img_bytes);
    if ((rc = joint(xn)) != DIT_OK) return rc;
    return hip_status(dit::launch_cfg_combine(reinterpret_cast<const uint16_t*>(xc),
                                              reinterpret_cast<const uint16_t*>(xn),
                                              static_cast<uint16_t*>(v_img),
                                              (long long)desc->n_img * js.D, desc->cfg_scale,
                                              stream));
  };
  // stage 1, image and reference: shared by both branches
  auto stage1_shared = [&]() -> int {
    if ((rc = copy(xc, x_img, img_bytes)) != DIT_OK) return rc;
    for (int i = 0; i < desc->n_img_blocks; ++i)
      if ((rc = run(di, bi[i], xc, pos)) != DIT_OK) return rc;
    if (refs) {
      if ((rc = copy(xc + img_bytes, x_ref, ref_bytes)) != DIT_OK) return rc;
      for (int i = 0; i < desc->n_ref_blocks; ++i)
        if ((rc = run(dr, br[i], xc + img_bytes, pos_ref)) != DIT_OK) return rc;
    }
    if (guided && (rc = copy(xn, xc, pre_bytes)) != DIT_OK) return rc;
    return DIT_OK;
  };

  if (desc->flags & DIT_STACK_TEXT_SIDE_STREAM) {
    // The text rows of each branch are filled and the fork recorded on the
    // caller's stream; the side stream runs both branches' text blocks (in
    // place on the text rows, with a block workspace of its own) while the
    // caller's stream runs the image and reference blocks on the other rows;
    // the joint blocks wait for the join.
    const SideStream* side = side_stream(&rc);
    if (!side) return rc;
    std::lock_guard<std::mutex> lock(*side->use);
    Shape ts = js;
    ts.N = desc->n_txt;
    char* wst = xn + act;
    const size_t wst_bytes = layout(ts, nullptr).bytes;
    if ((rc = copy(xc + pre_bytes, x_txt_cond, txt_bytes)) != DIT_OK) return rc;
    if (guided && (rc = copy(xn + pre_bytes, x_txt_neg, txt_bytes)) != DIT_OK) return rc;
    if ((rc = hip_status(hipEventRecord(side->fork, stream))) != DIT_OK ||
        (rc = hip_status(hipStreamWaitEvent(side->stream, side->fork, 0))) != DIT_OK)
      return rc;
    for (int b = 0; b < (guided ? 2 : 1); ++b) {
      char* h = (b ? xn : xc) + pre_bytes;
      for (int i = 0; i < desc->n_txt_blocks; ++i)
        if ((rc = run_on(dt, bt[i], h, pos_txt, wst, wst_bytes, side->stream)) != DIT_OK)
          return rc;
    }
    if ((rc = hip_status(hipEventRecord(side->join, side->stream))) != DIT_OK) return rc;
    if ((rc = stage1_shared()) != DIT_OK) return rc;
    if ((rc = hip_status(hipStreamWaitEvent(stream, side->join, 0))) != DIT_OK) return rc;
    return finish();
  }

  if ((rc = stage1_shared()) != DIT_OK) return rc;
  // stage 1, text, per branch (in place on the text rows of [image |
  // reference | text])
  for (int b = 0; b < (guided ? 2 : 1); ++b) {
    char* h = b ? xn : xc;
    if ((rc = copy(h + pre_bytes, b ? x_txt_neg : x_txt_cond, txt_bytes)) != DIT_OK) return rc;
    for (int i = 0; i < desc->n_txt_blocks; ++i)
      if ((rc = run(dt, bt[i], h + pre_bytes, pos_txt)) != DIT_OK) return rc;
  }
  return finish();
}

int dit_flow_sigmas(int32_t n_steps, double alpha, double* sigmas) {
  if (n_steps < 1 || n_steps > kMaxSteps) return DIT_ERR_SHAPE;
  if (!isfinite(alpha) || alpha <= 0.0) return DIT_ERR_ARG;
  if (!sigmas) return DIT_ERR_NULL;
  for (int i = 0; i <= n_steps; ++i) {
    const double u = 1.0 - (double)i / n_steps;
    sigmas[i] = alpha * u / (1.0 + (alpha - 1.0) * u);
  }
  return DIT_OK;
}

int dit_sampler_workspace_bytes(const dit_model_desc* desc, size_t* bytes) {
  Shape js;
  size_t need = 0;
  const int rc = check_model(desc, &js, &need);
  if (rc != DIT_OK) return rc;
  if (!bytes) return DIT_ERR_NULL;
  *bytes = need;
  return DIT_OK;
}

int dit_sampler_prepare(const dit_model_desc* desc, const dit_model_weights* weights,
                        const void* txt_cond, const void* txt_neg, const void* ref_latent,
                        const int32_t* pos, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  Shape js;
  size_t need = 0;
  int rc = check_model(desc, &js, &need);
  if (rc != DIT_OK) return rc;
  if ((rc = check_weights(desc, weights)) != DIT_OK) return rc;
  const dit_stack_desc& st = desc->stack;
  const bool guided = st.cfg_scale != 1.0f, refs = st.n_ref > 0;
  if (!txt_cond || (guided && !txt_neg) || (refs && !ref_latent) || !pos || !workspace)
    return DIT_ERR_NULL;
  if (misaligned(txt_cond) || (guided && misaligned(txt_neg)) ||
      (refs && misaligned(ref_latent)) || misaligned(pos) || misaligned(workspace))
    return DIT_ERR_ALIGN;
  if (workspace_bytes < need) return DIT_ERR_WORKSPACE;
  const SamplerWs ws = sampler_layout(desc, js, workspace);
  const int D = js.D;
  const double t0 = 0.0;
  if ((rc = time_embedding(weights, ws, &t0, 1, D, stream)) != DIT_OK) return rc;
  // references: embedded and run through their blocks at t = 0
  const int32_t* pos_ref = pos + (size_t)st.n_img * 4;
  const int32_t* pos_txt = pos_ref + (size_t)st.n_ref * 4;
  if (refs) {
    const dit_block_desc dr = stack_block_desc(&st, 1, st.n_ref);
    if ((rc = lin(ws.te, weights->mod_w[kGroupRef], weights->mod_b[kGroupRef], ws.mod_ref, 1,
                  3 * D, D, 3 * D, 0, stream)) != DIT_OK ||
        (rc = lin(ref_latent, weights->ref_in_w, weights->ref_in_b, ws.ref, st.n_ref, D,
                  desc->latent_ch, D, 0, stream)) != DIT_OK ||
        (rc = run_blocks(weights, ws, dr, st.n_img_blocks, st.n_ref_blocks, ws.mod_ref,
                         reinterpret_cast<char*>(ws.ref), pos_ref, stream)) != DIT_OK)
      return rc;
  }
  // text of each prompt: embedded and run through the text blocks at t = 0
  const dit_block_desc dt = stack_block_desc(&st, 1, st.n_txt);
  if ((rc = lin(ws.te, weights->mod_w[kGroupTxt], weights->mod_b[kGroupTxt], ws.mod_txt, 1,
                3 * D, D, 3 * D, 0, stream)) != DIT_OK)
    return rc;
  const int first_txt = st.n_img_blocks + st.n_ref_blocks;
  const void* feats[2] = {txt_cond, txt_neg};
  uint16_t* rows[2] = {ws.txt_c, ws.txt_n};
  for (int b = 0; b < (guided ? 2 : 1); ++b) {
    if ((rc = lin(feats[b], weights->txt_in_w, weights->txt_in_b, rows[b], st.n_txt, D,
                  desc->text_dim, D, 0, stream)) != DIT_OK ||
        (rc = run_blocks(weights, ws, dt, first_txt, st.n_txt_blocks, ws.mod_txt,
                         reinterpret_cast<char*>(rows[b]), pos_txt, stream)) != DIT_OK)
      return rc;
  }
  return DIT_OK;
}

int dit_sampler_step(const dit_model_desc* desc, const dit_model_weights* weights, void* z,
                     double sigma, double sigma_next, const int32_t* pos, void* v_out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Shape js;
  size_t need = 0;
  int rc = check_model(desc, &js, &need);
  if (rc != DIT_OK) return rc;
  if ((rc = check_weights(desc, weights)) != DIT_OK) return rc;
  if (!isfinite(sigma) || !isfinite(sigma_next)) return DIT_ERR_ARG;
  if (!z || !pos || !workspace) return DIT_ERR_NULL;
  if (misaligned(z) || misaligned(pos) || misaligned(workspace) || (v_out && misaligned(v_out)))
    return DIT_ERR_ALIGN;
  if (workspace_bytes < need) return DIT_ERR_WORKSPACE;
  const dit_stack_desc& st = desc->stack;
  const bool guided = st.cfg_scale != 1.0f, refs = st.n_ref > 0;
  const int D = js.D, C = desc->latent_ch;
  const size_t zb = (size_t)st.n_img * C * 2;
  if (overlaps(z, zb, workspace, need) || (v_out && overlaps(v_out, zb, workspace, need)) ||
      (v_out && overlaps(v_out, zb, z, zb)))
    return DIT_ERR_ARG;
  const SamplerWs ws = sampler_layout(desc, js, workspace);
  const size_t row = (size_t)D * 2;
  const size_t img_bytes = (size_t)st.n_img * row, pre_bytes = img_bytes + (size_t)st.n_ref * row;
  const size_t txt_bytes = (size_t)st.n_txt * row;

  // timestep path: row 0 at sigma (image tokens), row 1 at t = 0 (the others)
  const double ts[2] = {sigma, 0.0};
  if ((rc = time_embedding(weights, ws, ts, 2, D, stream)) != DIT_OK) return rc;
  if ((rc = lin(ws.te, weights->mod_w[kGroupImg], weights->mod_b[kGroupImg], ws.mod_img, 1,
                3 * D, D, 3 * D, 0, stream)) != DIT_OK ||
      (rc = lin(ws.te, weights->mod_w[kGroupJoint], weights->mod_b[kGroupJoint], ws.mod_joint, 2,
                3 * D, D, 3 * D, 0, stream)) != DIT_OK ||
      (rc = lin(ws.te, weights->out_mod_w, weights->out_mod_b, ws.out_mod, 1, 2 * D, D, 2 * D, 0,
                stream)) != DIT_OK)
    return rc;
  // joint modulation per stream: image at sigma, reference and text at 0
  if (refs && (rc = dcopy(ws.mod_joint + 6 * (size_t)D, ws.mod_joint + 3 * (size_t)D, 3 * row,
                          stream)) != DIT_OK)
    return rc;

  // image tokens: embedded, then the stage-1 image blocks (shared by both branches)
  const dit_block_desc di = stack_block_desc(&st, 1, st.n_img);
  if ((rc = lin(z, weights->img_in_w, weights->img_in_b, ws.xc, st.n_img, D, C, D, 0,
                stream)) != DIT_OK ||
      (rc = run_blocks(weights, ws, di, 0, st.n_img_blocks, ws.mod_img, ws.xc, pos, stream)) !=
          DIT_OK)
    return rc;
  if (refs && (rc = dcopy(ws.xc + img_bytes, ws.ref, pre_bytes - img_bytes, stream)) != DIT_OK)
    return rc;
  if ((rc = dcopy(ws.xc + pre_bytes, ws.txt_c, txt_bytes, stream)) != DIT_OK) return rc;
  if (guided && ((rc = dcopy(ws.xn, ws.xc, pre_bytes, stream)) != DIT_OK ||
                 (rc = dcopy(ws.xn + pre_bytes, ws.txt_n, txt_bytes, stream)) != DIT_OK))
    return rc;

  // joint blocks and output layers per branch
  const dit_block_desc dj = joint_desc(&st);
  const int first_joint = st.n_img_blocks + st.n_ref_blocks + st.n_txt_blocks;
  char* hs[2] = {ws.xc, ws.xn};
  uint16_t* vs[2] = {ws.v_c, ws.v_n};
  for (int b = 0; b < (guided ? 2 : 1); ++b) {
    if ((rc = run_blocks(weights, ws, dj, first_joint, st.n_joint_blocks, ws.mod_joint, hs[b],
                         pos, stream)) != DIT_OK ||
        (rc = hip_status(dit::launch_adaln(reinterpret_cast<const uint16_t*>(hs[b]), ws.out_mod,
                                           ws.u, st.n_img, D, st.n_img, st.n_img, st.ln_eps,
                                           stream))) != DIT_OK ||
        (rc = lin(ws.u, weights->out_w, weights->out_b, vs[b], st.n_img, C, D, C, 0, stream)) !=
            DIT_OK)
      return rc;
  }
  // guided velocity and the Euler update of the latent
  return hip_status(dit::launch_euler_cfg(static_cast<uint16_t*>(z), ws.v_c,
                                          guided ? ws.v_n : nullptr,
                                          static_cast<uint16_t*>(v_out), (long long)st.n_img * C,
                                          st.cfg_scale, (float)(sigma_next - sigma), stream));
}

int dit_linear(int32_t M, int32_t N, int32_t K, const void* x, const void* w, const void* b,
               int32_t act, void* y, hipStream_t stream) {
  if (M < 0 || N <= 0 || K <= 0) return DIT_ERR_SHAPE;
  if (N % 32 != 0 || K % 16 != 0) return DIT_ERR_UNSUPPORTED;
  if ((long long)M * K * 2 >= kMaxBytes * 4 || (long long)N * K * 2 >= kMaxBytes)
    return DIT_ERR_UNSUPPORTED;
  if (act != 0 && act != 1) return DIT_ERR_ARG;
  if (M == 0) return DIT_OK;
  if (!x || !w || !y) return DIT_ERR_NULL;
  if (misaligned(x) || misaligned(w) || (b && misaligned(b)) || misaligned(y))
    return DIT_ERR_ALIGN;
  const size_t yb = (size_t)M * N * 2;
  if (overlaps(y, yb, x, (size_t)M * K * 2) || overlaps(y, yb, w, (size_t)N * K * 2) ||
      (b && overlaps(y, yb, b, (size_t)N * 2)))
    return DIT_ERR_ARG;
  return lin(x, w, b, y, M, N, K, N, act, stream);
}

int dit_time_sinusoid(int32_t n_t, const double* t, void* out, hipStream_t stream) {
  if (n_t < 1 || n_t > 4) return DIT_ERR_SHAPE;
  if (!t || !out) return DIT_ERR_NULL;
  if (misaligned(out)) return DIT_ERR_ALIGN;
  for (int i = 0; i < n_t; ++i)
    if (!isfinite(t[i])) return DIT_ERR_ARG;
  return hip_status(dit::launch_sinusoid(t, n_t, DIT_TIME_DIM, 1000.0, 10000.0,
                                         static_cast<uint16_t*>(out), stream));
}

int dit_quantize_rows_fp8(int32_t M, int32_t K, const void* x, void* q, float* scale,
                          hipStream_t stream) {
  if (M < 0 || K <= 0) return DIT_ERR_SHAPE;
  if (K % 8 != 0) return DIT_ERR_UNSUPPORTED;
  if ((long long)M * K * 2 >= kMaxBytes * 4) return DIT_ERR_UNSUPPORTED;
  if (M == 0) return DIT_OK;
  if (!x || !q || !scale) return DIT_ERR_NULL;
  if (misaligned(x) || misaligned(q) || misaligned(scale)) return DIT_ERR_ALIGN;
  const size_t xb = (size_t)M * K * 2, qb = (size_t)M * K, sb = (size_t)M * 4;
  if (overlaps(q, qb, x, xb) || overlaps(scale, sb, x, xb) || overlaps(scale, sb, q, qb))
    return DIT_ERR_ARG;
  return hip_status(dit::launch_quant_rows(static_cast<const uint16_t*>(x),
                                           static_cast<uint8_t*>(q), scale, M, K, stream));
}

int dit_block_fp8_workspace_bytes(const dit_block_desc* desc, size_t* bytes) {
  Shape s;
  const int rc = check_desc(desc, &s);
  if (rc != DIT_OK) return rc;
  if (!bytes) return DIT_ERR_NULL;
  *bytes = layout_fp8(s, nullptr).bytes;
  return DIT_OK;
}

int dit_block_fwd_fp8(const dit_block_desc* desc, const void* x, const void* mod,
                      const int32_t* pos, const void* w_in8, const float* w_in_scale,
                      const void* w_out8, const float* w_out_scale, const void* q_scale,
                      const void* k_scale, void* y, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  return block_fwd_fp8(desc, x, mod, pos, w_in8, w_in_scale, w_out8, w_out_scale, q_scale,
                       k_scale, y, workspace, workspace_bytes, stream, nullptr);
}

int dit_block_fwd_fp8_events(const dit_block_desc* desc, const void* x, const void* mod,
                             const int32_t* pos, const void* w_in8, const float* w_in_scale,
                             const void* w_out8, const float* w_out_scale, const void* q_scale,
                             const void* k_scale, void* y, void* workspace,
                             size_t workspace_bytes, hipStream_t stream, void* const* events) {
  if (!events) return DIT_ERR_NULL;
  return block_fwd_fp8(desc, x, mod, pos, w_in8, w_in_scale, w_out8, w_out_scale, q_scale,
                       k_scale, y, workspace, workspace_bytes, stream, events);
}

const char* dit_status_str(int status) {
  switch (status) {
    case DIT_OK: return "DIT_OK";
    case DIT_ERR_NULL: return "DIT_ERR_NULL: a required pointer is null";
    case DIT_ERR_SHAPE: return "DIT_ERR_SHAPE: inconsistent or out-of-range sizes";
    case DIT_ERR_UNSUPPORTED: return "DIT_ERR_UNSUPPORTED: size this library does not implement";
    case DIT_ERR_ALIGN: return "DIT_ERR_ALIGN: pointer not 16-byte aligned";
    case DIT_ERR_WORKSPACE: return "DIT_ERR_WORKSPACE: workspace missing or too small";
    case DIT_ERR_HIP: return "DIT_ERR_HIP: the HIP runtime reported an error";
    case DIT_ERR_ARG: return "DIT_ERR_ARG: scalar argument out of range or buffers overlap";
    default: return "DIT_ERR_UNKNOWN";
  }
}

}  // extern "C"
