// C ABI of the DiT block library: host-side validation, workspace layout and
// the launch sequence of dit_block_fwd.  Every check runs before the first
// launch, so an error leaves all outputs untouched.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "dit.h"
#include "kernels.h"

namespace {

constexpr size_t kAlign = 256;
constexpr long long kMaxBytes = 1ll << 32;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

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
  float* partial;  // GEMM split-K partial tiles
  size_t bytes;
};

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
  w.bytes = off;
  return w;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DIT_OK : DIT_ERR_HIP; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int block_fwd(const dit_block_desc* desc, const void* x, const void* mod, const int32_t* pos,
              const void* w_in, const void* w_out, const void* q_scale, const void* k_scale,
              void* y, void* workspace, size_t ws_bytes, hipStream_t stream,
              void* const* events) {
  Shape s;
  int rc = check_desc(desc, &s);
  if (rc != DIT_OK) return rc;
  if (s.N == 0) return DIT_OK;
  if (!x || !mod || !pos || !w_in || !w_out || !q_scale || !k_scale || !y || !workspace)
    return DIT_ERR_NULL;
  if (misaligned(x) || misaligned(mod) || misaligned(pos) || misaligned(w_in) ||
      misaligned(w_out) || misaligned(q_scale) || misaligned(k_scale) || misaligned(y) ||
      misaligned(workspace))
    return DIT_ERR_ALIGN;
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
                                         stream))))
    return rc;
  if ((rc = mark(DIT_STAGE_GEMM_IN))) return rc;
  // the input projection applies the QK RMSNorm and RoPE in its epilogue, so
  // the rope stage is empty here (its events bracket no work)
  if ((rc = hip_status(dit::launch_gemm_in(
           w.u, static_cast<const uint16_t*>(w_in), s.N, s.D, s.F, w.q, w.k, w.v, w.cat, pos,
           static_cast<const uint16_t*>(q_scale), static_cast<const uint16_t*>(k_scale),
           desc->rope_theta, desc->qk_eps, w.partial, stream))))
    return rc;
  if ((rc = mark(DIT_STAGE_ROPE))) return rc;
  if ((rc = mark(DIT_STAGE_ATTN))) return rc;
  if ((rc = hip_status(dit::launch_attn(w.q, w.k, w.v, w.cat, s.N, s.H, s.D, s.D + s.F,
                                        1.0f / sqrtf((float)DIT_HEAD_DIM), stream))))
    return rc;
  if ((rc = mark(DIT_STAGE_GEMM_OUT))) return rc;
  if ((rc = hip_status(dit::launch_gemm_out(w.cat, static_cast<const uint16_t*>(w_out), s.N,
                                            s.D, s.F, xb, mb, static_cast<uint16_t*>(y), s.e0,
                                            s.e1, desc->flags, w.partial, stream))))
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
  const dit_block_desc jd = joint_desc(d);
  const int rc = check_desc(&jd, joint);
  if (rc != DIT_OK) return rc;
  const size_t act = round_up((size_t)joint->N * joint->D * 2);
  *bytes = layout(*joint, nullptr).bytes + 2 * act;
  return DIT_OK;
}

int check_params(const dit_block_params& p) {
  if (!p.mod || !p.w_in || !p.w_out || !p.q_scale || !p.k_scale) return DIT_ERR_NULL;
  if (misaligned(p.mod) || misaligned(p.w_in) || misaligned(p.w_out) || misaligned(p.q_scale) ||
      misaligned(p.k_scale))
    return DIT_ERR_ALIGN;
  return DIT_OK;
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

int dit_attn_fwd(int32_t n_tokens, int32_t n_heads, int32_t head_dim, const void* q,
                 const void* k, const void* v, void* o, float softmax_scale, hipStream_t stream) {
  if (n_tokens < 0 || n_tokens > DIT_MAX_TOKENS || n_heads <= 0 || head_dim <= 0)
    return DIT_ERR_SHAPE;
  if (head_dim != DIT_HEAD_DIM) return DIT_ERR_UNSUPPORTED;
  if ((long long)n_heads * head_dim > 65536) return DIT_ERR_UNSUPPORTED;
  if ((long long)n_tokens * n_heads * head_dim * 2 >= kMaxBytes) return DIT_ERR_UNSUPPORTED;
  if (bad_float(softmax_scale, true)) return DIT_ERR_ARG;
  if (n_tokens == 0) return DIT_OK;
  if (!q || !k || !v || !o) return DIT_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o)) return DIT_ERR_ALIGN;
  const size_t bytes = (size_t)n_tokens * n_heads * head_dim * 2;
  if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, k, bytes) || overlaps(o, bytes, v, bytes))
    return DIT_ERR_ARG;
  const int ld = n_heads * head_dim;
  return hip_status(dit::launch_attn(static_cast<const uint16_t*>(q),
                                     static_cast<const uint16_t*>(k),
                                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o),
                                     n_tokens, n_heads, ld, ld, softmax_scale, stream));
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
                                      theta, qk_eps, stream));
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
  auto run = [&](const dit_block_desc& d, const dit_block_params& p, char* h,
                 const int32_t* ps) -> int {
    return block_fwd(&d, h, p.mod, ps, p.w_in, p.w_out, p.q_scale, p.k_scale, h, wsp, block_ws,
                     stream, nullptr);
  };
  auto copy = [&](void* dst, const void* src, size_t n) -> int {
    return hip_status(hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, stream));
  };

  // stage 1, image and reference: shared by both branches
  if ((rc = copy(xc, x_img, img_bytes)) != DIT_OK) return rc;
  for (int i = 0; i < desc->n_img_blocks; ++i)
    if ((rc = run(di, bi[i], xc, pos)) != DIT_OK) return rc;
  if (refs) {
    if ((rc = copy(xc + img_bytes, x_ref, ref_bytes)) != DIT_OK) return rc;
    for (int i = 0; i < desc->n_ref_blocks; ++i)
      if ((rc = run(dr, br[i], xc + img_bytes, pos_ref)) != DIT_OK) return rc;
  }
  if (guided && (rc = copy(xn, xc, pre_bytes)) != DIT_OK) return rc;
  // stage 1, text, then the joint blocks, per branch (in place on
  // [image | reference | text])
  auto branch = [&](char* h, const void* x_txt) -> int {
    int r = copy(h + pre_bytes, x_txt, txt_bytes);
    if (r != DIT_OK) return r;
    for (int i = 0; i < desc->n_txt_blocks; ++i)
      if ((r = run(dt, bt[i], h + pre_bytes, pos_txt)) != DIT_OK) return r;
    for (int i = 0; i < desc->n_joint_blocks; ++i)
      if ((r = run(dj, bj[i], h, pos)) != DIT_OK) return r;
    return DIT_OK;
  };
  if ((rc = branch(xc, x_txt_cond)) != DIT_OK) return rc;
  if (!guided) return copy(v_img, xc, img_bytes);
  if ((rc = branch(xn, x_txt_neg)) != DIT_OK) return rc;
  return hip_status(dit::launch_cfg_combine(reinterpret_cast<const uint16_t*>(xc),
                                            reinterpret_cast<const uint16_t*>(xn),
                                            static_cast<uint16_t*>(v_img),
                                            (long long)desc->n_img * js.D, desc->cfg_scale,
                                            stream));
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
