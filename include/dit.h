/*
 * dit.h - C ABI of the MI355X (gfx950) forward of the FLUX.3 Image Klein
 * parallel DiT block.
 *
 * The block (pages: "Welcome FLUX.3 Image Klein in Diffusers", section
 * "How it works"; the miles page "FLUX 3 Image Klein", sections 1 and 3;
 * the NeMo AutoModel page, section "Image-Editing LoRA"):
 *   u  = LN(x) * (1 + scale_s) + shift_s          per-stream AdaLN modulation
 *   z  = u W_in^T = [q | k | v | gate | up]       to_q, to_k, to_v, ff.linear_in
 *   q, k <- RoPE4(RMSNorm_head(q|k) * g_q|g_k)    QK norm, 4-axis RoPE (t, h, w, l)
 *   o  = softmax(q k^T / sqrt(d)) v               full joint attention, no mask
 *   m  = silu(gate) * up                          SwiGLU, in parallel with attention
 *   r  = [o | m] W_out^T                          to_out.0 + ff.linear_out
 *   y  = x + gate_s * r                           gated residual
 * where s is the stream (image, reference, text) of the token.  Image tokens
 * carry the modulation of the current timestep t, text and reference tokens
 * the modulation of t = 0; the modulation vectors themselves are inputs.
 *
 * Around the block, in sections of their own below: the block with FP8
 * projections, the two-stage stack with classifier-free guidance, and the
 * flow-matching sampler (timestep modulation, embedders, output layers and
 * the guided Euler step).
 *
 * Conventions shared by every call:
 *   - Tensors are device pointers owned by the caller, row-major, bf16 stored
 *     as 16-bit patterns unless stated.  They must be 16-byte aligned.
 *   - Work is enqueued on `stream` (0 = the null stream); calls return once
 *     enqueued.  The library never allocates or frees device memory and
 *     never synchronizes with the host.  Its global state, per device: a
 *     cache of the CU count, the scratch array of dit_block_fwd_noalloc, and
 *     the side stream of DIT_STACK_TEXT_SIDE_STREAM with its events (created
 *     on first use); calls may come from several threads.
 *   - Validation runs on the host before any launch; on error nothing is
 *     launched and outputs are untouched.  Errors are negative status codes,
 *     and dit_status_str() names them.
 *   - Token order in a sequence is [image | reference | text]; a call names
 *     the token count of each segment present, in that order.
 *   - Supported shapes: head_dim = 128 (4 RoPE axes of 32 dims), width =
 *     n_heads * 128 with n_heads a multiple of 4 and width at most 8192,
 *     mlp_hidden a multiple of 128 (at most 65536), at most DIT_MAX_TOKENS
 *     tokens, and every tensor (including the [N, D + F] internal buffer)
 *     under 4 GiB; larger calls return DIT_ERR_UNSUPPORTED.  The FLUX.3
 *     Image Klein block is width 3072, 24 heads, mlp_hidden 9216.
 *   - A token count of 0 is a valid empty call: DIT_OK, nothing launched.
 */
#ifndef DIT_H
#define DIT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DIT_OK = 0,
  DIT_ERR_NULL = -1,        /* a required pointer is null */
  DIT_ERR_SHAPE = -2,       /* inconsistent sizes (negative counts, H*d != width, too many tokens) */
  DIT_ERR_UNSUPPORTED = -3, /* a size this library does not implement (head_dim != 128, ...) */
  DIT_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
  DIT_ERR_WORKSPACE = -5,   /* workspace null or smaller than dit_block_workspace_bytes() */
  DIT_ERR_HIP = -6,         /* the HIP runtime reported a launch error */
  DIT_ERR_ARG = -7          /* a scalar argument is out of range (eps, theta, flags) */
};

#define DIT_MAX_STREAMS 3
#define DIT_MAX_TOKENS 131072
#define DIT_HEAD_DIM 128

/* flags of dit_block_desc (diagnostics for checking the branch on its own) */
#define DIT_F_NO_RESIDUAL 1u /* y = gate_s * r            */
#define DIT_F_NO_GATE 2u     /* the gate is taken as 1     */

/* Stages of dit_block_fwd, in launch order (see dit_block_fwd_events). */
#define DIT_STAGE_ADALN 0    /* per-stream AdaLN -> u                           */
#define DIT_STAGE_GEMM_IN 1  /* u W_in^T -> q, k, v and SwiGLU m, with the QK    */
                             /* RMSNorm + 4-axis RoPE of q, k in its epilogue   */
#define DIT_STAGE_ROPE 2     /* empty: the RoPE is fused into the stage above   */
#define DIT_STAGE_ATTN 3     /* joint attention -> o                            */
#define DIT_STAGE_GEMM_OUT 4 /* [o | m] W_out^T, gated residual -> y            */
#define DIT_N_STAGES 5

typedef struct dit_block_desc {
  int32_t n_streams;                 /* 1..3 segments, in [image | reference | text] order */
  int32_t n_tokens[DIT_MAX_STREAMS]; /* tokens per present segment; N = their sum          */
  int32_t width;                     /* D, 3072                                            */
  int32_t n_heads;                   /* H, 24                                              */
  int32_t head_dim;                  /* d, 128                                             */
  int32_t mlp_hidden;                /* F, 9216                                            */
  float rope_theta;                  /* 10000                                              */
  float ln_eps;                      /* 1e-6, LayerNorm epsilon                            */
  float qk_eps;                      /* 1e-6, QK RMSNorm epsilon                           */
  uint32_t flags;                    /* DIT_F_* bits, 0 for the block itself               */
} dit_block_desc;

/* Bytes of device workspace dit_block_fwd needs for `desc`: u, q, k, v and the
 * [o | m] concat buffer, all bf16 (16 * N * D bytes at F = 3 D), plus a fixed
 * 128 MiB of fp32 scratch for the split tails of the GEMMs (and the split
 * partials of attention) and 4 KiB of attention counters.
 * After a call the workspace holds the block's intermediates, at offsets that
 * are multiples of R = (N * D * 2 rounded up to 256 bytes):
 *   0:   u   bf16 [N, D]      the modulated input
 *   R:   q   bf16 [N, H, d]   after QK RMSNorm and RoPE, multiplied by
 *                             (float)(1 / sqrt(128)) * (float)log2(e)
 *   2R:  k   bf16 [N, H, d]   after QK RMSNorm and RoPE
 *   3R:  v   bf16 [N, H, d]
 *   4R:  [o | m] bf16 [N, D + F]  attention output, then the SwiGLU product
 * (for inspection and tests; the layout is part of this contract). */
int dit_block_workspace_bytes(const dit_block_desc* desc, size_t* bytes);

/* One parallel block forward (the whole chain above).
 *   x        bf16 [N, D]             input tokens
 *   mod      bf16 [S, 3, D]          per stream: shift, scale, gate
 *   pos      int32 [N, 4]            (t, h, w, l) RoPE position of each token
 *   w_in     bf16 [3D + 2F, D]       rows: to_q | to_k | to_v | linear_in gate | linear_in up
 *   w_out    bf16 [D, D + F]         columns: to_out.0 (attention) | linear_out (MLP)
 *   q_scale  bf16 [d], k_scale bf16 [d]   QK RMSNorm scales
 *   y        bf16 [N, D]             output; y == x (in place) is allowed, any
 *                                    other overlap between y and an input is not
 *   workspace device memory of at least dit_block_workspace_bytes(desc)
 * Rounding: activations between stages are stored as bf16 (round to nearest
 * even); every sum is accumulated in fp32. */
int dit_block_fwd(const dit_block_desc* desc, const void* x, const void* mod, const int32_t* pos,
                  const void* w_in, const void* w_out, const void* q_scale, const void* k_scale,
                  void* y, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* dit_block_fwd that also records events[i] on `stream` before stage i and
 * events[DIT_N_STAGES] after the last stage, so the caller can time each
 * stage with hipEventElapsedTime.  events: host array of DIT_N_STAGES + 1
 * created hipEvent_t handles. */
int dit_block_fwd_events(const dit_block_desc* desc, const void* x, const void* mod,
                         const int32_t* pos, const void* w_in, const void* w_out,
                         const void* q_scale, const void* k_scale, void* y, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, void* const* events);

/* ---- The block without a caller-supplied workspace --------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the block
 * of dit_block_fwd with its workspace in a file-scope device array of the
 * library (dit_block_noalloc_scratch_bytes() bytes per GPU, about 348 MB),
 * held from the library's first use on that GPU until the process ends.  The array is sized for the
 * FLUX.3 block (width 3072, mlp_hidden 9216) at up to DIT_NOALLOC_MAX_TOKENS
 * tokens (a 1024^2 image with up to 256 text tokens, or any stage-1 block of
 * it); a descriptor whose workspace would not fit is refused with
 * DIT_ERR_WORKSPACE before anything is launched.  Arguments, results and
 * other errors as for dit_block_fwd; the call itself allocates nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (several streams, or several host threads) race and must be
 * serialized by the caller.  The array keeps the last call's contents; the
 * block writes every part of it it reads before reading it. */
#define DIT_NOALLOC_MAX_TOKENS 4352
#define DIT_NOALLOC_WIDTH 3072
#define DIT_NOALLOC_MLP_HIDDEN 9216

int dit_block_fwd_noalloc(const dit_block_desc* desc, const void* x, const void* mod,
                          const int32_t* pos, const void* w_in, const void* w_out,
                          const void* q_scale, const void* k_scale, void* y, hipStream_t stream);

/* Size in bytes of that per-GPU array (host query, no device access). */
int dit_block_noalloc_scratch_bytes(size_t* bytes);

/* Full (unmasked) multi-head attention over all N tokens
 * ("How it works": full attention in the 28 joint blocks; padding attended).
 *   q, k, v  bf16 [N, H, d]   o  bf16 [N, H, d] (must not overlap q, k, v)
 *   o[i, h] = sum_j softmax_j(q[i, h] . k[j, h] * softmax_scale) v[j, h]
 * Online softmax in fp32; the probabilities are rounded to bf16 before the
 * product with v.  softmax_scale must be finite and > 0 (1/sqrt(d) for the block). */
int dit_attn_fwd(int32_t n_tokens, int32_t n_heads, int32_t head_dim, const void* q,
                 const void* k, const void* v, void* o, float softmax_scale, hipStream_t stream);

/* Bytes of device workspace dit_attn_fwd_ws needs (a fixed size, about 71 MB,
 * for any valid shape; the shape is checked as in dit_attn_fwd). */
int dit_attn_workspace_bytes(int32_t n_tokens, int32_t n_heads, int32_t head_dim,
                             size_t* bytes);

/* dit_attn_fwd with a workspace, which lets it balance the work over the
 * CUs the way the block's attention does: when there are more (head, 256-query)
 * items than CUs, each CU takes an equal share of the key tiles of all
 * items, and an item cut between two shares is merged from two fp32
 * partials kept in the workspace.  With two or more rounds of items, all
 * but the last round and the remainder run as whole items first, one per CU
 * per round, and only the rest is shared out.  Same result definition and errors as
 * dit_attn_fwd, plus DIT_ERR_WORKSPACE (null or too small) and DIT_ERR_ARG
 * (workspace overlapping q, k, v or o). */
int dit_attn_fwd_ws(int32_t n_tokens, int32_t n_heads, int32_t head_dim, const void* q,
                    const void* k, const void* v, void* o, float softmax_scale, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/* In-place per-head QK RMSNorm (when q_scale and k_scale are both non-null)
 * followed by 4-axis RoPE on q and k ("How it works": axes t, h, w, l each
 * own 32 of the 128 head dims; the miles page, section 3: query_norm.scale,
 * key_norm.scale).
 *   q, k     bf16 [N, H, d], rotated in place
 *   pos      int32 [N, 4]   (t, h, w, l)
 *   Axis a owns dims [32a, 32a + 32); pair j = dims (32a + 2j, 32a + 2j + 1)
 *   turns by pos_a * theta^(-2j/32): (x, y) -> (x cos - y sin, x sin + y cos).
 *   RMSNorm: q / sqrt(mean q^2 + qk_eps) * q_scale per head (same for k).
 * q_scale and k_scale must both be null (no norm) or both be set. */
int rope4_apply(int32_t n_tokens, int32_t n_heads, int32_t head_dim, void* q, void* k,
                const int32_t* pos, float theta, const void* q_scale, const void* k_scale,
                float qk_eps, hipStream_t stream);

/* Per-stream AdaLN modulation ("How it works": shift and scale set
 * separately per stream, applied to the shared normalized input):
 *   out[i] = (x[i] - mean) / sqrt(var + eps) * (1 + scale_s) + shift_s
 * with the biased variance over the row, s the row's stream.
 *   n_tokens  HOST array of n_streams token counts ([image | reference | text])
 *   x, out    bf16 [N, width]   (out may equal x)
 *   mod       bf16 [n_streams, 3, width]; the gate row is not read here
 * width must be a multiple of 512 and at most 8192. */
int adaln_mod(int32_t n_streams, const int32_t* n_tokens, int32_t width, const void* x,
              const void* mod, void* out, float eps, hipStream_t stream);

/* ---- FP8 projections (rowwise-scaled e4m3) ---------------------------------
 * The analogue of the rowwise-scaled FP8 linear layers ("fp8r") that the
 * SGLang FLUX.3 page ships for latency, on gfx950's FP8 MFMA (OCP e4m3).
 * Rowwise quantization of a bf16 matrix X [M, K], per row r:
 *   a_r = max_k |x_rk|, inv_r = 448 / a_r and s_r = a_r / 448 (float32,
 *   correctly rounded), q_rk = e4m3(clamp(x_rk * inv_r, -448, 448)) rounded
 *   to nearest even, so x_rk ~ q_rk * s_r; an all-zero row gets s_r = 0 and
 *   q = 0.
 * The FP8 block is dit_block_fwd with both projections in FP8: u (the AdaLN
 * output, rounded to bf16) and [o | m] are quantized per token row, W_in and
 * W_out per output row (once, with dit_quantize_rows_fp8), and each product
 * is sum_k q_a q_w * s_a s_w with fp32 accumulation.  Everything else (the
 * QK norm, RoPE, attention, SwiGLU, gate and residual) is as in the bf16 block. */

/* Rowwise quantization: x bf16 [M, K] -> q e4m3 [M, K] (1 byte each), scale
 * float [M].  K a multiple of 8.  Device pointers, 16-byte aligned, not
 * overlapping. */
int dit_quantize_rows_fp8(int32_t M, int32_t K, const void* x, void* q, float* scale,
                          hipStream_t stream);

/* Bytes of device workspace dit_block_fwd_fp8 needs: the bf16 block's plus
 * the codes and scales of u and [o | m]. */
int dit_block_fp8_workspace_bytes(const dit_block_desc* desc, size_t* bytes);

/* The block with FP8 projections.  Arguments as dit_block_fwd, except:
 *   w_in8       e4m3 [3D + 2F, D]  and w_in_scale  float [3D + 2F]
 *   w_out8      e4m3 [D, D + F]    and w_out_scale float [D]
 * as produced by dit_quantize_rows_fp8 from the bf16 weights.  Errors as for
 * dit_block_fwd. */
int dit_block_fwd_fp8(const dit_block_desc* desc, const void* x, const void* mod,
                      const int32_t* pos, const void* w_in8, const float* w_in_scale,
                      const void* w_out8, const float* w_out_scale, const void* q_scale,
                      const void* k_scale, void* y, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* dit_block_fwd_fp8 with DIT_N_STAGES + 1 events recorded between its stages
 * (as dit_block_fwd_events; the quantization of [o | m] is in the output
 * projection's stage). */
int dit_block_fwd_fp8_events(const dit_block_desc* desc, const void* x, const void* mod,
                             const int32_t* pos, const void* w_in8, const float* w_in_scale,
                             const void* w_out8, const float* w_out_scale, const void* q_scale,
                             const void* k_scale, void* y, void* workspace,
                             size_t workspace_bytes, hipStream_t stream, void* const* events);

/* ---- Two-stage stack and classifier-free guidance -------------------------
 * One denoise step of the transformer ("Welcome FLUX.3 Image Klein in
 * Diffusers", section "How it works": each stream, text, image and
 * reference, first runs through blocks of its own, attending only to itself,
 * then the streams are concatenated and run through the shared joint blocks;
 * the miles page "FLUX 3 Image Klein", section 3: the guided prediction is
 * neg + scale * (pos - neg) from a forward with the prompt and one with the
 * negative prompt).  Every block is the parallel block of dit_block_fwd.
 * Embedders and output layers are not part of this call: the tokens enter as
 * given, and the guided result is taken on the image rows of the joint
 * stack's output.  All reference images form one reference stream (their
 * rows carry their own l index in pos), which runs the reference blocks as
 * one sequence. */
typedef struct dit_stack_desc {
  int32_t n_img;          /* image tokens (> 0)                                    */
  int32_t n_ref;          /* reference tokens, all references together (>= 0)     */
  int32_t n_txt;          /* text tokens of each branch (> 0)                      */
  int32_t n_img_blocks;   /* stage-1 image blocks (5)                              */
  int32_t n_ref_blocks;   /* stage-1 reference blocks (5; 0 when n_ref == 0)       */
  int32_t n_txt_blocks;   /* stage-1 text blocks (5)                               */
  int32_t n_joint_blocks; /* stage-2 joint blocks over [image | reference | text]  */
                          /* (28)                                                  */
  int32_t width;          /* D, 3072                                               */
  int32_t n_heads;        /* H, 24                                                 */
  int32_t head_dim;       /* 128                                                   */
  int32_t mlp_hidden;     /* F, 9216                                               */
  float rope_theta;       /* 10000                                                 */
  float ln_eps;           /* 1e-6                                                  */
  float qk_eps;           /* 1e-6                                                  */
  float cfg_scale;        /* guidance scale, finite; 1 runs the conditional branch */
                          /* only (no negative forward)                           */
  uint32_t flags;         /* DIT_STACK_* bits, 0 for none                          */
} dit_stack_desc;

/* Run the stage-1 text blocks of both branches on a second stream, beside
 * the stage-1 image and reference blocks (they read no image rows: "Welcome
 * FLUX.3 Image Klein in Diffusers", "How it works", the stage-1 streams are
 * processed separately).  The library owns that stream (one per device,
 * created on first use, non-blocking, default priority) and joins it back
 * into the caller's stream with events before the joint blocks, so the call
 * stays asynchronous and capturable in a HIP graph.  All calls on a device
 * share that stream, so their text blocks run one call after another.  Costs a second block
 * workspace at n_txt tokens (counted by dit_stack_workspace_bytes).  Results
 * are bitwise those of the serial order. */
#define DIT_STACK_TEXT_SIDE_STREAM 1u

/* Device pointers of one block's parameters. */
typedef struct dit_block_params {
  const void* mod;     /* bf16 [S, 3, D]: S = 1 for a stage-1 block; for a joint  */
                       /* block S = 3 (image, reference, text) when n_ref > 0,    */
                       /* else 2 (image, text)                                    */
  const void* w_in;    /* bf16 [3D + 2F, D], as in dit_block_fwd */
  const void* w_out;   /* bf16 [D, D + F]  */
  const void* q_scale; /* bf16 [d]         */
  const void* k_scale; /* bf16 [d]         */
} dit_block_params;

/* Bytes of device workspace dit_stack_fwd needs: the block workspace at
 * N = n_img + n_ref + n_txt plus two [N, D] bf16 activation buffers (one per
 * branch), plus a block workspace at n_txt tokens with
 * DIT_STACK_TEXT_SIDE_STREAM. */
int dit_stack_workspace_bytes(const dit_stack_desc* desc, size_t* bytes);

/* One guided stack forward.
 *   x_img       bf16 [n_img, D]   image tokens entering stage 1
 *   x_ref       bf16 [n_ref, D]   reference tokens (null when n_ref == 0)
 *   x_txt_cond  bf16 [n_txt, D]   text tokens of the prompt
 *   x_txt_neg   bf16 [n_txt, D]   text tokens of the negative prompt (may be
 *                                 null when cfg_scale == 1)
 *   pos         int32 [n_img + n_ref + n_txt, 4]  joint (t, h, w, l) positions
 *                                 in [image | reference | text] order;
 *                                 stage-1 blocks use their rows
 *   blocks      host array of n_img_blocks + n_ref_blocks + n_txt_blocks +
 *               n_joint_blocks entries in that order
 *   v_img       bf16 [n_img, D]   out: neg + cfg_scale * (cond - neg) on the
 *                                 image rows of the joint output, in fp32, rounded
 *                                 to bf16 (the cond rows when cfg_scale == 1)
 * The stage-1 image and reference blocks do not see the text, so both
 * branches share them.  Activations between blocks are bf16, as in
 * dit_block_fwd.  Inputs are only read; v_img must not overlap the
 * workspace.  Every size and block pointer is checked before the first
 * launch; errors as for dit_block_fwd. */
int dit_stack_fwd(const dit_stack_desc* desc, const void* x_img, const void* x_ref,
                  const void* x_txt_cond, const void* x_txt_neg, const int32_t* pos,
                  const dit_block_params* blocks, void* v_img, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);

/* ---- Flow-matching sampler around the stack --------------------------------
 * One Euler step of the latent from sigma to sigma_next, with the model's
 * layers around the stack.  What the pages fix: the schedule's rational
 * shift (alpha = 6.93: the DiffSynth-Studio FLUX.3 page, "Model Inference";
 * 44 of 50 steps above sigma = 0.5: "Welcome FLUX.3 Image Klein in
 * Diffusers", "How it works"), image tokens at the step's timestep and text
 * and reference tokens at t = 0, image tokens alone reaching the output
 * layers, 128-channel latent tokens and 20,480-wide text features (same
 * section), the embedders and proj_out by name (same page, the LoRA target
 * list) and neg + scale * (cond - neg) on the velocities (the miles page,
 * section 3).  Read where the pages are silent: every embedder and proj_out
 * is a linear layer with bias; the timestep t = sigma is embedded as 256
 * sinusoids [cos | sin] of 1000 t 10000^(-i/128), then Linear(256, D) + SiLU,
 * Linear(D, D) + SiLU = e; each block group (stage-1 image, reference, text;
 * joint) has one Linear(D, 3D) of e giving (shift, scale, gate) to all its
 * blocks, the joint group's applied per stream to that stream's e; the output
 * layers are LayerNorm(no affine) * (1 + scale) + shift with (shift, scale) =
 * Linear(D, 2D) of the image e, then proj_out; the velocity is dz / dsigma.
 * Every tensor is bf16 (fp32 accumulation), the update z + dsigma v is taken
 * in fp32 and rounded. */

#define DIT_N_GROUPS 4 /* block groups: stage-1 image, reference, text; joint */
#define DIT_TIME_DIM 256

typedef struct dit_model_desc {
  dit_stack_desc stack; /* tokens, block counts, widths, eps and cfg_scale; its     */
                        /* flags must be 0 (the text blocks run once, in           */
                        /* dit_sampler_prepare)                                    */
  int32_t latent_ch;    /* C, channels of a latent token (128): a multiple of 32,   */
                        /* at most 8192                                             */
  int32_t text_dim;     /* width of a text feature (20480): a multiple of 16        */
} dit_model_desc;

/* Device pointers of one block's weights (its modulation comes from its group). */
typedef struct dit_block_weights {
  const void* w_in;    /* bf16 [3D + 2F, D] */
  const void* w_out;   /* bf16 [D, D + F]   */
  const void* q_scale; /* bf16 [d]          */
  const void* k_scale; /* bf16 [d]          */
} dit_block_weights;

/* Device pointers of the layers around the blocks, all bf16, [out, in]. */
typedef struct dit_model_weights {
  const void* img_in_w;                /* [D, C]  x_embedders.image                       */
  const void* img_in_b;                /* [D]                                             */
  const void* ref_in_w;                /* [D, C]  x_embedders.image_cond (n_ref > 0 only) */
  const void* ref_in_b;                /* [D]                                             */
  const void* txt_in_w;                /* [D, text_dim]  context_embedder                 */
  const void* txt_in_b;                /* [D]                                             */
  const void* t_w1;                    /* [D, 256]  timestep MLP, first layer             */
  const void* t_b1;                    /* [D]                                             */
  const void* t_w2;                    /* [D, D]    second layer                          */
  const void* t_b2;                    /* [D]                                             */
  const void* mod_w[DIT_N_GROUPS];     /* [3D, D]  (shift | scale | gate) per group       */
  const void* mod_b[DIT_N_GROUPS];     /* [3D]                                            */
  const void* out_mod_w;               /* [2D, D]  (shift | scale) of the output norm     */
  const void* out_mod_b;               /* [2D]                                            */
  const void* out_w;                   /* [C, D]   proj_out                               */
  const void* out_b;                   /* [C]                                             */
  const dit_block_weights* blocks;     /* host array: n_img_blocks + n_ref_blocks +       */
                                       /* n_txt_blocks + n_joint_blocks, in that order    */
} dit_model_weights;

/* The n_steps + 1 sigmas of the shifted schedule into host memory:
 * sigma_i = alpha u / (1 + (alpha - 1) u), u = 1 - i / n_steps (1 down to 0).
 * n_steps in [1, 100000], alpha finite and > 0. */
int dit_flow_sigmas(int32_t n_steps, double alpha, double* sigmas);

/* Bytes of device workspace the sampler needs: the stack's workspace plus the
 * prepared text and reference rows, the timestep path and the velocities.
 * The same workspace must be passed to dit_sampler_prepare and every
 * following dit_sampler_step: it carries the prepared rows between calls. */
int dit_sampler_workspace_bytes(const dit_model_desc* desc, size_t* bytes);

/* The step-invariant part of sampling, once per generation: the text
 * features of both prompts and the reference latents embedded and run
 * through their stage-1 blocks at t = 0 (text and reference tokens always
 * get t = 0, so these rows are the same at every step).
 *   txt_cond    bf16 [n_txt, text_dim]  text features of the prompt
 *   txt_neg     bf16 [n_txt, text_dim]  of the negative prompt (null when
 *                                       cfg_scale == 1)
 *   ref_latent  bf16 [n_ref, C]         reference latent tokens (null when
 *                                       n_ref == 0)
 *   pos         int32 [N, 4]            (t, h, w, l) in [image | reference | text]
 * Writes only the workspace. */
int dit_sampler_prepare(const dit_model_desc* desc, const dit_model_weights* weights,
                        const void* txt_cond, const void* txt_neg, const void* ref_latent,
                        const int32_t* pos, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* One guided Euler step, in place on the latent:
 *   z      bf16 [n_img, C]  in: the latent at sigma; out: at sigma_next
 *   v_out  bf16 [n_img, C]  optional: the guided velocity
 * sigma and sigma_next finite (the sampler passes consecutive entries of
 * dit_flow_sigmas).  Needs a workspace prepared by dit_sampler_prepare with
 * the same desc, weights and pos. */
int dit_sampler_step(const dit_model_desc* desc, const dit_model_weights* weights, void* z,
                     double sigma, double sigma_next, const int32_t* pos, void* v_out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* y = act(x w^T + b), a linear layer as the sampler runs it (bf16, fp32
 * accumulation): x [M, K], w [N, K], b [N] or null, y [M, N], act 0 (none) or
 * 1 (SiLU after the bias).  K a multiple of 16, N of 32; y must not overlap x,
 * w or b. */
int dit_linear(int32_t M, int32_t N, int32_t K, const void* x, const void* w, const void* b,
               int32_t act, void* y, hipStream_t stream);

/* out bf16 [n_t, 256]: the timestep sinusoids of n_t (1..4) host values t. */
int dit_time_sinusoid(int32_t n_t, const double* t, void* out, hipStream_t stream);

/* Static name of a status code ("DIT_OK", "DIT_ERR_SHAPE: ...", ...). */
const char* dit_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* DIT_H */
