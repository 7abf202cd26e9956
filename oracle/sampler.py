"""Plain float64 CPU oracle for one flow-matching denoise step of the model
around the block stack: timestep embedding and modulation, the token
embedders, the output layers, classifier-free guidance and the Euler step.

TEST INFRASTRUCTURE ONLY, like the block oracle next to it: only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it.

What the pages fix (sources are the pages' sections):

* The schedule: the DiffSynth-Studio FLUX.3 page, section "Model Inference",
  names a rational-shift coefficient alpha = 6.93 for the flow-matching
  schedule, and "Welcome FLUX.3 Image Klein in Diffusers", section "How it
  works", says that with this shift 44 of 50 steps run above sigma = 0.5.
  The shift is sigma' = alpha s / (1 + (alpha - 1) s) over s = 1 - i / n,
  i = 0 .. n, which gives exactly that count (the pin in the tests).
* Image tokens get the current timestep, text and reference tokens t = 0
  ("How it works").
* Only the image tokens reach the output layers, which give the velocity
  ("How it works", the diagram); the embedders and proj_out are named as
  LoRA targets (x_embedders.image, x_embedders.image_cond, context_embedder,
  proj_out) on the same page.
* A latent token has 128 channels (a 2 x 2 patch of the 32-channel latent,
  "How it works"); text features are 20,480 wide (8 Qwen3-VL layers stacked,
  same section).
* The guided velocity is neg + scale (cond - neg) (the miles page, section 3).

Readings taken where the pages are silent (parity of these against the
pages is unpinned; the tests pin each against mathematics instead):
  every embedder and proj_out is a linear layer with bias;
  the timestep enters as the sigma of the step, embedded as 256 sinusoids
  [cos | sin] of 1000 t times 10000^(-i/128), i = 0 .. 127, then
  Linear(256, D) + SiLU, Linear(D, D) + SiLU (the activated embedding e);
  shift, scale and gate are one Linear(D, 3D) of e per block group (stage-1
  image, stage-1 reference, stage-1 text, joint), shared by the blocks of
  the group, with the joint group's linear applied per stream to that
  stream's e;
  the output layers are LayerNorm (no affine) * (1 + scale) + shift with
  (shift, scale) = Linear(D, 2D) of the image e, then proj_out;
  the velocity is d z / d sigma, and one Euler step is
  z + (sigma_next - sigma) v;
  every layer's output is a bf16 tensor (the model runs in bf16): each layer
  is computed in float64 from bf16 inputs and its output rounded to bf16;
  the guided velocity and the Euler update are computed together in full
  precision and only the new latent is rounded.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .dit_block import layer_norm, silu, widen_bf16
from .stack import _run, cfg_combine, round_bf16

TIME_DIM = 256
TIME_MAX_PERIOD = 10000.0
TIME_SCALE = 1000.0
# block groups, in the order of the modulation linears
GROUP_IMG, GROUP_REF, GROUP_TXT, GROUP_JOINT = 0, 1, 2, 3


def f64(a) -> np.ndarray:
    a = np.asarray(a)
    return widen_bf16(a) if a.dtype == np.uint16 else a.astype(np.float64)


def flow_sigmas(n_steps: int, alpha: float) -> np.ndarray:
    """The n_steps + 1 sigmas of the shifted schedule, 1 down to 0."""
    s = 1.0 - np.arange(n_steps + 1, dtype=np.float64) / n_steps
    return alpha * s / (1.0 + (alpha - 1.0) * s)


def timestep_sinusoid(t: float, dim: int = TIME_DIM) -> np.ndarray:
    """[cos | sin] of TIME_SCALE t times the frequencies 10000^(-i / (dim/2))."""
    half = dim // 2
    freq = np.exp(-np.log(TIME_MAX_PERIOD) * np.arange(half, dtype=np.float64) / half)
    arg = TIME_SCALE * float(t) * freq
    return np.concatenate([np.cos(arg), np.sin(arg)])


def linear(x, w, b=None) -> np.ndarray:
    """x [.., K] times w [N, K] transposed, plus b [N]."""
    y = f64(x) @ f64(w).T
    return y if b is None else y + f64(b)


def time_embedding(t: float, w: Dict) -> np.ndarray:
    """The activated timestep embedding e = SiLU(Linear(SiLU(Linear(phi(t)))))."""
    phi = round_bf16(timestep_sinusoid(t))
    h = round_bf16(silu(linear(phi, w["t_w1"], w["t_b1"])))
    return round_bf16(silu(linear(h, w["t_w2"], w["t_b2"])))


def modulation(e: np.ndarray, w: Dict, group: int) -> np.ndarray:
    """(shift, scale, gate) [3, D] of one block group for embedding e."""
    return round_bf16(linear(e, w["mod_w"][group], w["mod_b"][group])).reshape(3, -1)


def output_layers(h_img: np.ndarray, e: np.ndarray, w: Dict, ln_eps: float) -> np.ndarray:
    """Velocity [n_img, C] of the image rows h_img [n_img, D]."""
    shift, scale = np.split(round_bf16(linear(e, w["out_mod_w"], w["out_mod_b"])), 2)
    u = round_bf16(layer_norm(f64(h_img), ln_eps) * (1.0 + scale) + shift)
    return round_bf16(linear(u, w["out_w"], w["out_b"]))


def euler_cfg_step(z, v_cond, v_neg: Optional[np.ndarray], scale: float, sigma: float,
                   sigma_next: float):
    """(z + (sigma_next - sigma) v, v) with v the guided velocity (v_cond when
    v_neg is None).  No rounding here."""
    v = f64(v_cond) if v_neg is None else cfg_combine(v_cond, v_neg, scale)
    return f64(z) + (sigma_next - sigma) * v, v


def _with_mod(blocks: Sequence[Dict], mod: np.ndarray) -> list:
    return [dict(b, mod=mod) for b in blocks]


def _groups(w: Dict, d: Dict):
    blocks = w["blocks"]
    a = d["n_img_blocks"]
    b = a + d["n_ref_blocks"]
    c = b + d["n_txt_blocks"]
    return blocks[:a], blocks[a:b], blocks[b:c], blocks[c:]


def sampler_prepare(w: Dict, d: Dict, pos, txt_cond, txt_neg=None, ref_latent=None) -> Dict:
    """The step-invariant part: text features and reference latents embedded
    and run through their stage-1 blocks at t = 0.

    d: dims (n_heads, head_dim, mlp_hidden, theta, ln_eps, qk_eps) plus
    n_img, n_img_blocks, n_ref_blocks, n_txt_blocks.
    """
    pos = np.asarray(pos, dtype=np.int64)
    n_img = d["n_img"]
    _, b_ref, b_txt, _ = _groups(w, d)
    e0 = time_embedding(0.0, w)
    out = {"e0": e0}
    n_ref = 0
    if ref_latent is not None and np.asarray(ref_latent).shape[0] > 0:
        n_ref = np.asarray(ref_latent).shape[0]
        x = round_bf16(linear(ref_latent, w["ref_in_w"], w["ref_in_b"]))
        m = modulation(e0, w, GROUP_REF)[None]
        out["ref"] = _run(x, _with_mod(b_ref, m), pos[n_img:n_img + n_ref], [n_ref], d)
    m = modulation(e0, w, GROUP_TXT)[None]
    p_txt = pos[n_img + n_ref:]
    for key, feat in (("txt_cond", txt_cond), ("txt_neg", txt_neg)):
        if feat is None:
            continue
        x = round_bf16(linear(feat, w["txt_in_w"], w["txt_in_b"]))
        out[key] = _run(x, _with_mod(b_txt, m), p_txt, [x.shape[0]], d)
    return out


def denoise_step(w: Dict, d: Dict, prep: Dict, z, sigma: float, sigma_next: float, pos,
                 cfg_scale: float):
    """One Euler step of the latent z [n_img, C] from sigma to sigma_next.

    Returns (z_next rounded to bf16, the guided velocity, the per-branch
    velocities)."""
    pos = np.asarray(pos, dtype=np.int64)
    n_img = d["n_img"]
    b_img, _, _, b_joint = _groups(w, d)
    e = time_embedding(sigma, w)
    e0 = prep["e0"]
    x = round_bf16(linear(z, w["img_in_w"], w["img_in_b"]))
    h_img = _run(x, _with_mod(b_img, modulation(e, w, GROUP_IMG)[None]), pos[:n_img], [n_img], d)
    mj_img, mj_ctx = modulation(e, w, GROUP_JOINT), modulation(e0, w, GROUP_JOINT)
    has_ref = "ref" in prep
    mod_joint = np.stack([mj_img, mj_ctx, mj_ctx] if has_ref else [mj_img, mj_ctx])
    joint = _with_mod(b_joint, mod_joint)

    def branch(txt):
        parts = [h_img] + ([prep["ref"]] if has_ref else []) + [txt]
        n_tokens = [p.shape[0] for p in parts]
        h = _run(np.concatenate(parts), joint, pos, n_tokens, d)
        return output_layers(h[:n_img], e, w, d.get("ln_eps", 1e-6))

    v_c = branch(prep["txt_cond"])
    v_n = branch(prep["txt_neg"]) if cfg_scale != 1.0 else None
    z_next, v = euler_cfg_step(z, v_c, v_n, cfg_scale, sigma, sigma_next)
    return round_bf16(z_next), v, (v_c, v_n)


def sample(w: Dict, d: Dict, pos, z, txt_cond, txt_neg, ref_latent, n_steps: int, alpha: float,
           cfg_scale: float) -> np.ndarray:
    """n_steps Euler steps from sigma = 1 to 0 of the shifted schedule."""
    sig = flow_sigmas(n_steps, alpha)
    prep = sampler_prepare(w, d, pos, txt_cond, txt_neg if cfg_scale != 1.0 else None,
                           ref_latent)
    z = f64(z)
    for i in range(n_steps):
        z = denoise_step(w, d, prep, z, sig[i], sig[i + 1], pos, cfg_scale)[0]
    return z
