"""Seeded synthetic inputs for the parallel DiT block.

This module only draws and encodes numbers; it holds none of the block's
arithmetic.  Both the fp64 oracle (through the tests) and the HIP path read the
exact same bytes from here.

Recipe (the pages ship no tensors, weights or data, so seeded random tensors of
the pages' shapes stand in for them):
  * generator: numpy PCG64 keyed by SeedSequence([seed, config_id, block_id,
    tensor_id, ...]); values drawn in float64, scaled, then rounded
    round-to-nearest-even straight from float64 to bfloat16;
  * x ~ N(0, 1); W_in ~ N(0, 1/width); W_out ~ N(0, 1/(width + mlp_hidden));
    per-stream shift / scale / gate ~ N(0, 0.1) (0.1 read as the variance);
  * QK-norm scales are ones (their initial value);
  * positions (t, h, w, l): image token i of a rows x cols grid is
    (0, i // cols, i % cols, 0); a reference uses the same grid with l = 1;
    text token k is (k, 0, 0, 0), padding included.  This follows the 4-axis
    RoPE description in "Welcome FLUX.3 Image Klein in Diffusers", section
    "How it works" (references share (h, w) with the output);
  * the sampler's layers around the blocks (make_sampler_inputs): every
    weight ~ N(0, 1/fan_in) except the modulation linears, N(0, 0.1/fan_in),
    so shift / scale / gate come out at about the size above; biases
    ~ N(0, 0.01); the latent, reference latents and text features ~ N(0, 1).
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .configs import BlockConfig, STREAM_IMAGE, STREAM_REF, STREAM_TEXT, Stream

TENSOR_X = 1
TENSOR_MOD = 2
TENSOR_W_IN = 3
TENSOR_W_OUT = 4
TENSOR_QKV = 5  # standalone attention inputs
TENSOR_SAMPLER = 6

_CHUNK = 1 << 22


def f64_to_bf16_bits(a) -> np.ndarray:
    """Round float64 values to bfloat16, round-to-nearest-even, in one step.

    Returns the raw 16-bit patterns as uint16.  bfloat16 keeps 8 significant
    bits, so the low 45 of float64's 52 mantissa bits are rounded away; the
    result then converts exactly to float32, whose top half is the bf16
    pattern.  Values must be finite and outside float32's subnormal range.
    """
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite value in bf16 encode")
    b = a.view(np.uint64)
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    b = (b + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    r = b.view(np.float64)
    mag = np.abs(r)
    if np.any((mag != 0) & (mag < 2.0 ** -126)) or np.any(mag >= 2.0 ** 128):
        raise ValueError("value outside the bf16 normal range")
    f = r.astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def normal_bf16(shape, std: float, *key: int) -> np.ndarray:
    """N(0, std^2) draws in float64, rounded to bf16 bits; drawn in chunks."""
    rng = _rng(*key)
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.uint16)
    for s in range(0, total, _CHUNK):
        e = min(total, s + _CHUNK)
        out[s:e] = f64_to_bf16_bits(rng.standard_normal(e - s) * std)
    return out.reshape(shape)


def positions(cfg: BlockConfig) -> np.ndarray:
    """int32 [N, 4] position table (t, h, w, l) in [image | reference | text] order."""
    rows = []
    for s in cfg.streams:
        p = np.zeros((s.n, 4), dtype=np.int32)
        if s.kind in (STREAM_IMAGE, STREAM_REF):
            gr, gc = s.grid
            if gr * gc != s.n:
                raise ValueError(f"grid {s.grid} does not match {s.n} tokens")
            i = np.arange(s.n)
            p[:, 1] = i // gc
            p[:, 2] = i % gc
            p[:, 3] = 1 if s.kind == STREAM_REF else 0
        elif s.kind == STREAM_TEXT:
            p[:, 0] = np.arange(s.n)
        else:
            raise ValueError(s.kind)
        rows.append(p)
    return np.concatenate(rows, axis=0)


def make_block_inputs(cfg: BlockConfig, seed: int = 0, block_id: int = 0,
                      weights: bool = True) -> Dict[str, np.ndarray]:
    """All inputs of one block forward as bf16 bit patterns (uint16) / int32.

    Keys: x [N, D], mod [S, 3, D] (shift, scale, gate per stream), pos [N, 4],
    w_in [3D + 2F, D] (rows q | k | v | gate | up), w_out [D, D + F]
    (columns attention-out | mlp-out), q_scale [d], k_scale [d].
    """
    D, F, d = cfg.width, cfg.mlp_hidden, cfg.head_dim
    out: Dict[str, np.ndarray] = {}
    out["x"] = normal_bf16((cfg.N, D), 1.0, seed, cfg.config_id, block_id, TENSOR_X)
    mods = []
    for si, s in enumerate(cfg.streams):
        mods.append(normal_bf16((3, D), np.sqrt(0.1), seed, cfg.config_id, block_id,
                                TENSOR_MOD, si, int(round(s.t * 1000))))
    out["mod"] = np.stack(mods, axis=0)
    out["pos"] = positions(cfg)
    if weights:
        out["w_in"] = normal_bf16((3 * D + 2 * F, D), 1.0 / np.sqrt(D),
                                  seed, cfg.config_id, block_id, TENSOR_W_IN)
        out["w_out"] = normal_bf16((D, D + F), 1.0 / np.sqrt(D + F),
                                   seed, cfg.config_id, block_id, TENSOR_W_OUT)
    one = f64_to_bf16_bits(np.ones(d))
    out["q_scale"] = one.copy()
    out["k_scale"] = one.copy()
    return out


def make_attn_inputs(n_tokens: int, n_heads: int, head_dim: int, seed: int = 0,
                     logit_std: float = 1.0, case: int = 0) -> Dict[str, np.ndarray]:
    """Standalone attention inputs q, k, v as bf16 bits [N, H, d].

    q and k entries are drawn with std sqrt(logit_std): a dot product of d such
    products has variance d * logit_std^2, so the scaled logits q.k / sqrt(d)
    have standard deviation about logit_std.
    """
    qk_std = float(np.sqrt(logit_std))
    shape = (n_tokens, n_heads, head_dim)
    return {
        "q": normal_bf16(shape, qk_std, seed, 100 + case, n_tokens, TENSOR_QKV, 0),
        "k": normal_bf16(shape, qk_std, seed, 100 + case, n_tokens, TENSOR_QKV, 1),
        "v": normal_bf16(shape, 1.0, seed, 100 + case, n_tokens, TENSOR_QKV, 2),
    }


def make_sampler_inputs(n_img_side: int, n_ref_side: int, n_txt: int, blocks, seed: int = 0,
                        width: int = 3072, n_heads: int = 24, head_dim: int = 128,
                        mlp_hidden: int = 9216, latent_ch: int = 128, text_dim: int = 20480,
                        time_dim: int = 256) -> Dict:
    """Host inputs of the sampler as bf16 bits: the model's layers around the
    blocks, the blocks' weights (blocks = (n_img, n_ref, n_txt, n_joint)
    counts), the latent z, text features of both prompts, one reference of
    n_ref_side^2 tokens (none when 0) and the joint positions."""
    D, F, C, T = width, mlp_hidden, latent_ch, text_dim
    key = (seed, TENSOR_SAMPLER)
    k = [0]

    def draw(shape, std):
        k[0] += 1
        return normal_bf16(shape, std, *key, k[0])

    m = {"img_in_w": draw((D, C), C ** -0.5), "img_in_b": draw((D,), 0.1),
         "ref_in_w": draw((D, C), C ** -0.5), "ref_in_b": draw((D,), 0.1),
         "txt_in_w": draw((D, T), T ** -0.5), "txt_in_b": draw((D,), 0.1),
         "t_w1": draw((D, time_dim), time_dim ** -0.5), "t_b1": draw((D,), 0.1),
         "t_w2": draw((D, D), D ** -0.5), "t_b2": draw((D,), 0.1),
         "mod_w": [draw((3 * D, D), (0.1 / D) ** 0.5) for _ in range(4)],
         "mod_b": [draw((3 * D,), 0.1) for _ in range(4)],
         "out_mod_w": draw((2 * D, D), (0.1 / D) ** 0.5), "out_mod_b": draw((2 * D,), 0.1),
         "out_w": draw((C, D), D ** -0.5), "out_b": draw((C,), 0.1)}
    one = f64_to_bf16_bits(np.ones(head_dim))
    m["blocks"] = [{"w_in": draw((3 * D + 2 * F, D), D ** -0.5),
                    "w_out": draw((D, D + F), (D + F) ** -0.5),
                    "q_scale": one.copy(), "k_scale": one.copy()} for _ in range(sum(blocks))]
    n_img, n_ref = n_img_side ** 2, n_ref_side ** 2
    streams = [Stream(STREAM_IMAGE, n_img, (n_img_side, n_img_side), 0.0)]
    if n_ref:
        streams.append(Stream(STREAM_REF, n_ref, (n_ref_side, n_ref_side), 0.0))
    streams.append(Stream(STREAM_TEXT, n_txt))
    return {"model": m, "z": draw((n_img, C), 1.0), "txt_cond": draw((n_txt, T), 1.0),
            "txt_neg": draw((n_txt, T), 1.0),
            "ref_latent": draw((n_ref, C), 1.0) if n_ref else None,
            "pos": positions(BlockConfig("sampler", 0, tuple(streams), width, n_heads, head_dim,
                                         mlp_hidden))}
