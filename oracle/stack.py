"""Plain float64 CPU oracle for the two-stage DiT stack and the CFG pair.

TEST INFRASTRUCTURE ONLY, like the block oracle next to it: only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it.

What is computed (sources are the pages' sections):

* Two-stage transformer: "Welcome FLUX.3 Image Klein in Diffusers", section
  "How it works": each stream (text, image, reference) first runs through
  blocks of its own (own weights, attending only to itself), then the streams
  are concatenated in [image | reference | text] order and run through the
  shared joint blocks (5 own blocks per stream, then 28 joint blocks).
* Classifier-free guidance: the miles page "FLUX 3 Image Klein", section 3
  "Family config": the guided prediction is neg + scale * (pos - neg), from
  one forward with the prompt and one with the negative prompt; a scale of 1
  runs the conditional branch only.

Readings taken where the pages are silent:
  the image tokens enter the stack as given (embedders are out of scope) and
  the guided combination is taken on the image-token rows of the joint stack's
  output (the output layers, also out of scope, act on image tokens only);
  activations are bf16 between blocks (the model runs in bf16), rounded to
  nearest even; the stage-1 image blocks do not depend on the text, so both
  branches share them, as they share the reference blocks; stage-1 blocks use
  their own rows of the joint sequence's position table; all reference images
  together form the one reference stream (each keeps its own l index in the
  positions) and run the reference blocks as one sequence.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np

from .dit_block import block_ref, widen_bf16


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as float64.

    The float64 significand is rounded to bf16's 8 bits directly on the bit
    pattern (a float32 detour would round twice): keep the sign, exponent and
    top 7 stored mantissa bits and round on the other 45.  Exact for values in
    bf16's normal range, which is where block activations live.
    """
    a = np.asarray(a, dtype=np.float64)
    bits = a.view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    rounded = (bits + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    out = rounded.view(np.float64)
    # values whose bf16 exponent overflows become inf, as in the bf16 store
    return np.where(np.abs(out) > 3.3895313892515355e38, np.copysign(np.inf, a), out)


def cfg_combine(cond: np.ndarray, neg: np.ndarray, scale: float) -> np.ndarray:
    """Guided prediction neg + scale * (cond - neg) (the miles page, section 3)."""
    cond = np.asarray(cond, dtype=np.float64)
    neg = np.asarray(neg, dtype=np.float64)
    return neg + scale * (cond - neg)


def _run(h: np.ndarray, blocks: Sequence[Dict], pos: np.ndarray, n_tokens: Sequence[int],
         dims: Dict) -> np.ndarray:
    for b in blocks:
        y = block_ref(h, b["mod"], pos, b["w_in"], b["w_out"], b["q_scale"], b["k_scale"],
                      n_tokens, dims["n_heads"], dims["head_dim"], dims["mlp_hidden"],
                      dims.get("theta", 10000.0), dims.get("ln_eps", 1e-6),
                      dims.get("qk_eps", 1e-6))["y"]
        h = round_bf16(y)
    return h


def _bits_or_float(a) -> np.ndarray:
    a = np.asarray(a)
    return widen_bf16(a) if a.dtype == np.uint16 else a.astype(np.float64)


def stack_branch(x_img, x_txt, pos, img_blocks: List[Dict], txt_blocks: List[Dict],
                 joint_blocks: List[Dict], dims: Dict, x_ref=None,
                 ref_blocks: Sequence[Dict] = ()) -> np.ndarray:
    """One forward of the two-stage stack: stage-1 image blocks on the image
    rows, stage-1 reference blocks on the reference rows (when there are
    references), stage-1 text blocks on the text rows, then the joint blocks
    over [image | reference | text].  Returns the joint output [N, D] (bf16
    values)."""
    x_img, x_txt = _bits_or_float(x_img), _bits_or_float(x_txt)
    pos = np.asarray(pos, dtype=np.int64)
    n_img, n_txt = x_img.shape[0], x_txt.shape[0]
    parts, n_tokens = [_run(x_img, img_blocks, pos[:n_img], [n_img], dims)], [n_img]
    if x_ref is not None and np.asarray(x_ref).shape[0] > 0:
        x_ref = _bits_or_float(x_ref)
        n_ref = x_ref.shape[0]
        parts.append(_run(x_ref, ref_blocks, pos[n_img:n_img + n_ref], [n_ref], dims))
        n_tokens.append(n_ref)
    elif len(ref_blocks):
        raise ValueError("reference blocks without reference tokens")
    n_pre = sum(n_tokens)
    parts.append(_run(x_txt, txt_blocks, pos[n_pre:], [n_txt], dims))
    n_tokens.append(n_txt)
    if pos.shape[0] != n_pre + n_txt:
        raise ValueError("pos does not cover [image | reference | text]")
    return _run(np.concatenate(parts, axis=0), joint_blocks, pos, n_tokens, dims)


def stack_cfg_ref(x_img, x_txt_cond, x_txt_neg, pos, img_blocks, txt_blocks, joint_blocks,
                  dims: Dict, cfg_scale: float, x_ref=None, ref_blocks: Sequence[Dict] = ()
                  ) -> np.ndarray:
    """Guided image rows neg + s (cond - neg) of two stack forwards, rounded to
    bf16 like the GPU output.  cfg_scale == 1 runs the conditional branch only."""
    n_img = np.asarray(x_img).shape[0]
    cond = stack_branch(x_img, x_txt_cond, pos, img_blocks, txt_blocks, joint_blocks, dims,
                        x_ref, ref_blocks)
    if cfg_scale == 1.0:
        return cond[:n_img]
    neg = stack_branch(x_img, x_txt_neg, pos, img_blocks, txt_blocks, joint_blocks, dims,
                       x_ref, ref_blocks)
    return round_bf16(cfg_combine(cond[:n_img], neg[:n_img], cfg_scale))
