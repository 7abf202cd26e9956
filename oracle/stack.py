"""Plain float64 CPU oracle for the two-stage DiT stack and the CFG pair.

TEST INFRASTRUCTURE ONLY, like the block oracle next to it: only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it.

What is computed (sources are the pages' sections):

* Two-stage transformer: "Welcome FLUX.3 Image Klein in Diffusers", section
  "How it works": each stream (text, image, reference) first runs through
  blocks of its own (own weights, attending only to itself), then the streams
  are concatenated and run through the shared joint blocks (5 own blocks per
  stream, then 28 joint blocks).
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
  branches share them; stage-1 blocks use the image rows' (resp. text rows')
  positions of the joint sequence.
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


def stack_branch(x_img, x_txt, pos, img_blocks: List[Dict], txt_blocks: List[Dict],
                 joint_blocks: List[Dict], dims: Dict) -> np.ndarray:
    """One forward of the two-stage stack: stage-1 image blocks on the image
    rows, stage-1 text blocks on the text rows, then the joint blocks over
    [image | text].  Returns the joint output [n_img + n_txt, D] (bf16 values)."""
    x_img = widen_bf16(x_img) if np.asarray(x_img).dtype == np.uint16 else np.asarray(x_img, np.float64)
    x_txt = widen_bf16(x_txt) if np.asarray(x_txt).dtype == np.uint16 else np.asarray(x_txt, np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    n_img, n_txt = x_img.shape[0], x_txt.shape[0]
    h_img = _run(x_img, img_blocks, pos[:n_img], [n_img], dims)
    h_txt = _run(x_txt, txt_blocks, pos[n_img:], [n_txt], dims)
    h = np.concatenate([h_img, h_txt], axis=0)
    return _run(h, joint_blocks, pos, [n_img, n_txt], dims)


def stack_cfg_ref(x_img, x_txt_cond, x_txt_neg, pos, img_blocks, txt_blocks, joint_blocks,
                  dims: Dict, cfg_scale: float) -> np.ndarray:
    """Guided image rows neg + s (cond - neg) of two stack forwards, rounded to
    bf16 like the GPU output.  cfg_scale == 1 runs the conditional branch only."""
    n_img = np.asarray(x_img).shape[0]
    cond = stack_branch(x_img, x_txt_cond, pos, img_blocks, txt_blocks, joint_blocks, dims)
    if cfg_scale == 1.0:
        return cond[:n_img]
    neg = stack_branch(x_img, x_txt_neg, pos, img_blocks, txt_blocks, joint_blocks, dims)
    return round_bf16(cfg_combine(cond[:n_img], neg[:n_img], cfg_scale))
