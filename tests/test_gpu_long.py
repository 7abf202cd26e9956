"""Long and multi-reference sequences: several references packed in the
reference segment (each with its own l index), a 2048^2 joint sequence, and
attention at the longest editing length the pages describe."""
import numpy as np
import pytest
import torch

import oracle
from _gpu import oracle_block, require_gpu, run_block, sample_rows, to_dev, widen
from flow_matching_diffusion_adaln_amd import configs, inputs, ops

pytestmark = pytest.mark.gpu
TOL_BLOCK = 1e-2
TOL_ATTN = 5e-3


def log(msg):
    print(msg, flush=True)


def check(cfg, d, rows=None):
    dv = to_dev(d)
    y = widen(run_block(dv, cfg))
    r = widen(run_block(dv, cfg, flags=ops.DIT_F_NO_RESIDUAL | ops.DIT_F_NO_GATE))
    ref = oracle_block(d, cfg, rows=rows)
    if rows is not None:
        y, r = y[rows], r[rows]
    ey, er = oracle.rel_l2(y, ref["y"]), oracle.rel_l2(r, ref["r"])
    log(f"  relL2 y={ey:.3e} r={er:.3e}")
    assert ey <= TOL_BLOCK and er <= TOL_BLOCK


def test_three_references_in_one_segment():
    # image 16x16 | references 3 x (8x8) with l = 1, 2, 3 | 40 text tokens.
    # References share the t = 0 modulation, so they form one segment whose
    # rows carry their own (h, w, l) positions.
    require_gpu()
    n_ref = 3 * 64
    cfg = configs.BlockConfig("multiref", 90, (configs.Stream("image", 256, (16, 16), 0.7),
                                               configs.Stream("reference", n_ref, (1, n_ref), 0.0),
                                               configs.Stream("text", 40)))
    d = inputs.make_block_inputs(cfg, seed=5)
    pos = d["pos"].copy()
    for r in range(3):
        i = np.arange(64)
        rows = 256 + 64 * r + i
        pos[rows, 0] = 0
        pos[rows, 1] = i // 8
        pos[rows, 2] = i % 8
        pos[rows, 3] = r + 1
    d["pos"] = pos
    log(f"block multiref N={cfg.N}")
    check(cfg, d)


def test_block_2048sq_sampled():
    # 2048^2 image: a 128 x 128 latent grid (16,384 tokens) + 160 text tokens
    require_gpu()
    cfg = configs.BlockConfig("2048sq", 91, (configs.Stream("image", 16384, (128, 128), 0.7),
                                             configs.Stream("text", 160)))
    d = inputs.make_block_inputs(cfg, seed=6)
    rows = sample_rows(cfg, n_random=24)
    log(f"block 2048^2 N={cfg.N} rows={len(rows)}")
    check(cfg, d, rows)


def test_attention_45k_sampled():
    # the longest editing sequences the pages describe, about 45k tokens
    require_gpu()
    N, H, dd = 45056, 24, 128
    a = inputs.make_attn_inputs(N, H, dd, seed=7, logit_std=2.0, case=9)
    dv = to_dev(a)
    o = ops.attn_fwd(dv["q"], dv["k"], dv["v"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 40, replace=False)]))
    q, k, v = (oracle.widen_bf16(a[n]) for n in ("q", "k", "v"))
    want = oracle.attention_ref(q[rows], k, v, 1.0 / np.sqrt(dd))
    got = widen(o)[rows]
    e = oracle.rel_l2(got, want)
    log(f"attention N={N} sampled rows={len(rows)} relL2 {e:.3e}")
    assert e <= TOL_ATTN


def test_block_edit2048_sampled():
    # the long edit the bench times: 2048^2 image (16,384 tokens) | one
    # 2048^2 reference sharing its (h, w) with l = 1 (16,384) | 160 text,
    # 32,928 tokens in three streams; attention is then 62% of the FLOPs and
    # its balanced split cuts many items
    require_gpu()
    cfg = configs.EDIT_2048
    d = inputs.make_block_inputs(cfg, seed=8)
    rows = sample_rows(cfg, n_random=24)
    log(f"block {cfg.name} N={cfg.N} rows={len(rows)}")
    check(cfg, d, rows)
