"""GPU parity of every C-ABI entry point against the fp64 oracle.

Bounds.  The full block and attention bounds are the targets stated for this
path: relative L2 <= 1e-2 for the block output y and for its branch r, and
<= 5e-3 for attention alone.  AdaLN and RoPE have no stated bound; their only
error is the final round to bf16 (at most 2^-8 relative per element: half an
ulp of an 8-bit significand) plus fp32 arithmetic (~1e-6), so they are held
to 2^-8 + 1e-5 relative L2, which no mix of per-element errors within those
bounds can exceed.
Inputs are the seeded bf16 tensors shared with the oracle; sizes span several
tiles and ragged tails, and the full-size configurations are checked on
sampled rows the oracle evaluates one by one.
"""
import numpy as np
import pytest
import torch

import oracle
from flow_matching_diffusion_adaln_amd import configs, inputs, ops

from _gpu import (block_config, oracle_block, require_gpu, run_block, sample_rows, to_dev,
                  widen)

pytestmark = pytest.mark.gpu

TOL_BLOCK = 1e-2
TOL_ATTN = 5e-3
TOL_ROUND = 2.0 ** -8 + 1e-5


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------- adaln_mod ----

@pytest.mark.parametrize("n_tokens", [(256, 80), (200, 57, 80), (1,), (4096, 160)])
def test_adaln_parity(n_tokens):
    cfg = block_config("adaln", n_tokens, 60 + len(n_tokens))
    d = inputs.make_block_inputs(cfg, seed=1, weights=False)
    dv = to_dev(d)
    log(f"adaln n_tokens={n_tokens}")
    out = ops.adaln_mod(dv["x"], dv["mod"], n_tokens)
    torch.cuda.synchronize()
    ref = oracle.adaln_ref(oracle.widen_bf16(d["x"]), oracle.widen_bf16(d["mod"]), n_tokens,
                           configs.LN_EPS)
    got = widen(out)
    assert oracle.rel_l2(got, ref) <= TOL_ROUND
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)


def test_adaln_in_place():
    cfg = block_config("adaln", (300, 80), 70)
    d = inputs.make_block_inputs(cfg, seed=2, weights=False)
    dv = to_dev(d)
    ref = ops.adaln_mod(dv["x"], dv["mod"], cfg.n_tokens)
    x2 = dv["x"].clone()
    ops.adaln_mod(x2, dv["mod"], cfg.n_tokens, out=x2)
    torch.cuda.synchronize()
    assert torch.equal(x2.view(torch.int16), ref.view(torch.int16))


# ------------------------------------------------------------ rope4_apply ----

@pytest.mark.parametrize("n_tokens,norm", [((256, 80), True), ((200, 57, 80), True),
                                           ((256, 80), False), ((4096, 160), True)])
def test_rope4_parity(n_tokens, norm):
    cfg = block_config("rope", n_tokens, 80 + len(n_tokens))
    pos = inputs.positions(cfg)
    N, H, dh = cfg.N, cfg.n_heads, cfg.head_dim
    q = inputs.normal_bf16((N, H, dh), 1.5, 3, N, 1)
    k = inputs.normal_bf16((N, H, dh), 0.7, 3, N, 2)
    g = inputs.normal_bf16((2, dh), 0.2, 3, N, 3)
    g = inputs.f64_to_bf16_bits(1.0 + oracle.widen_bf16(g))
    log(f"rope4 n_tokens={n_tokens} norm={norm}")
    qd, kd = ops.to_device_bf16(q), ops.to_device_bf16(k)
    gq, gk = (ops.to_device_bf16(g[0]), ops.to_device_bf16(g[1])) if norm else (None, None)
    ops.rope4_apply(qd, kd, torch.from_numpy(pos).cuda(), configs.ROPE_THETA, gq, gk)
    torch.cuda.synchronize()
    for src, dev, gs in ((q, qd, g[0]), (k, kd, g[1])):
        x = oracle.widen_bf16(src)
        if norm:
            x = oracle.head_rms_norm(x, oracle.widen_bf16(gs), configs.QK_EPS)
        ref = oracle.rope4_ref(x, pos, configs.ROPE_THETA)
        got = widen(dev)
        assert oracle.rel_l2(got, ref) <= TOL_ROUND
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)


# ----------------------------------------------------------- dit_attn_fwd ----

@pytest.mark.parametrize("N,logit_std", [(1, 1.0), (63, 1.0), (64, 1.0), (65, 4.0), (336, 1.0),
                                         (337, 8.0), (1000, 2.0)])
def test_attn_parity_full(N, logit_std):
    d = inputs.make_attn_inputs(N, 24, 128, seed=5, logit_std=logit_std)
    log(f"attn N={N} logit_std={logit_std}")
    dv = to_dev(d)
    o = ops.attn_fwd(dv["q"], dv["k"], dv["v"])
    torch.cuda.synchronize()
    q, k, v = (oracle.widen_bf16(d[n]) for n in ("q", "k", "v"))
    ref = oracle.attention_ref(q, k, v, 128 ** -0.5)
    assert oracle.rel_l2(widen(o), ref) <= TOL_ATTN


@pytest.mark.parametrize("N,logit_std", [(4256, 1.0), (4256, 6.0), (8352, 2.0)])
def test_attn_parity_sampled(N, logit_std):
    d = inputs.make_attn_inputs(N, 24, 128, seed=6, logit_std=logit_std)
    log(f"attn sampled N={N} logit_std={logit_std}")
    dv = to_dev(d)
    o = ops.attn_fwd(dv["q"], dv["k"], dv["v"])
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 127, 128, N - 1, N - 2],
                                     np.random.default_rng(1).choice(N, 58, replace=False)]))
    q, k, v = (oracle.widen_bf16(d[n]) for n in ("q", "k", "v"))
    ref = oracle.attention_ref(q[rows], k, v, 128 ** -0.5)
    assert oracle.rel_l2(widen(o)[rows], ref) <= TOL_ATTN


# dit_attn_fwd_ws splits the work into one equal share of key tiles per CU
# when there are more (head, 256-query) items than CUs; an item cut between
# two shares is merged from two fp32 partials by whichever share ends last.
# On a 256-CU device: 3,000 tokens x 24 heads = 288 items (almost every item
# cut, checked on every row), 4,256 x 24 = 408 items (the block's shape),
# 8,352 x 24 = 792, and 16,484 tokens x 4 heads = 260 items of 258 key tiles
# against shares of 262 (every share holds the tail of one item and the head
# of the next).  With at least two rounds of items the kernel first runs whole
# items round by round: 8,352 x 24 (two whole rounds, then 280 items in
# shares) and 2,100 tokens x 64 heads = 576 items (one whole round, then 320
# items in 256 shares, checked on every row).  logit_std 1 to 8 runs the
# running-max merge with references far apart.
@pytest.mark.parametrize("N,H,logit_std,all_rows", [(3000, 24, 2.0, True), (4256, 24, 1.0, False),
                                                    (4256, 24, 8.0, False),
                                                    (8352, 24, 2.0, False),
                                                    (2100, 64, 2.0, True),
                                                    (16484, 4, 4.0, False)])
def test_attn_ws_split_parity(N, H, logit_std, all_rows):
    d = inputs.make_attn_inputs(N, H, 128, seed=8, logit_std=logit_std)
    log(f"attn_ws N={N} H={H} logit_std={logit_std}")
    dv = to_dev(d)
    # output and workspace start as NaN patterns, so a cut item that nobody
    # finished shows up
    ws = torch.full((ops.attn_workspace_bytes(N, H),), 0xFF, dtype=torch.uint8, device="cuda")
    o = ops.attn_fwd_ws(dv["q"], dv["k"], dv["v"], o=torch.full_like(dv["q"], float("nan")),
                        workspace=ws)
    torch.cuda.synchronize()
    if all_rows:
        rows = np.arange(N)
    else:
        rows = np.unique(np.concatenate([[0, 1, 255, 256, N - 1, N - 2],
                                         np.random.default_rng(2).choice(N, 90, replace=False)]))
    q, k, v = (oracle.widen_bf16(d[n]) for n in ("q", "k", "v"))
    ref = oracle.attention_ref(q[rows], k, v, 128 ** -0.5)
    e = oracle.rel_l2(widen(o)[rows], ref)
    log(f"  relL2 {e:.3e}")
    assert e <= TOL_ATTN
    # the merge is symmetric in the two parts: a second run is bitwise equal
    o2 = ops.attn_fwd_ws(dv["q"], dv["k"], dv["v"], o=torch.full_like(dv["q"], float("nan")),
                         workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))


def test_attn_softmax_scale_argument():
    N = 300
    d = inputs.make_attn_inputs(N, 24, 128, seed=7)
    dv = to_dev(d)
    o = ops.attn_fwd(dv["q"], dv["k"], dv["v"], softmax_scale=0.3)
    torch.cuda.synchronize()
    q, k, v = (oracle.widen_bf16(d[n]) for n in ("q", "k", "v"))
    assert oracle.rel_l2(widen(o), oracle.attention_ref(q, k, v, 0.3)) <= TOL_ATTN


# ---------------------------------------------------------- dit_block_fwd ----

def qk_scales(d, seed, gq=3.0):
    """Per-dim QK-norm scales: q around gq (peaked logits), k around 1."""
    dh = d["q_scale"].shape[0]
    g = oracle.widen_bf16(inputs.normal_bf16((2, dh), 0.2, seed, 77, 1))
    d["q_scale"] = inputs.f64_to_bf16_bits(gq * (1.0 + g[0]))
    d["k_scale"] = inputs.f64_to_bf16_bits(1.0 + g[1])
    return d


def check_block(cfg, seed=0, rows=None, scaled=False):
    d = inputs.make_block_inputs(cfg, seed=seed)
    if scaled:
        d = qk_scales(d, seed)
    log(f"block {cfg.name} N={cfg.N} rows={'all' if rows is None else len(rows)}"
        f"{' qk scales' if scaled else ''}")
    dv = to_dev(d)
    y = widen(run_block(dv, cfg))
    r = widen(run_block(dv, cfg, flags=ops.DIT_F_NO_RESIDUAL | ops.DIT_F_NO_GATE))
    ref = oracle_block(d, cfg, rows=rows)
    if rows is not None:
        y, r = y[rows], r[rows]
    ey, er = oracle.rel_l2(y, ref["y"]), oracle.rel_l2(r, ref["r"])
    log(f"  relL2 y={ey:.3e} r={er:.3e}")
    assert ey <= TOL_BLOCK and er <= TOL_BLOCK
    return ey, er


def test_block_parity_c1_full():
    check_block(configs.C1)


def test_block_parity_qk_scales():
    # learnable QK-norm scales away from one (q around 3: peaked logits) go
    # through the fused norm + RoPE epilogue of the input projection
    check_block(configs.C1, seed=4, scaled=True)
    check_block(configs.C2, seed=4, rows=sample_rows(configs.C2, n_random=24), scaled=True)


@pytest.mark.parametrize("g", [1.546875, 1.5625])
def test_block_parity_score_bound_edges(g):
    # constant QK-norm scales g: attention's score bound c 128 g^2 (1.01) is
    # 39.5, just under the 40 that lets the kernel use a fixed softmax
    # reference (weights then down to about 2^-30), or 40.3, just over it
    # (running max).  Both must match the oracle.
    cfg = configs.C1
    d = inputs.make_block_inputs(cfg, seed=6)
    d["q_scale"] = inputs.f64_to_bf16_bits(np.full(cfg.head_dim, g))
    d["k_scale"] = inputs.f64_to_bf16_bits(np.full(cfg.head_dim, g))
    log(f"block c1 with constant qk scales {g}")
    dv = to_dev(d)
    y = widen(run_block(dv, cfg))
    r = widen(run_block(dv, cfg, flags=ops.DIT_F_NO_RESIDUAL | ops.DIT_F_NO_GATE))
    ref = oracle_block(d, cfg)
    ey, er = oracle.rel_l2(y, ref["y"]), oracle.rel_l2(r, ref["r"])
    log(f"  relL2 y={ey:.3e} r={er:.3e}")
    assert ey <= TOL_BLOCK and er <= TOL_BLOCK


def test_block_parity_ragged_three_streams():
    # 337 tokens: not a multiple of 64, 128 or 256, with all three streams
    check_block(block_config("ragged3", (200, 57, 80), 91))


def test_block_parity_single_token():
    check_block(block_config("one", (1,), 92))


# At most 160 tokens the projections stream their weights: a workgroup per
# 128 weight rows with every token in the other MFMA operand (4 blocks of 32
# at 128 tokens, 5 at 160, a last block only partly inside M at 97 and 129),
# the output projection's K cut into pieces merged by the last to arrive, and
# two streams (100 image + 28 text) for the per-stream gate.
@pytest.mark.parametrize("n_tokens,cid", [((128,), 97), ((97,), 98), ((100, 28), 99),
                                          ((160,), 104), ((129,), 105)])
def test_block_parity_short_128_row_tiles(n_tokens, cid):
    check_block(block_config(f"short{sum(n_tokens)}", n_tokens, cid))


def test_block_parity_short_qk_scales():
    # QK-norm scales away from one through the short-sequence input
    # projection's norm + RoPE epilogue (the head's sum of squares meets
    # across its four waves in LDS)
    check_block(block_config("short80s", (80,), 102), seed=5, scaled=True)


# The short-sequence projections at width 2,048 (16 heads) with SwiGLU 6,144
# (K of 2,048 and 8,192, whole numbers of the 4-stage ring's 256 columns),
# and with SwiGLU 6,016, whose output-projection K = 8,064 is not, so the
# block takes the tiled GEMMs with every tile split along K and the separate
# norm + RoPE pass.
@pytest.mark.parametrize("width,heads,mlp,cid", [(2048, 16, 6144, 100), (2048, 16, 6016, 101)])
def test_block_parity_short_other_widths(width, heads, mlp, cid):
    cfg = block_config(f"short_w{width}", (80,), cid, width=width, n_heads=heads,
                       mlp_hidden=mlp)
    check_block(cfg)


# On a 256-CU device these token counts make the GEMMs cut their last, partly
# filled round of tiles along K (fp32 partial tiles + a fix-up pass):
#   513:   input projection (3 x 108 tiles of 256 rows), 1 round + 68 tiles
#   700:   input projection, likewise 1 round + 68 tiles
#   4,256: input projection, 256-row tiles, 7 rounds + 44 tiles (the 1024^2
#          workload, covered by the c2 tests)
#   5,601: both projections, 256-row tiles (output: 1 round + 8 tiles)
#   6,000: both projections, 256-row tiles (output: 1 round + 32 tiles)
@pytest.mark.parametrize("n_tokens,cid", [((449, 64), 93), ((620, 80), 94)])
def test_block_parity_split_tail_small(n_tokens, cid):
    check_block(block_config(f"split{sum(n_tokens)}", n_tokens, cid))


@pytest.mark.parametrize("n_tokens,cid", [((5441, 160), 95), ((5840, 160), 96)])
def test_block_parity_split_tail_both_gemms(n_tokens, cid):
    cfg = block_config(f"split{sum(n_tokens)}", n_tokens, cid)
    check_block(cfg, rows=sample_rows(cfg, n_random=32))


def test_block_parity_narrow_width():
    # width 2,048 (16 heads), SwiGLU 6,144: K = 2,048 and 8,192 are not
    # multiples of 6 k tiles of 64, so both GEMMs run their 2-slot A ring
    cfg = block_config("w2048", (700, 80), 97, width=2048, n_heads=16, mlp_hidden=6144)
    check_block(cfg, rows=sample_rows(cfg, n_random=32))


def test_block_parity_c2_sampled():
    check_block(configs.C2, rows=sample_rows(configs.C2))


def test_block_parity_c3_stage1():
    check_block(configs.C3_TXT)
    check_block(configs.C3_IMG, rows=sample_rows(configs.C3_IMG, n_random=32))


def test_block_parity_c4_sampled():
    check_block(configs.C4, rows=sample_rows(configs.C4, n_random=32))
