"""GPU tests of the FP8 projections (dit_quantize_rows_fp8, dit_block_fwd_fp8)
against the FP8 oracle (oracle/fp8.py), and of their distance from the bf16
block.

Bounds.
* The quantizer is integer work decided in float32 on both sides: codes and
  scales must match bit for bit.
* The FP8 block against the FP8 oracle: y (residual-dominated) keeps the
  block's 1e-2.  The branch r gets its own bound.  The GPU quantizes its own
  bf16 u and [o | m], which differ from the oracle's float64 values by the
  bf16 path's error (relative RMS delta of a few 1e-3).  Such a difference
  moves a value across an e4m3 rounding boundary with probability about
  delta / s, where s is the relative code spacing (2^-4 .. 2^-3), and each
  crossing costs one spacing.  The RMS effect is therefore sqrt(delta * s):
  about 1.5e-2 at delta = 3e-3 and s = 0.09.  The bound is twice that,
  3e-2.
* The FP8 block against the bf16 oracle: e4m3 keeps 3 mantissa bits, so each
  quantized operand carries a relative RMS error of about 2^-4 / sqrt(3) of
  its scale-relative size.  Two operands per product and two products in
  series give a few percent on r; the bound is 0.1.
"""
import numpy as np
import pytest
import torch

import oracle
from _gpu import block_config, require_gpu, sample_rows, to_dev, widen
from flow_matching_diffusion_adaln_amd import configs, inputs, ops

pytestmark = pytest.mark.gpu

TOL_Y = 1e-2
TOL_R_F8 = 3e-2
TOL_R_VS_BF16 = 0.1


def log(msg):
    print(msg, flush=True)


def test_quantize_rows_bit_exact():
    require_gpu()
    rng = np.random.default_rng(5)
    x = rng.standard_normal((37, 3072)) * 2.0 ** rng.integers(-20, 20, size=(37, 1))
    x[3] = 0.0                       # all-zero row
    x[4] = 1e-30 * rng.standard_normal(3072)   # tiny row (subnormal codes)
    x[5, :] = 0.0
    x[5, 7] = -2.5                   # one non-zero element
    x[6] = np.where(rng.random(3072) < 0.5, 1.0, -1.0) * 3.0   # constant magnitude
    xb = inputs.f64_to_bf16_bits(x)
    cases = [("structured 37 x 3072", xb),
             ("c1 w_out 3072 x 12288", inputs.make_block_inputs(configs.C1, seed=0)["w_out"]),
             ("activations 333 x 12288", inputs.normal_bf16((333, 12288), 0.5, 9, 1))]
    for name, bits in cases:
        log(f"quantize {name}")
        q, s = ops.quantize_rows_fp8(ops.to_device_bf16(bits))
        torch.cuda.synchronize()
        qo, so = oracle.quantize_rows(bits)
        gq, gs = q.cpu().numpy(), s.cpu().numpy()
        bad = int((gq != qo).sum())
        log(f"  code mismatches {bad} of {qo.size}; scale mismatches "
            f"{int((gs.view(np.uint32) != so.view(np.uint32)).sum())}")
        assert bad == 0
        assert np.array_equal(gs.view(np.uint32), so.view(np.uint32))


_WQ = {}


def run_fp8(cfg, d, flags=0):
    dv = to_dev(d)
    key = (cfg.name, cfg.config_id)
    if key not in _WQ:
        _WQ[key] = (ops.quantize_rows_fp8(dv["w_in"]), ops.quantize_rows_fp8(dv["w_out"]))
    (wi, si), (wo, so) = _WQ[key]
    desc = ops.make_desc(cfg.n_tokens, cfg.width, cfg.n_heads, cfg.head_dim, cfg.mlp_hidden,
                         flags=flags)
    y = ops.block_fwd_fp8(dv["x"], dv["mod"], dv["pos"], wi, si, wo, so, dv["q_scale"],
                          dv["k_scale"], desc)
    torch.cuda.synchronize()
    return widen(y)


def check_fp8(cfg, d, rows=None, vs_bf16=True):
    y = run_fp8(cfg, d)
    r = run_fp8(cfg, d, ops.DIT_F_NO_RESIDUAL | ops.DIT_F_NO_GATE)
    args = (d["x"], d["mod"], d["pos"], d["w_in"], d["w_out"], d["q_scale"], d["k_scale"],
            cfg.n_tokens, cfg.n_heads, cfg.head_dim, cfg.mlp_hidden, configs.ROPE_THETA,
            configs.LN_EPS, configs.QK_EPS)
    wq = (oracle.quantize_rows(d["w_in"]), oracle.quantize_rows(d["w_out"]))
    ref = oracle.block_ref_fp8(*args, rows=rows, w_in_q=wq[0], w_out_q=wq[1])
    if rows is not None:
        y, r = y[rows], r[rows]
    ey, er = oracle.rel_l2(y, ref["y"]), oracle.rel_l2(r, ref["r"])
    msg = f"  relL2 vs fp8 oracle y={ey:.3e} r={er:.3e}"
    if vs_bf16:
        ref16 = oracle.block_ref(*args, flags=0, rows=rows)
        eb = oracle.rel_l2(r, ref16["r"])
        msg += f"; r vs bf16 oracle {eb:.3e}"
        assert eb <= TOL_R_VS_BF16
    log(msg)
    assert ey <= TOL_Y and er <= TOL_R_F8


def test_fp8_block_c1_full():
    require_gpu()
    cfg = configs.C1
    log(f"fp8 block c1 N={cfg.N}")
    check_fp8(cfg, inputs.make_block_inputs(cfg, seed=0))


def test_fp8_block_ragged_three_streams():
    require_gpu()
    cfg = block_config("ragged3", (200, 57, 80), 41)
    log(f"fp8 block ragged N={cfg.N}")
    check_fp8(cfg, inputs.make_block_inputs(cfg, seed=1))


@pytest.mark.parametrize("n_tokens,cid", [((4096, 160), 2), ((513,), 43), ((5441, 160), 44)])
def test_fp8_block_sampled(n_tokens, cid):
    # c2, and sizes whose last round of tiles is split along K
    require_gpu()
    cfg = configs.C2 if cid == 2 else block_config(f"f8_{cid}", n_tokens, cid)
    rows = sample_rows(cfg, n_random=24)
    log(f"fp8 block N={cfg.N} rows={len(rows)}")
    check_fp8(cfg, inputs.make_block_inputs(cfg, seed=2), rows=rows, vs_bf16=cid == 2)


def test_fp8_block_narrow_width():
    # width 2,048: K = 2,048 and 8,192 bytes are 16 and 64 k tiles, not
    # multiples of 6, so both FP8 GEMMs run their 2-slot A ring
    require_gpu()
    cfg = block_config("f8w2048", (700, 80), 45, width=2048, n_heads=16, mlp_hidden=6144)
    rows = sample_rows(cfg, n_random=24)
    log(f"fp8 block width 2048 N={cfg.N} rows={len(rows)}")
    check_fp8(cfg, inputs.make_block_inputs(cfg, seed=4), rows=rows, vs_bf16=False)


def test_fp8_block_qk_scales():
    # non-unit QK-norm scales through the FP8 input projection's epilogue
    require_gpu()
    cfg = configs.C1
    d = inputs.make_block_inputs(cfg, seed=5)
    g = oracle.widen_bf16(inputs.normal_bf16((2, cfg.head_dim), 0.2, 5, 77, 1))
    d["q_scale"] = inputs.f64_to_bf16_bits(3.0 * (1.0 + g[0]))
    d["k_scale"] = inputs.f64_to_bf16_bits(1.0 + g[1])
    _WQ.pop((cfg.name, cfg.config_id), None)
    log("fp8 block c1 with qk scales")
    check_fp8(cfg, d, vs_bf16=False)


def test_fp8_zero_gate_returns_x():
    require_gpu()
    cfg = configs.C1
    d = inputs.make_block_inputs(cfg, seed=3)
    d["mod"] = d["mod"].copy()
    d["mod"][:, 2, :] = 0
    y = run_fp8(cfg, d)
    assert np.array_equal(y, oracle.widen_bf16(d["x"]))
