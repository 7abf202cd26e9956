"""Properties of the GPU path that hold exactly (bitwise) or at any size."""
import numpy as np
import pytest
import torch

import oracle
from flow_matching_diffusion_adaln_amd import configs, inputs, ops

from _gpu import block_config, require_gpu, run_block, to_dev, widen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


@pytest.fixture(scope="module")
def c1():
    d = inputs.make_block_inputs(configs.C1)
    return d, to_dev(d)


def bits(t):
    return t.view(torch.int16)


def test_zero_gate_returns_x_bitwise(c1):
    d, dv = c1
    dv = dict(dv)
    mod = dv["mod"].clone()
    mod[:, 2, :] = 0
    dv["mod"] = mod
    y = run_block(dv, configs.C1)
    assert torch.equal(bits(y), bits(dv["x"]))


def test_zero_gate_on_one_stream_only(c1):
    d, dv = c1
    dv = dict(dv)
    mod = dv["mod"].clone()
    mod[1, 2, :] = 0
    dv["mod"] = mod
    y = run_block(dv, configs.C1)
    assert torch.equal(bits(y[256:]), bits(dv["x"][256:]))
    assert not torch.equal(bits(y[:256]), bits(dv["x"][:256]))


def test_runs_are_bitwise_deterministic(c1):
    d, dv = c1
    a = run_block(dv, configs.C1).clone()
    b = run_block(dv, configs.C1)
    assert torch.equal(bits(a), bits(b))


def test_c2_runs_are_bitwise_deterministic():
    d = inputs.make_block_inputs(configs.C2)
    dv = to_dev(d)
    a = run_block(dv, configs.C2).clone()
    b = run_block(dv, configs.C2)
    assert torch.equal(bits(a), bits(b))


def test_in_place_output(c1):
    d, dv = c1
    ref = run_block(dv, configs.C1).clone()
    dv2 = dict(dv)
    dv2["x"] = dv["x"].clone()
    y = run_block(dv2, configs.C1, y=dv2["x"])
    assert y.data_ptr() == dv2["x"].data_ptr()
    assert torch.equal(bits(y), bits(ref))


def test_permuting_a_stream_permutes_outputs(c1):
    d, dv = c1
    perm = np.concatenate([np.random.default_rng(3).permutation(256), np.arange(256, 336)])
    dp = dict(d)
    dp["x"] = d["x"][perm]
    dp["pos"] = d["pos"][perm]
    y = widen(run_block(dv, configs.C1))
    yp = widen(run_block(to_dev(dp), configs.C1))
    # key order changes fp32 summation order inside attention only
    assert oracle.rel_l2(yp, y[perm]) <= 2e-3


def test_one_token_attention_returns_v():
    d = inputs.make_attn_inputs(1, 24, 128, seed=9)
    dv = to_dev(d)
    o = ops.attn_fwd(dv["q"], dv["k"], dv["v"])
    torch.cuda.synchronize()
    assert torch.equal(bits(o), bits(dv["v"]))


def test_identical_keys_give_mean_of_v():
    N = 200
    d = inputs.make_attn_inputs(N, 24, 128, seed=10)
    d["k"] = np.tile(d["k"][:1], (N, 1, 1))
    dv = to_dev(d)
    o = widen(ops.attn_fwd(dv["q"], dv["k"], dv["v"]))
    mean_v = oracle.widen_bf16(d["v"]).mean(axis=0, keepdims=True)
    assert oracle.rel_l2(o, np.tile(mean_v, (N, 1, 1))) <= 5e-3


def test_rope_zero_positions_without_norm_is_identity():
    N = 130
    q = inputs.normal_bf16((N, 24, 128), 1.0, 11, 0, 1)
    k = inputs.normal_bf16((N, 24, 128), 1.0, 11, 0, 2)
    qd, kd = ops.to_device_bf16(q), ops.to_device_bf16(k)
    ops.rope4_apply(qd, kd, torch.zeros((N, 4), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(ops.to_host_bits(qd), q) and np.array_equal(ops.to_host_bits(kd), k)


def test_rope_relative_positions_on_gpu():
    # q.k after RoPE depends only on position differences (up to bf16 rounding)
    N = 64
    q = inputs.normal_bf16((N, 24, 128), 1.0, 12, 0, 1)
    k = inputs.normal_bf16((N, 24, 128), 1.0, 12, 0, 2)
    rng = np.random.default_rng(0)
    pos = rng.integers(0, 60, size=(N, 4)).astype(np.int32)
    dots = []
    for shift in (0, 37):
        qd, kd = ops.to_device_bf16(q), ops.to_device_bf16(k)
        ops.rope4_apply(qd, kd, torch.from_numpy(pos + shift).cuda())
        torch.cuda.synchronize()
        a, b = widen(qd), widen(kd)
        dots.append(np.einsum("nhd,mhd->hnm", a, b))
    assert oracle.rel_l2(dots[1], dots[0]) <= 1e-2
