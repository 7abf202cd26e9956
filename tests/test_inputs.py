"""Seeded input generator and workload shapes (CPU only)."""
import numpy as np
import pytest
import torch

from flow_matching_diffusion_adaln_amd import configs, inputs


def test_bf16_round_to_nearest_even_hand_picked():
    cases = [
        (1.0, 0x3F80),
        (-2.0, 0xC000),
        (1.0 + 2 ** -8, 0x3F80),               # tie between 1 and 1+2^-7 -> even (1)
        (1.0 + 3 * 2 ** -8, 0x3F82),           # tie between 1+2^-7 and 1+2^-6 -> even
        (1.0 + 2 ** -8 + 2 ** -30, 0x3F81),    # just above the tie -> up
        (1.0 + 2 ** -8 - 2 ** -40, 0x3F80),    # just below the tie -> down
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (1.0 - 2 ** -9, 0x3F80),               # tie 1-2^-8 .. 1 -> even (1.0)
        (3.0e38, 0x7F62),
    ]
    got = inputs.f64_to_bf16_bits(np.array([c[0] for c in cases]))
    assert [int(g) for g in got] == [c[1] for c in cases]


def test_bf16_matches_torch_rne_on_float32_values():
    # torch's float32 -> bfloat16 cast rounds to nearest even; on values that
    # are exact in float32 the direct float64 rounding must agree with it
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    ours = inputs.f64_to_bf16_bits(a.astype(np.float64))
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_roundtrip_and_errors():
    bits = np.arange(0x3F00, 0x4100, dtype=np.uint16)
    back = inputs.f64_to_bf16_bits(inputs.bf16_bits_to_f32(bits).astype(np.float64))
    np.testing.assert_array_equal(back, bits)
    with pytest.raises(ValueError):
        inputs.f64_to_bf16_bits(np.array([np.inf]))
    with pytest.raises(ValueError):
        inputs.f64_to_bf16_bits(np.array([1e-40]))


def test_generator_is_deterministic_and_keyed():
    a = inputs.normal_bf16((64, 32), 1.0, 0, 1, 0, inputs.TENSOR_X)
    b = inputs.normal_bf16((64, 32), 1.0, 0, 1, 0, inputs.TENSOR_X)
    c = inputs.normal_bf16((64, 32), 1.0, 0, 1, 1, inputs.TENSOR_X)
    np.testing.assert_array_equal(a, b)
    assert np.mean(a != c) > 0.9


def test_block_inputs_shapes_and_distributions(block_inputs):
    cfg = configs.C1
    d = block_inputs("c1")
    D, F = cfg.width, cfg.mlp_hidden
    assert d["x"].shape == (336, D) and d["x"].dtype == np.uint16
    assert d["mod"].shape == (2, 3, D)
    assert d["w_in"].shape == (3 * D + 2 * F, D)
    assert d["w_out"].shape == (D, D + F)
    f = inputs.bf16_bits_to_f32
    assert abs(f(d["x"]).std() - 1.0) < 0.01
    assert abs(f(d["w_in"]).std() * np.sqrt(D) - 1.0) < 0.01
    assert abs(f(d["w_out"]).std() * np.sqrt(D + F) - 1.0) < 0.01
    assert abs(f(d["mod"]).std() - np.sqrt(0.1)) < 0.01
    assert np.all(f(d["q_scale"]) == 1) and np.all(f(d["k_scale"]) == 1)
    # the two streams' modulation vectors are different draws
    assert np.mean(d["mod"][0] != d["mod"][1]) > 0.9


def test_positions_layout():
    p = inputs.positions(configs.C1)
    assert p.shape == (336, 4) and p.dtype == np.int32
    # image: row-major 16x16 grid, t = l = 0
    assert list(p[0]) == [0, 0, 0, 0] and list(p[1]) == [0, 0, 1, 0]
    assert list(p[17]) == [0, 1, 1, 0] and list(p[255]) == [0, 15, 15, 0]
    # text: t = k, including padding positions
    assert list(p[256]) == [0, 0, 0, 0] and list(p[335]) == [79, 0, 0, 0]
    p4 = inputs.positions(configs.C4)
    # the reference shares (h, w) with the output image and takes l = 1
    np.testing.assert_array_equal(p4[4096:8192, 1:3], p4[:4096, 1:3])
    assert np.all(p4[4096:8192, 3] == 1) and np.all(p4[:4096, 3] == 0)
    assert list(p4[-1]) == [159, 0, 0, 0]


def test_workload_constants_from_the_pages():
    # "Welcome FLUX.3 Image Klein in Diffusers", "How it works": one token per
    # 16x16 pixels, so 1024^2 -> 4,096 tokens; prompts padded to multiples of 80;
    # RoPE axes take 32 of the 128 head dims each.
    assert configs.C2.streams[0].n == (1024 // 16) ** 2 == 4096
    assert all(s.n % 80 == 0 for c in configs.CONFIGS.values() for s in c.streams
               if s.kind == configs.STREAM_TEXT)
    assert configs.WIDTH == configs.N_HEADS * configs.HEAD_DIM == 3072
    assert 4 * 32 == configs.HEAD_DIM
    assert (configs.C5.n_stage1, configs.C5.n_joint) == (5, 28)
    assert configs.C2.N == 4256 and configs.C4.N == 8352 and configs.C1.N == 336


def test_flop_model():
    c2 = configs.C2
    assert c2.gemm_flop() == pytest.approx(1044.3e9, rel=1e-3)
    assert c2.attn_flop() == pytest.approx(222.6e9, rel=1e-3)
    assert configs.C4.flop() == pytest.approx(2906.5e9, rel=1e-3)
