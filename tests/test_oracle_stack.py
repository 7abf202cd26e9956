"""Pins of the stack / CFG oracle (oracle/stack.py) against facts that do not
come from the oracle itself: a comparison-based bf16 rounding, the guidance
formula's closed form, and properties the two-stage structure implies."""
import numpy as np
import pytest

import oracle

DIMS = dict(n_heads=2, head_dim=8, mlp_hidden=24)
D = 16


def nearest_bf16_bruteforce(x: float) -> float:
    """Nearest bf16 by comparing the two bracketing bf16 values (ties to the
    one whose last kept mantissa bit is 0)."""
    b = np.array([x], dtype=np.float64).view(np.uint64)[0]
    lo_bits = b & ~np.uint64((1 << 45) - 1)
    lo = np.array([lo_bits], dtype=np.uint64).view(np.float64)[0]
    hi = np.array([lo_bits + np.uint64(1 << 45)], dtype=np.uint64).view(np.float64)[0]
    dlo, dhi = abs(x - lo), abs(hi - x)
    if dlo < dhi:
        return lo
    if dhi < dlo:
        return hi
    return lo if ((int(lo_bits) >> 45) & 1) == 0 else hi


def test_round_bf16_matches_bruteforce():
    rng = np.random.default_rng(5)
    xs = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-6, 6, 3000),
                         rng.standard_normal(200)])
    got = oracle.round_bf16(xs)
    want = np.array([nearest_bf16_bruteforce(float(x)) for x in xs])
    assert np.array_equal(got, want)


def test_round_bf16_ties_to_even_and_idempotent():
    one = 1.0
    ulp = 2.0 ** -7
    # 1 + ulp/2 is a tie between 1 (even) and 1 + ulp (odd): rounds to 1
    assert oracle.round_bf16(np.array([one + ulp / 2]))[0] == one
    # 1 + 3 ulp/2 is a tie between 1 + ulp (odd) and 1 + 2 ulp (even)
    assert oracle.round_bf16(np.array([one + 1.5 * ulp]))[0] == one + 2 * ulp
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # the NaN patterns among them
        vals = oracle.widen_bf16(bits)
    vals = vals[np.isfinite(vals)]
    assert np.array_equal(oracle.round_bf16(vals), vals)


def test_cfg_combine_closed_form():
    cond, neg = np.array([3.0, -1.0]), np.array([1.0, 2.0])
    assert np.allclose(oracle.cfg_combine(cond, neg, 4.0), [9.0, -10.0])
    assert np.array_equal(oracle.cfg_combine(cond, neg, 1.0), cond)
    assert np.array_equal(oracle.cfg_combine(cond, neg, 0.0), neg)


def _block(seed, n_streams, zero_gate=False):
    rng = np.random.default_rng(seed)
    F = DIMS["mlp_hidden"]
    mod = rng.standard_normal((n_streams, 3, D)) * 0.3
    if zero_gate:
        mod[:, 2, :] = 0.0
    return {"mod": mod, "w_in": rng.standard_normal((3 * D + 2 * F, D)) / np.sqrt(D),
            "w_out": rng.standard_normal((D, D + F)) / np.sqrt(D + F),
            "q_scale": np.ones(8), "k_scale": np.ones(8)}


def _inputs(n_img=12, n_txt=5, seed=0):
    rng = np.random.default_rng(seed)
    x_img = oracle.round_bf16(rng.standard_normal((n_img, D)))
    x_c = oracle.round_bf16(rng.standard_normal((n_txt, D)))
    x_n = oracle.round_bf16(rng.standard_normal((n_txt, D)))
    pos = np.zeros((n_img + n_txt, 4), dtype=np.int64)
    pos[:n_img, 1] = np.arange(n_img) // 4
    pos[:n_img, 2] = np.arange(n_img) % 4
    pos[n_img:, 0] = np.arange(n_txt)
    return x_img, x_c, x_n, pos


def test_zero_gates_return_the_image_tokens():
    # every block with a zero gate returns its input exactly, so both branches
    # leave the image rows unchanged and the guided result is x_img
    x_img, x_c, x_n, pos = _inputs()
    img = [_block(1, 1, True)]
    txt = [_block(2, 1, True)]
    joint = [_block(3, 2, True), _block(4, 2, True)]
    out = oracle.stack_cfg_ref(x_img, x_c, x_n, pos, img, txt, joint, DIMS, 4.0)
    assert np.array_equal(out, x_img)


def test_one_joint_block_is_the_block():
    x_img, x_c, _, pos = _inputs()
    b = _block(7, 2)
    h = oracle.stack_branch(x_img, x_c, pos, [], [], [b], DIMS)
    x = np.concatenate([x_img, x_c])
    y = oracle.block_ref(x, b["mod"], pos, b["w_in"], b["w_out"], b["q_scale"], b["k_scale"],
                         [12, 5], 2, 8, 24)["y"]
    assert np.array_equal(h, oracle.round_bf16(y))


def test_stage1_image_blocks_do_not_see_the_text():
    x_img, x_c, x_n, pos = _inputs()
    img, txt = [_block(11, 1)], [_block(12, 1)]
    a = oracle.stack_branch(x_img, x_c, pos, img, txt, [], DIMS)
    b = oracle.stack_branch(x_img, x_n, pos, img, txt, [], DIMS)
    assert np.array_equal(a[:12], b[:12])
    assert not np.array_equal(a[12:], b[12:])


def test_scale_one_is_the_conditional_branch_and_identical_prompts_cancel():
    x_img, x_c, x_n, pos = _inputs()
    img, txt, joint = [_block(21, 1)], [_block(22, 1)], [_block(23, 2)]
    cond = oracle.stack_branch(x_img, x_c, pos, img, txt, joint, DIMS)[:12]
    assert np.array_equal(oracle.stack_cfg_ref(x_img, x_c, x_n, pos, img, txt, joint, DIMS, 1.0),
                          cond)
    # same prompt in both branches: neg + s (cond - neg) = cond
    assert np.array_equal(oracle.stack_cfg_ref(x_img, x_c, x_c, pos, img, txt, joint, DIMS, 4.0),
                          cond)


def test_guidance_is_linear_in_the_branch_difference():
    x_img, x_c, x_n, pos = _inputs()
    img, txt, joint = [_block(31, 1)], [_block(32, 1)], [_block(33, 2)]
    cond = oracle.stack_branch(x_img, x_c, pos, img, txt, joint, DIMS)[:12]
    neg = oracle.stack_branch(x_img, x_n, pos, img, txt, joint, DIMS)[:12]
    g = oracle.stack_cfg_ref(x_img, x_c, x_n, pos, img, txt, joint, DIMS, 4.0)
    assert np.allclose(g, neg + 4.0 * (cond - neg), rtol=2 ** -8, atol=0)


def test_stage1_blocks_apply_per_stream_with_their_own_positions():
    x_img, x_c, _, pos = _inputs()
    bi, bt = _block(41, 1), _block(42, 1)
    h = oracle.stack_branch(x_img, x_c, pos, [bi], [bt], [], DIMS)
    yi = oracle.block_ref(x_img, bi["mod"], pos[:12], bi["w_in"], bi["w_out"], bi["q_scale"],
                          bi["k_scale"], [12], 2, 8, 24)["y"]
    yt = oracle.block_ref(x_c, bt["mod"], pos[12:], bt["w_in"], bt["w_out"], bt["q_scale"],
                          bt["k_scale"], [5], 2, 8, 24)["y"]
    assert np.array_equal(h[:12], oracle.round_bf16(yi))
    assert np.array_equal(h[12:], oracle.round_bf16(yt))


def _ref_inputs(n_img=12, n_ref=8, n_txt=5, seed=0):
    """Two references of 4 tokens each (2 x 2 grids, l = 1 and 2) between the
    image and the text rows."""
    x_img, x_c, x_n, p = _inputs(n_img, n_txt, seed)
    x_ref = oracle.round_bf16(np.random.default_rng(seed + 100).standard_normal((n_ref, D)))
    pr = np.zeros((n_ref, 4), dtype=np.int64)
    i = np.arange(n_ref)
    pr[:, 1], pr[:, 2], pr[:, 3] = (i % 4) // 2, i % 2, 1 + i // 4
    pos = np.concatenate([p[:n_img], pr, p[n_img:]])
    return x_img, x_ref, x_c, x_n, pos


def test_reference_stage1_blocks_run_on_the_reference_rows():
    x_img, x_ref, x_c, _, pos = _ref_inputs()
    bi, br, bt = _block(51, 1), _block(52, 1), _block(53, 1)
    h = oracle.stack_branch(x_img, x_c, pos, [bi], [bt], [], DIMS, x_ref=x_ref, ref_blocks=[br])
    yr = oracle.block_ref(x_ref, br["mod"], pos[12:20], br["w_in"], br["w_out"], br["q_scale"],
                          br["k_scale"], [8], 2, 8, 24)["y"]
    yt = oracle.block_ref(x_c, bt["mod"], pos[20:], bt["w_in"], bt["w_out"], bt["q_scale"],
                          bt["k_scale"], [5], 2, 8, 24)["y"]
    assert h.shape == (25, D)
    assert np.array_equal(h[12:20], oracle.round_bf16(yr))
    assert np.array_equal(h[20:], oracle.round_bf16(yt))


def test_joint_block_with_references_is_the_three_stream_block():
    x_img, x_ref, x_c, _, pos = _ref_inputs()
    b = _block(61, 3)
    h = oracle.stack_branch(x_img, x_c, pos, [], [], [b], DIMS, x_ref=x_ref)
    x = np.concatenate([x_img, x_ref, x_c])
    y = oracle.block_ref(x, b["mod"], pos, b["w_in"], b["w_out"], b["q_scale"], b["k_scale"],
                         [12, 8, 5], 2, 8, 24)["y"]
    assert np.array_equal(h, oracle.round_bf16(y))


def test_reference_stage_does_not_see_the_text_and_zero_gates_keep_the_image():
    x_img, x_ref, x_c, x_n, pos = _ref_inputs()
    br, bt = [_block(71, 1)], [_block(72, 1)]
    a = oracle.stack_branch(x_img, x_c, pos, [], bt, [], DIMS, x_ref=x_ref, ref_blocks=br)
    b = oracle.stack_branch(x_img, x_n, pos, [], bt, [], DIMS, x_ref=x_ref, ref_blocks=br)
    assert np.array_equal(a[:20], b[:20])
    zi, zr, zt = [_block(73, 1, True)], [_block(74, 1, True)], [_block(75, 1, True)]
    out = oracle.stack_cfg_ref(x_img, x_c, x_n, pos, zi, zt, [_block(76, 3, True)], DIMS, 4.0,
                               x_ref=x_ref, ref_blocks=zr)
    assert np.array_equal(out, x_img)


def test_the_reference_index_reaches_the_image_rows():
    # the same reference tokens at l = 1, 2 or at l = 3, 4 give a different
    # joint output on the image rows (RoPE's fourth axis is live)
    x_img, x_ref, x_c, _, pos = _ref_inputs()
    b = _block(81, 3)
    a = oracle.stack_branch(x_img, x_c, pos, [], [], [b], DIMS, x_ref=x_ref)
    pos2 = pos.copy()
    pos2[12:20, 3] += 2
    c = oracle.stack_branch(x_img, x_c, pos2, [], [], [b], DIMS, x_ref=x_ref)
    assert not np.array_equal(a[:12], c[:12])
