"""Pins of the sampler oracle (oracle/sampler.py) against facts that do not
come from the oracle itself: the schedule count the pages print, closed
forms of the shift and the sinusoids, Euler's exactness on a straight flow,
brute-force loops for the layers, and properties of the composed step."""
import math

import numpy as np
import pytest

import oracle
from oracle.sampler import GROUP_IMG, GROUP_JOINT, GROUP_REF, GROUP_TXT

D, H, HD, F, C, T = 16, 2, 8, 24, 8, 12
DIMS = dict(n_heads=H, head_dim=HD, mlp_hidden=F)


# ---- schedule ---------------------------------------------------------------

def test_44_of_50_steps_run_above_half():
    # "Welcome FLUX.3 Image Klein in Diffusers", How it works: with the time
    # shift of 6.93, 44 of 50 steps run above sigma = 0.5
    s = oracle.flow_sigmas(50, 6.93)
    assert len(s) == 51
    assert int((s[:50] > 0.5).sum()) == 44


def test_shift_endpoints_monotone_and_threshold():
    for n, a in ((50, 6.93), (16, 6.93), (10, 3.0), (7, 1.0)):
        s = oracle.flow_sigmas(n, a)
        assert s[0] == 1.0 and s[-1] == 0.0
        assert np.all(np.diff(s) < 0)
        # sigma' > 1/2  <=>  a u > (1 + (a - 1) u) / 2  <=>  u > 1 / (a + 1);
        # count the grid points u = 1 - i/n above it by hand
        want = sum(1 for i in range(n) if (1 - i / n) > 1 / (a + 1))
        assert int((s[:n] > 0.5).sum()) == want
    # alpha = 1 is the unshifted linear schedule
    assert np.allclose(oracle.flow_sigmas(8, 1.0), np.linspace(1, 0, 9), rtol=0, atol=1e-15)


def test_shift_of_a_midpoint_by_hand():
    # u = 1/2, alpha = 6.93: 3.465 / 3.965
    s = oracle.flow_sigmas(2, 6.93)
    assert s[1] == pytest.approx(3.465 / 3.965, rel=1e-15)


# ---- timestep sinusoids ---------------------------------------------------------

def test_sinusoid_closed_forms():
    phi0 = oracle.timestep_sinusoid(0.0)
    assert phi0.shape == (256,)
    assert np.array_equal(phi0[:128], np.ones(128)) and np.array_equal(phi0[128:], np.zeros(128))
    t = 0.37
    phi = oracle.timestep_sinusoid(t)
    # the first frequency is 1 and the last 10000^(-127/128)
    assert phi[0] == pytest.approx(math.cos(370.0), abs=1e-12)
    assert phi[128] == pytest.approx(math.sin(370.0), abs=1e-12)
    assert phi[127] == pytest.approx(math.cos(370.0 * 10000.0 ** (-127 / 128)), abs=1e-12)
    assert np.allclose(phi[:128] ** 2 + phi[128:] ** 2, 1.0, rtol=0, atol=1e-12)


# ---- layers --------------------------------------------------------------------

def test_linear_against_loops():
    rng = np.random.default_rng(1)
    x, w, b = rng.standard_normal((3, 5)), rng.standard_normal((4, 5)), rng.standard_normal(4)
    want = np.zeros((3, 4))
    for i in range(3):
        for j in range(4):
            acc = b[j]
            for k in range(5):
                acc += x[i, k] * w[j, k]
            want[i, j] = acc
    assert np.allclose(oracle.linear(x, w, b), want, rtol=1e-14, atol=1e-14)


def test_output_layers_against_loops():
    rng = np.random.default_rng(2)
    n = 3
    w = {"out_mod_w": rng.standard_normal((2 * D, D)) * 0.2, "out_mod_b": rng.standard_normal(2 * D),
         "out_w": rng.standard_normal((C, D)), "out_b": rng.standard_normal(C)}
    h = oracle.round_bf16(rng.standard_normal((n, D)) * 3 + 1)
    e = oracle.round_bf16(rng.standard_normal(D))
    got = oracle.output_layers(h, e, w, 1e-6)
    ss = oracle.round_bf16(w["out_mod_w"] @ e + w["out_mod_b"])
    shift, scale = ss[:D], ss[D:]
    for r in range(n):
        mean = sum(h[r]) / D
        var = sum((v - mean) ** 2 for v in h[r]) / D
        u = [oracle.round_bf16(np.array([(h[r, c] - mean) / math.sqrt(var + 1e-6) * (1 + scale[c])
                                         + shift[c]]))[0] for c in range(D)]
        for j in range(C):
            want = oracle.round_bf16(np.array([sum(u[c] * w["out_w"][j, c] for c in range(D))
                                               + w["out_b"][j]]))[0]
            assert got[r, j] == pytest.approx(want, rel=2 ** -7)


def test_time_embedding_composition():
    # zero first layer: the embedding no longer depends on t and equals
    # SiLU(W2 SiLU(b1) + b2), each stage rounded to bf16
    rng = np.random.default_rng(3)
    b1 = rng.standard_normal(D)
    w2, b2 = rng.standard_normal((D, D)) * 0.3, rng.standard_normal(D)
    w = {"t_w1": np.zeros((D, 256)), "t_b1": b1, "t_w2": w2, "t_b2": b2}
    silu = lambda a: a / (1 + np.exp(-a))  # noqa: E731
    h = oracle.round_bf16(silu(b1))
    want = oracle.round_bf16(silu(w2 @ h + b2))
    for t in (0.0, 0.3, 1.0):
        assert np.array_equal(oracle.time_embedding(t, w), want)


# ---- Euler and guidance ----------------------------------------------------------

def test_euler_is_exact_on_a_straight_flow():
    # x(sigma) = (1 - sigma) x0 + sigma eps has the constant velocity eps - x0,
    # so Euler steps over any schedule land on x0 from eps
    rng = np.random.default_rng(4)
    x0, eps = rng.standard_normal((5, C)), rng.standard_normal((5, C))
    s = oracle.flow_sigmas(13, 6.93)
    z = eps.copy()
    for i in range(13):
        z, v = oracle.euler_cfg_step(z, eps - x0, None, 1.0, s[i], s[i + 1])
        # and the state stays on the path
        assert np.allclose(z, (1 - s[i + 1]) * x0 + s[i + 1] * eps, rtol=0, atol=1e-12)
    assert np.allclose(z, x0, rtol=0, atol=1e-12)


def test_euler_with_guidance_closed_form():
    z = np.array([1.0, 2.0])
    zc, v = oracle.euler_cfg_step(z, np.array([3.0, -1.0]), np.array([1.0, 2.0]), 4.0, 0.75, 0.5)
    assert np.array_equal(v, [9.0, -10.0])
    assert np.array_equal(zc, [1.0 - 0.25 * 9.0, 2.0 + 0.25 * 10.0])


# ---- the composed step ----------------------------------------------------------

def model(seed, n_img_b=1, n_ref_b=1, n_txt_b=1, n_joint_b=2, zero_gates=False):
    rng = np.random.default_rng(seed)

    def r(*shape, std=1.0):
        return rng.standard_normal(shape) * std

    mod_w = [r(3 * D, D, std=0.3) for _ in range(4)]
    mod_b = [r(3 * D, std=0.3) for _ in range(4)]
    if zero_gates:
        for g in range(4):
            mod_w[g][2 * D:] = 0.0
            mod_b[g][2 * D:] = 0.0
    n_blocks = n_img_b + n_ref_b + n_txt_b + n_joint_b
    blocks = [{"w_in": r(3 * D + 2 * F, D, std=D ** -0.5), "w_out": r(D, D + F, std=(D + F) ** -0.5),
               "q_scale": np.ones(HD), "k_scale": np.ones(HD)} for _ in range(n_blocks)]
    return {"img_in_w": r(D, C, std=C ** -0.5), "img_in_b": r(D, std=0.1),
            "ref_in_w": r(D, C, std=C ** -0.5), "ref_in_b": r(D, std=0.1),
            "txt_in_w": r(D, T, std=T ** -0.5), "txt_in_b": r(D, std=0.1),
            "t_w1": r(D, 256, std=1 / 16), "t_b1": r(D, std=0.1),
            "t_w2": r(D, D, std=D ** -0.5), "t_b2": r(D, std=0.1),
            "mod_w": mod_w, "mod_b": mod_b,
            "out_mod_w": r(2 * D, D, std=0.3), "out_mod_b": r(2 * D, std=0.1),
            "out_w": r(C, D, std=D ** -0.5), "out_b": r(C, std=0.1), "blocks": blocks}


def dims(n_img, n_img_b=1, n_ref_b=1, n_txt_b=1):
    return dict(DIMS, n_img=n_img, n_img_blocks=n_img_b, n_ref_blocks=n_ref_b,
                n_txt_blocks=n_txt_b)


def step_inputs(n_img=8, n_ref=4, n_txt=3, seed=0):
    rng = np.random.default_rng(seed + 50)
    z = oracle.round_bf16(rng.standard_normal((n_img, C)))
    tc = oracle.round_bf16(rng.standard_normal((n_txt, T)))
    tn = oracle.round_bf16(rng.standard_normal((n_txt, T)))
    ref = oracle.round_bf16(rng.standard_normal((n_ref, C))) if n_ref else None
    pos = np.zeros((n_img + n_ref + n_txt, 4), dtype=np.int64)
    pos[:n_img, 1], pos[:n_img, 2] = np.arange(n_img) // 4, np.arange(n_img) % 4
    if n_ref:
        pos[n_img:n_img + n_ref, 1] = np.arange(n_ref) // 2
        pos[n_img:n_img + n_ref, 2] = np.arange(n_ref) % 2
        pos[n_img:n_img + n_ref, 3] = 1
    pos[n_img + n_ref:, 0] = np.arange(n_txt)
    return z, tc, tn, ref, pos


def test_zero_gates_reduce_the_step_to_embed_norm_project():
    # with every gate zero each block returns its input, so the image rows
    # reaching the output layers are the embedded latent, the text cannot
    # reach them (both branches agree) and the step has a closed form
    w = model(5, zero_gates=True)
    d = dims(8)
    z, tc, tn, ref, pos = step_inputs()
    prep = oracle.sampler_prepare(w, d, pos, tc, tn, ref)
    zn, v, (vc, vn) = oracle.denoise_step(w, d, prep, z, 0.8, 0.6, pos, 4.0)
    assert np.array_equal(vc, vn)
    x = oracle.round_bf16(z @ w["img_in_w"].T + w["img_in_b"])
    e = oracle.time_embedding(0.8, w)
    want_v = oracle.output_layers(x, e, w, 1e-6)
    assert np.array_equal(v, want_v)
    assert np.array_equal(zn, oracle.round_bf16(z - 0.2 * want_v))


def test_step_equals_the_stack_with_the_groups_modulation():
    # the step's conditional velocity is the output layers applied to the
    # (separately pinned) stack oracle run with the modulation the groups give
    w = model(6)
    d = dims(8)
    z, tc, tn, ref, pos = step_inputs(seed=1)
    prep = oracle.sampler_prepare(w, d, pos, tc, tn, ref)
    _, _, (vc, _) = oracle.denoise_step(w, d, prep, z, 0.9, 0.7, pos, 4.0)
    e, e0 = oracle.time_embedding(0.9, w), oracle.time_embedding(0.0, w)
    mi = oracle.modulation(e, w, GROUP_IMG)[None]
    mr = oracle.modulation(e0, w, GROUP_REF)[None]
    mt = oracle.modulation(e0, w, GROUP_TXT)[None]
    mj = np.stack([oracle.modulation(e, w, GROUP_JOINT), oracle.modulation(e0, w, GROUP_JOINT),
                   oracle.modulation(e0, w, GROUP_JOINT)])
    b = w["blocks"]
    x_img = oracle.round_bf16(z @ w["img_in_w"].T + w["img_in_b"])
    x_ref = oracle.round_bf16(ref @ w["ref_in_w"].T + w["ref_in_b"])
    x_txt = oracle.round_bf16(tc @ w["txt_in_w"].T + w["txt_in_b"])
    h = oracle.stack_branch(x_img, x_txt, pos, [dict(b[0], mod=mi)], [dict(b[2], mod=mt)],
                            [dict(bb, mod=mj) for bb in b[3:]], DIMS, x_ref=x_ref,
                            ref_blocks=[dict(b[1], mod=mr)])
    assert np.array_equal(vc, oracle.output_layers(h[:8], e, w, 1e-6))


def test_guidance_scale_one_and_identical_prompts():
    w = model(7)
    d = dims(8)
    z, tc, tn, ref, pos = step_inputs(seed=2)
    prep = oracle.sampler_prepare(w, d, pos, tc, tn, ref)
    z1, v1, _ = oracle.denoise_step(w, d, prep, z, 0.5, 0.25, pos, 1.0)
    prep_same = oracle.sampler_prepare(w, d, pos, tc, tc, ref)
    z4, v4, _ = oracle.denoise_step(w, d, prep_same, z, 0.5, 0.25, pos, 4.0)
    assert np.array_equal(z1, z4) and np.array_equal(v1, v4)
    # different prompts do reach the image rows
    _, vg, (vc, vn) = oracle.denoise_step(w, d, prep, z, 0.5, 0.25, pos, 4.0)
    assert not np.array_equal(vc, vn)
    assert np.allclose(vg, vn + 4 * (vc - vn), rtol=1e-15, atol=0)


def test_sample_runs_the_schedule_and_no_references():
    # two steps by hand equal sample(); a sequence without references works
    w = model(8, n_ref_b=0)
    d = dims(8, n_ref_b=0)
    z, tc, tn, _, pos = step_inputs(n_ref=0, seed=3)
    s = oracle.flow_sigmas(2, 6.93)
    prep = oracle.sampler_prepare(w, d, pos, tc, tn, None)
    z1 = oracle.denoise_step(w, d, prep, z, s[0], s[1], pos, 3.5)[0]
    z2 = oracle.denoise_step(w, d, prep, z1, s[1], s[2], pos, 3.5)[0]
    assert np.array_equal(oracle.sample(w, d, pos, z, tc, tn, None, 2, 6.93, 3.5), z2)
