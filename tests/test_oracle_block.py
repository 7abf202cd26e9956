"""Pins for the oracle's whole-block composition (CPU only).

The block's wiring (which rows of W_in are q, k, v, gate, up; which columns of
W_out take attention vs MLP; one gate per stream; joint attention across all
streams) is pinned by a scalar-loop brute force on a tiny block and by
special inputs whose result has a closed form.
"""
import math

import numpy as np
import pytest

import oracle

# tiny generic shape: width 16 = 2 heads x 8 dims (each RoPE axis one pair), F = 8
D, H, d, F = 16, 2, 8, 8


def tiny_inputs(seed, n_tok=(5, 3)):
    rng = np.random.default_rng(seed)
    N = sum(n_tok)
    return dict(
        x=rng.normal(size=(N, D)),
        mod=rng.normal(scale=0.3, size=(len(n_tok), 3, D)),
        pos=rng.integers(0, 9, size=(N, 4)),
        w_in=rng.normal(scale=D ** -0.5, size=(3 * D + 2 * F, D)),
        w_out=rng.normal(scale=(D + F) ** -0.5, size=(D, D + F)),
        q_scale=rng.uniform(0.5, 1.5, size=d),
        k_scale=rng.uniform(0.5, 1.5, size=d),
    ), list(n_tok)


def run(inp, n_tok, **kw):
    return oracle.block_ref(inp["x"], inp["mod"], inp["pos"], inp["w_in"], inp["w_out"],
                            inp["q_scale"], inp["k_scale"], n_tok, H, d, F, **kw)


def brute_block(inp, n_tok, theta=10000.0, eps=1e-6):
    """The block in scalar Python loops, written from the pages' description."""
    x, mod, pos = inp["x"], inp["mod"], inp["pos"]
    w_in, w_out, gq, gk = inp["w_in"], inp["w_out"], inp["q_scale"], inp["k_scale"]
    N = x.shape[0]
    stream = []
    for s, n in enumerate(n_tok):
        stream += [s] * n
    u = [[0.0] * D for _ in range(N)]
    for i in range(N):
        mu = sum(x[i]) / D
        var = sum((t - mu) ** 2 for t in x[i]) / D
        for j in range(D):
            s = stream[i]
            u[i][j] = (x[i][j] - mu) / math.sqrt(var + eps) * (1 + mod[s][1][j]) + mod[s][0][j]

    def proj(i, row0, n_out):
        return [sum(u[i][c] * w_in[row0 + o][c] for c in range(D)) for o in range(n_out)]

    def norm_rope(vec, g, p):
        out = [0.0] * D
        for h in range(H):
            seg = vec[h * d:(h + 1) * d]
            rms = math.sqrt(sum(t * t for t in seg) / d + eps)
            seg = [seg[e] / rms * g[e] for e in range(d)]
            da = d // 4
            for a in range(4):
                for j in range(da // 2):
                    ang = p[a] * theta ** (-2.0 * j / da)
                    e0 = a * da + 2 * j
                    xa, ya = seg[e0], seg[e0 + 1]
                    out[h * d + e0] = xa * math.cos(ang) - ya * math.sin(ang)
                    out[h * d + e0 + 1] = xa * math.sin(ang) + ya * math.cos(ang)
        return out

    Q = [norm_rope(proj(i, 0, D), gq, pos[i]) for i in range(N)]
    K = [norm_rope(proj(i, D, D), gk, pos[i]) for i in range(N)]
    V = [proj(i, 2 * D, D) for i in range(N)]
    y = np.zeros((N, D))
    r_all = np.zeros((N, D))
    for i in range(N):
        o = [0.0] * D
        for h in range(H):
            lg = [sum(Q[i][h * d + e] * K[j][h * d + e] for e in range(d)) / math.sqrt(d)
                  for j in range(N)]
            mx = max(lg)
            w = [math.exp(t - mx) for t in lg]
            for e in range(d):
                o[h * d + e] = sum(w[j] * V[j][h * d + e] for j in range(N)) / sum(w)
        gate = proj(i, 3 * D, F)
        up = proj(i, 3 * D + F, F)
        m = [gate[c] / (1 + math.exp(-gate[c])) * up[c] for c in range(F)]
        cat = o + m
        for c in range(D):
            r = sum(cat[t] * w_out[c][t] for t in range(D + F))
            r_all[i, c] = r
            y[i, c] = x[i][c] + mod[stream[i]][2][c] * r
    return y, r_all


@pytest.mark.parametrize("seed,n_tok", [(0, (5, 3)), (1, (4,)), (2, (3, 2, 4))])
def test_block_matches_scalar_brute_force(seed, n_tok):
    inp, n_tok = tiny_inputs(seed, n_tok)
    y, r = brute_block(inp, n_tok)
    out = run(inp, n_tok)
    np.testing.assert_allclose(out["y"], y, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["r"], r, rtol=0, atol=1e-12)


def test_zero_gate_returns_residual_exactly():
    inp, n_tok = tiny_inputs(3)
    inp["mod"][:, 2] = 0.0
    np.testing.assert_array_equal(run(inp, n_tok)["y"], inp["x"])


def test_zero_gate_on_one_stream():
    inp, n_tok = tiny_inputs(4, (5, 3))
    inp["mod"][1, 2] = 0.0
    y = run(inp, n_tok)["y"]
    np.testing.assert_array_equal(y[5:], inp["x"][5:])
    assert np.all(np.abs(y[:5] - inp["x"][:5]).max(axis=1) > 1e-6)


def test_flags():
    inp, n_tok = tiny_inputs(5)
    base = run(inp, n_tok)
    s = oracle.stream_index(n_tok)
    gate = inp["mod"][s, 2, :]
    np.testing.assert_allclose(run(inp, n_tok, flags=oracle.FLAG_NO_RESIDUAL)["y"],
                               gate * base["r"], atol=1e-15)
    np.testing.assert_allclose(run(inp, n_tok, flags=oracle.FLAG_NO_GATE)["y"],
                               inp["x"] + base["r"], atol=1e-15)
    np.testing.assert_allclose(
        run(inp, n_tok, flags=oracle.FLAG_NO_GATE | oracle.FLAG_NO_RESIDUAL)["y"], base["r"],
        atol=1e-15)


def test_uniform_attention_is_joint_and_feeds_first_wout_columns():
    # q = k = 0 (zero q/k rows of W_in) -> every token attends uniformly to all
    # tokens of every stream; gate/up rows zero -> the MLP branch is 0.  Then the
    # branch r is mean(v) times the first D columns of W_out, for every row.
    inp, n_tok = tiny_inputs(6, (5, 3))
    inp["w_in"][0:2 * D] = 0.0
    inp["w_in"][3 * D:] = 0.0
    out = run(inp, n_tok)
    u = oracle.adaln_ref(inp["x"], inp["mod"], n_tok, 1e-6)
    vbar = (u @ inp["w_in"][2 * D:3 * D].T).mean(axis=0)
    r_want = np.array([sum(vbar[t] * inp["w_out"][c][t] for t in range(D)) for c in range(D)])
    np.testing.assert_allclose(out["r"], np.tile(r_want, (8, 1)), atol=1e-12)
    assert np.all(out["m"] == 0)


def test_mlp_branch_uses_gate_rows_then_up_rows():
    # v = 0 -> attention out is 0; r = silu(u Wg^T) * (u Wu^T) @ W_out[:, D:]^T
    inp, n_tok = tiny_inputs(7)
    inp["w_in"][2 * D:3 * D] = 0.0
    out = run(inp, n_tok)
    u = oracle.adaln_ref(inp["x"], inp["mod"], n_tok, 1e-6)
    for i in range(u.shape[0]):
        g = [sum(u[i, c] * inp["w_in"][3 * D + f, c] for c in range(D)) for f in range(F)]
        p = [sum(u[i, c] * inp["w_in"][3 * D + F + f, c] for c in range(D)) for f in range(F)]
        m = [g[f] / (1 + math.exp(-g[f])) * p[f] for f in range(F)]
        r = [sum(m[f] * inp["w_out"][c, D + f] for f in range(F)) for c in range(D)]
        np.testing.assert_allclose(out["r"][i], r, atol=1e-12)
    assert np.all(out["o"] == 0)


def test_permutation_within_a_stream_permutes_outputs():
    inp, n_tok = tiny_inputs(8, (6, 3))
    perm = np.concatenate([np.random.default_rng(0).permutation(6), np.arange(6, 9)])
    p_inp = dict(inp)
    p_inp["x"] = inp["x"][perm]
    p_inp["pos"] = inp["pos"][perm]
    np.testing.assert_allclose(run(p_inp, n_tok)["y"], run(inp, n_tok)["y"][perm], atol=1e-12)


def test_row_sampling_matches_full_evaluation():
    inp, n_tok = tiny_inputs(9, (6, 4))
    full = run(inp, n_tok)
    rows = np.array([0, 3, 7, 9])
    part = run(inp, n_tok, rows=rows)
    for key in ("y", "r", "o", "m", "q"):
        np.testing.assert_allclose(part[key], full[key][rows], atol=1e-13)
    np.testing.assert_allclose(part["k"], full["k"], atol=1e-13)  # keys cover every token


def test_bf16_bits_are_widened_exactly():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F], dtype=np.uint16)
    want = [1.0, -2.0, 1.0 + 2 ** -7, 0.0, -0.0, (2 - 2 ** -7) * 2.0 ** 127]
    got = oracle.widen_bf16(bits)
    assert list(got) == want
    assert math.copysign(1.0, got[4]) == -1.0


def test_rel_l2():
    assert oracle.rel_l2([3.0, 4.0], [3.0, 4.0]) == 0.0
    assert oracle.rel_l2([3.0, 4.0 + 5.0], [3.0, 4.0]) == pytest.approx(1.0)


def test_fused_projections_equal_the_separate_layers():
    # the input projection is to_q, to_k, to_v and ff.linear_in stacked by
    # rows, and the output projection is to_out.0 plus ff.linear_out: the
    # block equals the composition of the separate products
    rng = np.random.default_rng(21)
    n, D, F = [9, 4], 16, 24
    N = sum(n)
    x = rng.standard_normal((N, D))
    mod = rng.standard_normal((2, 3, D)) * 0.3
    pos = np.zeros((N, 4), dtype=np.int64)
    pos[:9, 1], pos[:9, 2], pos[9:, 0] = np.arange(9) // 3, np.arange(9) % 3, np.arange(4)
    w_q, w_k, w_v = (rng.standard_normal((D, D)) / 4 for _ in range(3))
    w_lin = rng.standard_normal((2 * F, D)) / 4
    w_o, w_lo = rng.standard_normal((D, D)) / 4, rng.standard_normal((D, F)) / 5
    g = np.ones(8)
    out = oracle.block_ref(x, mod, pos, np.concatenate([w_q, w_k, w_v, w_lin]),
                           np.concatenate([w_o, w_lo], axis=1), g, g, n, 2, 8, F)
    u = oracle.adaln_ref(x, mod, n, 1e-6)
    q = oracle.rope4_ref(oracle.head_rms_norm((u @ w_q.T).reshape(N, 2, 8), g, 1e-6), pos, 1e4)
    k = oracle.rope4_ref(oracle.head_rms_norm((u @ w_k.T).reshape(N, 2, 8), g, 1e-6), pos, 1e4)
    v = (u @ w_v.T).reshape(N, 2, 8)
    o = oracle.attention_ref(q, k, v, 1 / np.sqrt(8)).reshape(N, D)
    lin = u @ w_lin.T
    m = oracle.swiglu_ref(lin[:, :F], lin[:, F:])
    r = o @ w_o.T + m @ w_lo.T
    assert np.allclose(out["r"], r, rtol=1e-12, atol=1e-12)
