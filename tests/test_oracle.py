"""Pins for the fp64 oracle, independent of the oracle itself (CPU only).

Each check comes from the pages' worked closed forms (tests/golden), from a
mathematical invariant of the operation, or from a brute-force scalar-loop
evaluation on tiny inputs.  Together they are meant to fail on a dropped term,
a wrong sign or index, or a transposed operand anywhere in the oracle.
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
_MATH = {"__builtins__": {}, "cos": math.cos, "sin": math.sin, "log": math.log,
         "sqrt": math.sqrt}


def ev(expr: str) -> float:
    return float(eval(expr, _MATH))  # closed forms from our own fixture files


def golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


def kv_rows(name):
    out = {}
    for line in golden_rows(name):
        key, *vals = line.split()
        out.setdefault(key, []).append(vals)
    return out


# ----------------------------------------------------------------- AdaLN ----

def test_adaln_golden_two_streams():
    g = kv_rows("adaln_two_streams.txt")
    x = np.array([[ev(v) for v in g["x0"][0]], [ev(v) for v in g["x1"][0]]])
    mod = np.zeros((2, 3, 4))
    mod[0, 0], mod[0, 1] = [ev(v) for v in g["shift0"][0]], [ev(v) for v in g["scale0"][0]]
    mod[1, 0], mod[1, 1] = [ev(v) for v in g["shift1"][0]], [ev(v) for v in g["scale1"][0]]
    mod[:, 2] = 123.0  # the gate plays no part in the modulated input
    u = oracle.adaln_ref(x, mod, [1, 1], 1e-6)
    want = np.array([[ev(v) for v in g["u0"][0]], [ev(v) for v in g["u1"][0]]])
    np.testing.assert_allclose(u, want, rtol=0, atol=1e-13)


def test_layernorm_moments():
    rng = np.random.default_rng(1)
    x = rng.normal(3.0, 2.5, size=(7, 96))
    eps = 1e-6
    y = oracle.layer_norm(x, eps)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-13)
    np.testing.assert_allclose(y.var(axis=1), var / (var + eps), rtol=1e-12)


def test_adaln_matches_scalar_loops():
    rng = np.random.default_rng(2)
    n_tok = [3, 2, 4]
    x = rng.normal(size=(9, 16))
    mod = rng.normal(size=(3, 3, 16))
    eps = 1e-6
    want = np.zeros_like(x)
    row = 0
    for s, n in enumerate(n_tok):
        for _ in range(n):
            mu = sum(x[row]) / 16
            var = sum((v - mu) ** 2 for v in x[row]) / 16
            for j in range(16):
                xh = (x[row, j] - mu) / math.sqrt(var + eps)
                want[row, j] = xh * (1 + mod[s, 1, j]) + mod[s, 0, j]
            row += 1
    np.testing.assert_allclose(oracle.adaln_ref(x, mod, n_tok, eps), want, rtol=0, atol=1e-12)


def test_adaln_segment_boundaries():
    # stream 1 gets scale = -1, so its rows collapse to its shift exactly
    rng = np.random.default_rng(3)
    n_tok = [5, 4, 3]
    x = rng.normal(size=(12, 32))
    mod = np.zeros((3, 3, 32))
    mod[1, 1] = -1.0
    mod[1, 0] = np.arange(32)
    mod[2, 0] = 7.0
    u = oracle.adaln_ref(x, mod, n_tok, 1e-6)
    np.testing.assert_array_equal(u[5:9], np.tile(np.arange(32.0), (4, 1)))
    np.testing.assert_allclose(u[:5].mean(axis=1), 0, atol=1e-13)
    np.testing.assert_allclose(u[9:].mean(axis=1), 7, atol=1e-13)
    assert list(oracle.stream_index(n_tok)) == [0] * 5 + [1] * 4 + [2] * 3


# ----------------------------------------------------------- QK RMSNorm ----

def test_rmsnorm_golden():
    g = kv_rows("swiglu_rmsnorm.txt")
    q = np.array([[[ev(v) for v in g["rms_q"][0]]]])
    gg = np.array([ev(v) for v in g["rms_g"][0]])
    want = np.array([ev(v) for v in g["rms_o"][0]])
    np.testing.assert_allclose(oracle.head_rms_norm(q, gg, 1e-6)[0, 0], want, atol=1e-14)


def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(4)
    q = rng.normal(size=(5, 3, 128))
    out = oracle.head_rms_norm(q, np.ones(128), 0.0)
    np.testing.assert_allclose(np.sqrt((out ** 2).mean(axis=-1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(oracle.head_rms_norm(7.5 * q, np.ones(128), 0.0), out, rtol=1e-12)
    # each head is normalized on its own
    q2 = q.copy()
    q2[:, 1] *= 100
    np.testing.assert_allclose(oracle.head_rms_norm(q2, np.ones(128), 0.0), out, rtol=1e-12)


# ---------------------------------------------------------------- RoPE ----

def test_rope_golden_unit_vectors():
    for line in golden_rows("rope4_unit_vectors.txt"):
        p, din, dout, expr = [s.strip() for s in line.split("|")]
        pos = np.array([[int(t) for t in p.split()]], dtype=np.int64)
        q = np.zeros((1, 1, 128))
        q[0, 0, int(din)] = 1.0
        out = oracle.rope4_ref(q, pos, 10000.0)[0, 0]
        assert out[int(dout)] == pytest.approx(ev(expr), abs=1e-12), line
        # a unit vector stays inside its own pair
        pair = int(din) // 2 * 2
        rest = np.delete(out, [pair, pair + 1])
        assert np.all(rest == 0), line


def test_rope_omega_values():
    assert oracle.rope_omega(0, 32, 10000.0) == 1.0
    assert oracle.rope_omega(8, 32, 10000.0) == pytest.approx(0.01, rel=1e-14)
    assert oracle.rope_omega(15, 32, 10000.0) == pytest.approx(10000 ** (-30 / 32), rel=1e-14)


def _rand_pos(rng, n, hi=200):
    return rng.integers(0, hi, size=(n, 4))


def test_rope_preserves_pair_norms():
    rng = np.random.default_rng(5)
    q = rng.normal(size=(11, 3, 128))
    out = oracle.rope4_ref(q, _rand_pos(rng, 11), 10000.0)
    pn = lambda a: np.sqrt(a[..., 0::2] ** 2 + a[..., 1::2] ** 2)  # noqa: E731
    np.testing.assert_allclose(pn(out), pn(q), rtol=1e-12)


def test_rope_relative_positions():
    # <R(p+c) q, R(p'+c) k> == <R(p) q, R(p') k> for any integer shift c in Z^4
    rng = np.random.default_rng(6)
    q = rng.normal(size=(8, 2, 128))
    k = rng.normal(size=(8, 2, 128))
    pq, pk = _rand_pos(rng, 8), _rand_pos(rng, 8)
    base = np.einsum("nhd,nhd->nh", oracle.rope4_ref(q, pq, 1e4), oracle.rope4_ref(k, pk, 1e4))
    for _ in range(3):
        c = rng.integers(-500, 500, size=(1, 4))
        sh = np.einsum("nhd,nhd->nh", oracle.rope4_ref(q, pq + c, 1e4),
                       oracle.rope4_ref(k, pk + c, 1e4))
        np.testing.assert_allclose(sh, base, rtol=1e-9, atol=1e-9)
    # and it does depend on the difference: moving one side breaks equality
    moved = np.einsum("nhd,nhd->nh", oracle.rope4_ref(q, pq + np.array([[0, 1, 0, 0]]), 1e4),
                      oracle.rope4_ref(k, pk, 1e4))
    assert np.max(np.abs(moved - base)) > 1e-3


def test_rope_identity_and_axis_locality():
    rng = np.random.default_rng(7)
    q = rng.normal(size=(6, 2, 128))
    np.testing.assert_array_equal(oracle.rope4_ref(q, np.zeros((6, 4), np.int64), 1e4), q)
    pos = _rand_pos(rng, 6)
    base = oracle.rope4_ref(q, pos, 1e4)
    for a in range(4):
        p2 = pos.copy()
        p2[:, a] += 13
        out = oracle.rope4_ref(q, p2, 1e4)
        touched = np.any(out != base, axis=(0, 1))
        assert touched[32 * a:32 * a + 32].all()
        assert not touched[:32 * a].any() and not touched[32 * a + 32:].any()


def test_rmsnorm_and_rope_commute_with_unit_scale():
    rng = np.random.default_rng(8)
    q = rng.normal(size=(5, 3, 128))
    pos = _rand_pos(rng, 5)
    g = np.ones(128)
    a = oracle.rope4_ref(oracle.head_rms_norm(q, g, 1e-6), pos, 1e4)
    b = oracle.head_rms_norm(oracle.rope4_ref(q, pos, 1e4), g, 1e-6)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------- softmax ----

def test_softmax_rows_sum_to_one_and_shift_invariant():
    rng = np.random.default_rng(9)
    s = rng.normal(scale=8.0, size=(6, 40))
    p = oracle.softmax_rows(s)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p > 0)
    np.testing.assert_allclose(oracle.softmax_rows(s + rng.normal(size=(6, 1)) * 100), p,
                               rtol=1e-12)
    # it follows the logits' order
    assert np.all(np.argsort(p, axis=1) == np.argsort(s, axis=1))


# ----------------------------------------------------------- attention ----

def test_attention_golden_three_keys():
    g = kv_rows("attention_three_keys.txt")
    vec = lambda key: np.array([ev(v) for v in g[key][0]])  # noqa: E731
    q = vec("q")[None, None, :]
    k = np.stack([vec("k0"), vec("k1"), vec("k2")])[:, None, :]
    v = np.stack([vec("v0"), vec("v1"), vec("v2")])[:, None, :]
    o = oracle.attention_ref(q, k, v, 1.0 / math.sqrt(4))
    np.testing.assert_allclose(o[0, 0], vec("o"), rtol=0, atol=1e-13)
    s = (q[0, 0] @ k[:, 0].T) / 2
    np.testing.assert_allclose(oracle.softmax_rows(s[None])[0], vec("p"), atol=1e-15)


def test_attention_matches_per_query_loops():
    rng = np.random.default_rng(10)
    N, H, d = 7, 3, 8
    q, k, v = (rng.normal(size=(N, H, d)) for _ in range(3))
    scale = 1 / math.sqrt(d)
    want = np.zeros((N, H, d))
    for h, i in itertools.product(range(H), range(N)):
        logits = [sum(q[i, h, e] * k[j, h, e] for e in range(d)) * scale for j in range(N)]
        mx = max(logits)
        w = [math.exp(t - mx) for t in logits]
        tot = sum(w)
        for e in range(d):
            want[i, h, e] = sum(w[j] * v[j, h, e] for j in range(N)) / tot
    np.testing.assert_allclose(oracle.attention_ref(q, k, v, scale), want, rtol=0, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(11)
    N, H, d = 9, 2, 16
    q = rng.normal(size=(N, H, d))
    v = rng.normal(size=(N, H, d))
    # identical keys -> uniform weights -> mean of v
    k = np.tile(rng.normal(size=(1, H, d)), (N, 1, 1))
    np.testing.assert_allclose(oracle.attention_ref(q, k, v, 0.25),
                               np.tile(v.mean(axis=0, keepdims=True), (N, 1, 1)), atol=1e-12)
    # one dominant logit -> that token's value
    qq = rng.normal(size=(1, H, d))
    k = rng.normal(size=(N, H, d)) * 0.01
    k[4] = qq[0] * 50
    o = oracle.attention_ref(qq, k, v, 1.0)
    np.testing.assert_allclose(o[0], v[4], atol=1e-9)
    # a single token attends to itself only
    np.testing.assert_allclose(oracle.attention_ref(q[:1], k[:1], v[:1], 1.0), v[:1], atol=1e-15)


# -------------------------------------------------------------- SwiGLU ----

def test_swiglu_golden():
    for line in golden_rows("swiglu_rmsnorm.txt"):
        key, *vals = line.split()
        if key == "silu":
            assert oracle.silu(np.array(ev(vals[0]))) == pytest.approx(ev(vals[1]), abs=1e-15)
        elif key == "swiglu":
            got = oracle.swiglu_ref(np.array(ev(vals[0])), np.array(ev(vals[1])))
            assert got == pytest.approx(ev(vals[2]), abs=1e-14)
    # the gate half goes through silu, the up half does not
    assert oracle.swiglu_ref(np.array(0.0), np.array(5.0)) == 0.0
    assert oracle.swiglu_ref(np.array(5.0), np.array(0.0)) == 0.0
    assert oracle.swiglu_ref(np.array(1.0), np.array(2.0)) == pytest.approx(2 / (1 + math.exp(-1)))
