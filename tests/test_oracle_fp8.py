"""Pins of the FP8 oracle (oracle/fp8.py): the e4m3 format from its
definition, rounding against brute force and hand-worked encodings, the
rowwise quantizer's invariants and error bound, exactness of the FP8 linear
on exactly representable operands, and the FP8 block against the bf16 block
within the quantization error, and the whole FP8 block against a scalar-loop
brute force written from the rowwise rule."""
import math

import numpy as np
import pytest

import oracle

DIMS = dict(n_heads=2, head_dim=8, mlp_hidden=24)
D = 16


def test_e4m3_table_from_the_format():
    v = oracle.e4m3_values()
    assert len(v) == 127 and np.all(np.diff(v) > 0)
    assert v[0] == 0 and v[1] == 2.0 ** -9            # smallest subnormal: 1/8 * 2^-6
    assert v[8] == 2.0 ** -6                           # smallest normal
    assert v[126] == 448.0                             # 1.75 * 2^8, S.1111.110
    assert v[0x38] == 1.0                              # exponent 7 = bias
    # 8 values per binade, spaced 2^(e-3)
    assert np.allclose(np.diff(v[0x38:0x41]), 1 / 8)
    assert np.isnan(oracle.e4m3_decode([0x7F])[0]) and np.isnan(oracle.e4m3_decode([0xFF])[0])
    assert oracle.e4m3_decode([0xFE])[0] == -448.0


def nearest_bruteforce(x: float) -> int:
    best, bd = None, None
    for c in range(127):
        val = oracle.e4m3_values()[c]
        dd = abs(val - abs(x))
        if bd is None or dd < bd or (dd == bd and c % 2 == 0):
            best, bd = c, dd
    return best | (0x80 if np.signbit(x) else 0)


def test_e4m3_round_against_bruteforce():
    v = oracle.e4m3_values()
    rng = np.random.default_rng(0)
    xs = np.concatenate([
        rng.uniform(-448, 448, 1500),
        rng.standard_normal(1500) * 2.0 ** rng.integers(-12, 6, 1500),
        (v[:-1] + v[1:]) / 2,                          # every tie
        -(v[:-1] + v[1:]) / 2,
        v, -v])
    xs = np.clip(xs, -448, 448)
    got = oracle.e4m3_round(xs)
    want = np.array([nearest_bruteforce(float(x)) for x in xs], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_hand_encodings():
    cases = {1.0: 0x38, 1.0625: 0x38, 1.1875: 0x3A, 448.0: 0x7E, -448.0: 0xFE, 0.0: 0x00,
             2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, 0.75: 0x34, 3.0: 0x44, 240.0: 0x77,
             232.0: 0x76, -1.0: 0xB8}
    # 1.0625: tie between 1 (0x38) and 1.125 (0x39), to the even code
    # 2^-10: tie between 0 and 2^-9; 3 * 2^-10: tie between 2^-9 and 2^-8 (0x02)
    # 232: tie between 224 (0x76) and 240 (0x77); 0.75 = 1.5 * 2^-1: 0 0110 100
    for x, c in cases.items():
        assert oracle.e4m3_round([x])[0] == c, (x, hex(c))
    with pytest.raises(ValueError):
        oracle.e4m3_round([449.0])


def test_quantize_rows_invariants_and_error_bound():
    rng = np.random.default_rng(1)
    x = oracle.round_bf16(rng.standard_normal((6, 64)) * np.array([1e-3, 0.1, 1, 10, 300, 1e4])[:, None])
    x[2, :] = 0.0                                      # an all-zero row
    q, s = oracle.quantize_rows(x)
    assert q.dtype == np.uint8 and s.dtype == np.float32
    assert s[2] == 0 and np.all(q[2] == 0)
    for r in (0, 1, 3, 4, 5):
        # the largest element maps to +-448 exactly
        assert np.max(q[r] & 0x7F) == 0x7E
        assert s[r] == np.float32(np.max(np.abs(x[r]))) / np.float32(448)
    back = oracle.dequantize_rows(q, s)
    # half a spacing of 3 mantissa bits (2^-4 relative) in the normal range,
    # half the subnormal spacing (2^-10 s) below it, plus float32 steps
    err = np.abs(back - x)
    bound = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * s[:, None] + 1e-6 * np.abs(x)
    assert np.all(err <= bound)


def test_fp8_linear_is_exact_on_representable_operands():
    # rows whose largest magnitude is exactly 448 * 2^k and whose entries are
    # e4m3 values times 2^k quantize losslessly, so the FP8 product is exact
    rng = np.random.default_rng(2)
    v = oracle.e4m3_values()

    def rows(n, k):
        m = rng.choice(v, size=(n, k)) * rng.choice([-1, 1], size=(n, k))
        m[:, 0] = 448.0
        return m * 2.0 ** rng.integers(-8, 4, size=(n, 1))

    a, w = rows(5, 32), rows(7, 32)
    assert np.array_equal(oracle.fp8_linear(a, w), a @ w.T)
    # a transposed scale (s_w on rows) would break this on unequal row scales
    qa, sa = oracle.quantize_rows(a)
    assert np.array_equal(oracle.dequantize_rows(qa, sa), a)


def _block_inputs(seed=3, n=(12, 5)):
    rng = np.random.default_rng(seed)
    N, F = sum(n), DIMS["mlp_hidden"]
    x = oracle.round_bf16(rng.standard_normal((N, D)))
    mod = oracle.round_bf16(rng.standard_normal((len(n), 3, D)) * 0.3)
    pos = np.zeros((N, 4), dtype=np.int64)
    pos[:n[0], 1], pos[:n[0], 2] = np.arange(n[0]) // 4, np.arange(n[0]) % 4
    pos[n[0]:, 0] = np.arange(N - n[0])
    w_in = oracle.round_bf16(rng.standard_normal((3 * D + 2 * F, D)) / np.sqrt(D))
    w_out = oracle.round_bf16(rng.standard_normal((D, D + F)) / np.sqrt(D + F))
    g = np.ones(8)
    return x, mod, pos, w_in, w_out, g, list(n)


def test_fp8_block_tracks_the_bf16_block_within_quantization_error():
    x, mod, pos, w_in, w_out, g, n = _block_inputs()
    ref = oracle.block_ref(x, mod, pos, w_in, w_out, g, g, n, **DIMS, flags=3)["r"]
    got = oracle.block_ref_fp8(x, mod, pos, w_in, w_out, g, g, n, **DIMS, flags=3)["r"]
    e = oracle.rel_l2(got, ref)
    # each FP8 operand carries about 2^-4 / sqrt(3) relative RMS error; two
    # quantized products in series stay well under 0.15
    assert 1e-3 < e < 0.15


def test_fp8_block_rows_and_prequantized_weights_agree():
    x, mod, pos, w_in, w_out, g, n = _block_inputs(seed=4)
    full = oracle.block_ref_fp8(x, mod, pos, w_in, w_out, g, g, n, **DIMS)
    rows = np.array([0, 5, 11, 12, 16])
    part = oracle.block_ref_fp8(x, mod, pos, None, None, g, g, n, **DIMS, rows=rows,
                                w_in_q=oracle.quantize_rows(w_in),
                                w_out_q=oracle.quantize_rows(w_out))
    assert np.allclose(part["y"], full["y"][rows], rtol=1e-12, atol=1e-12)
    # a zero gate returns x exactly, as in the bf16 block
    mod0 = mod.copy()
    mod0[:, 2, :] = 0
    assert np.array_equal(oracle.block_ref_fp8(x, mod0, pos, w_in, w_out, g, g, n, **DIMS)["y"],
                          x)


# ---- a scalar-loop FP8 block, written from the rowwise rule alone ----------

def bf16_nearest(v: float) -> float:
    """Nearest bf16 value to v (8 significant bits), ties to the even
    significand, from frexp: v = m 2^e with 0.5 <= |m| < 1, so the bf16
    spacing around v is 2^(e - 8); v / spacing is exact in float64."""
    if v == 0.0:
        return v
    _, e = math.frexp(v)
    sp = 2.0 ** (e - 8)
    return round(v / sp) * sp  # round() takes exact halves to the even integer


def quantize_row_scalar(row):
    """Rowwise e4m3 quantization of one row of bf16 values, each step in
    float32 as the rule states: a = max |x|, inv = 448 / a, s = a / 448,
    code = nearest e4m3 of clamp(x * inv) (found by brute force)."""
    a = np.float32(max(abs(float(t)) for t in row))
    if a == 0:
        return [0.0] * len(row), 0.0
    inv = np.float32(448.0) / a
    s = a / np.float32(448.0)
    table = oracle.e4m3_values()
    vals = []
    for t in row:
        y = float(min(max(np.float32(t) * inv, np.float32(-448.0)), np.float32(448.0)))
        c = nearest_bruteforce(y)
        vals.append(-table[c & 0x7F] if c & 0x80 else table[c & 0x7F])
    return vals, float(s)


def brute_block_fp8(x, mod, pos, w_in, w_out, n_tok, theta=10000.0, eps=1e-6):
    """The FP8 block in scalar loops: the bf16 AdaLN output u and the bf16
    [o | m] quantized per token row, W_in and W_out per output row, each
    product sum_k code_a code_w times s_a s_w; everything else as the bf16
    block (QK scales of one)."""
    H, d, F = DIMS["n_heads"], DIMS["head_dim"], DIMS["mlp_hidden"]
    N = x.shape[0]
    stream = []
    for s, n in enumerate(n_tok):
        stream += [s] * n
    u = []
    for i in range(N):
        mu = sum(x[i]) / D
        var = sum((t - mu) ** 2 for t in x[i]) / D
        s = stream[i]
        u.append([bf16_nearest((x[i][j] - mu) / math.sqrt(var + eps) * (1 + mod[s][1][j])
                               + mod[s][0][j]) for j in range(D)])
    qu = [quantize_row_scalar(u[i]) for i in range(N)]
    qwi = [quantize_row_scalar(w_in[o]) for o in range(w_in.shape[0])]
    qwo = [quantize_row_scalar(w_out[c]) for c in range(D)]

    def lin(qa, qw):
        return sum(qa[0][t] * qw[0][t] for t in range(len(qa[0]))) * qa[1] * qw[1]

    def norm_rope(vec, p):
        out = [0.0] * D
        for h in range(H):
            seg = vec[h * d:(h + 1) * d]
            rms = math.sqrt(sum(t * t for t in seg) / d + eps)
            seg = [t / rms for t in seg]
            for a in range(4):
                for j in range(d // 8):
                    ang = p[a] * theta ** (-2.0 * j / (d // 4))
                    e0 = a * (d // 4) + 2 * j
                    xa, ya = seg[e0], seg[e0 + 1]
                    out[h * d + e0] = xa * math.cos(ang) - ya * math.sin(ang)
                    out[h * d + e0 + 1] = xa * math.sin(ang) + ya * math.cos(ang)
        return out

    z = [[lin(qu[i], qwi[o]) for o in range(3 * D + 2 * F)] for i in range(N)]
    Q = [norm_rope(z[i][0:D], pos[i]) for i in range(N)]
    K = [norm_rope(z[i][D:2 * D], pos[i]) for i in range(N)]
    V = [z[i][2 * D:3 * D] for i in range(N)]
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
        gate, up = z[i][3 * D:3 * D + F], z[i][3 * D + F:3 * D + 2 * F]
        m = [gate[c] / (1 + math.exp(-gate[c])) * up[c] for c in range(F)]
        qc = quantize_row_scalar([bf16_nearest(t) for t in o + m])
        for c in range(D):
            r = lin(qc, qwo[c])
            r_all[i, c] = r
            y[i, c] = x[i][c] + mod[stream[i]][2][c] * r
    return y, r_all


def test_bf16_nearest_hand_values():
    assert bf16_nearest(1.0 + 2.0 ** -8) == 1.0                  # tie, to the even significand
    assert bf16_nearest(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6  # tie, to the even significand
    assert bf16_nearest(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7
    assert bf16_nearest(-3.0) == -3.0 and bf16_nearest(0.0) == 0.0
    assert np.array_equal(oracle.round_bf16(np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8])),
                          [1.0, 1.0 + 2.0 ** -6])


@pytest.mark.parametrize("seed,n_tok", [(5, (6, 3)), (6, (4, 2, 3))])
def test_fp8_block_matches_scalar_brute_force(seed, n_tok):
    x, mod, pos, w_in, w_out, g, n = _block_inputs(seed=seed, n=n_tok)
    got = oracle.block_ref_fp8(x, mod, pos, w_in, w_out, g, g, n, **DIMS)
    y, r = brute_block_fp8(x, mod, pos, w_in, w_out, n)
    np.testing.assert_allclose(got["r"], r, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["y"], y, rtol=0, atol=1e-12)
