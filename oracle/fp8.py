"""Plain CPU oracle for the FP8 (rowwise-scaled e4m3) projections of the block.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it.

Source: the SGLang diffusion cookbook page "FLUX.3" ships rowwise-scaled FP8
("fp8r") linear layers for latency; the pages give no formula, so the plain
reading of rowwise FP8 is taken:

* e4m3 is the OCP FP8 E4M3 format (sign, 4 exponent bits with bias 7, 3
  mantissa bits, subnormals at exponent 0, no infinities, S.1111.111 is NaN,
  largest finite 448), the format of gfx950's FP8 matrix cores;
* a bf16 matrix is quantized per row r: a_r = max |x_r|, inv_r = 448 / a_r
  and s_r = a_r / 448 in float32 (correctly rounded), codes
  q = e4m3(clamp(x * inv_r, -448, 448)) rounded to nearest, ties to the even
  code, the product x * inv_r rounded to float32 first; x ~ q * s_r.  An
  all-zero row has s_r = 0 and q = 0.  The float32 steps make the integer
  decisions in the precision the GPU takes them;
* a linear layer is sum_k q_a[m, k] q_w[n, k] * s_a[m] s_w[n], with both
  operands quantized per row (tokens for activations, output rows for
  weights);
* the FP8 block is the bf16 block with both projections FP8: u (the AdaLN
  output, rounded to bf16, as the bf16 path stores it) and the bf16 [o | m]
  are quantized per token row, W_in and W_out per output row; everything
  else is the block oracle's float64 arithmetic.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .dit_block import (FLAG_NO_GATE, FLAG_NO_RESIDUAL, adaln_ref, attention_ref, head_rms_norm,
                        rope4_ref, stream_index, swiglu_ref, widen_bf16)
from .stack import round_bf16

E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """The 127 finite non-negative e4m3 values, by code 0 .. 126 (ascending)."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of e4m3 codes (uint8); the NaN codes decode to NaN."""
    codes = np.asarray(codes, dtype=np.uint8)
    mag = codes & 0x7F
    vals = np.concatenate([e4m3_values(), [np.nan]])[mag]
    return np.where(codes & 0x80, -vals, vals)


def e4m3_round(x) -> np.ndarray:
    """Codes (uint8) of the e4m3 values nearest to x (|x| <= 448), ties to the
    even code; the sign bit follows x's sign (so -0.0 and small negatives that
    round to zero give 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX) or np.any(np.isnan(x)):
        raise ValueError("e4m3_round takes finite values within +-448")
    vals = e4m3_values()
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for s in range(0, flat.size, 1 << 22):  # in chunks, to bound the temporaries
        xc = flat[s:s + (1 << 22)]
        a = np.abs(xc)
        hi = np.clip(np.searchsorted(vals, a, side="left"), 0, 126)  # vals[hi] >= a
        lo = np.clip(hi - 1, 0, 126)
        dlo, dhi = a - vals[lo], vals[hi] - a
        pick = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(lo % 2 == 0, lo, hi)))
        pick = np.where(a == vals[hi], hi, pick)
        out[s:s + xc.size] = pick | np.where(np.signbit(xc), 0x80, 0)
    return out.reshape(x.shape)


def quantize_rows(x):
    """Rowwise e4m3 quantization of x [M, K] (bf16 bits or values exactly
    representable in float32).  Returns (codes uint8 [M, K], scales float32 [M])."""
    x = np.asarray(x)
    x32 = (widen_bf16(x) if x.dtype == np.uint16 else x).astype(np.float32)
    amax = np.max(np.abs(x32), axis=1)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, np.float32(E4M3_MAX) / amax, np.float32(0)).astype(np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    y = np.clip(x32 * inv[:, None], np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_round(y.astype(np.float64)), scale


def dequantize_rows(codes, scale) -> np.ndarray:
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[:, None]


def _qlin(qa, sa, qw, sw) -> np.ndarray:
    """sum_k q_a[m, k] q_w[n, k] * s_a[m] s_w[n] from codes and scales."""
    return (e4m3_decode(qa) @ e4m3_decode(qw).T) * (np.asarray(sa, np.float64)[:, None]
                                                    * np.asarray(sw, np.float64)[None, :])


def fp8_linear(x, w=None, wq=None) -> np.ndarray:
    """x [M, K] w [N, K]^T with both quantized per row: sum_k q_x q_w s_x s_w.
    wq = (codes, scales) of w, when already quantized."""
    qx, sx = quantize_rows(x)
    qw, sw = quantize_rows(w) if wq is None else wq
    return _qlin(qx, sx, qw, sw)


def block_ref_fp8(x, mod, pos, w_in, w_out, q_scale, k_scale, n_tokens: Sequence[int],
                  n_heads: int, head_dim: int, mlp_hidden: int, theta: float = 10000.0,
                  ln_eps: float = 1e-6, qk_eps: float = 1e-6, flags: int = 0,
                  rows: Optional[np.ndarray] = None, w_in_q=None, w_out_q=None):
    """The block with FP8 projections (see the module docstring); outputs as
    block_ref: y, r at the selected rows.  w_in_q / w_out_q: the weights'
    (codes, scales) when already quantized (w_in / w_out are then unused)."""
    def f(a):
        a = np.asarray(a)
        return widen_bf16(a) if a.dtype == np.uint16 else a.astype(np.float64)

    x, mod, gq, gk = (f(a) for a in (x, mod, q_scale, k_scale))
    pos = np.asarray(pos, dtype=np.int64)
    N, D = x.shape
    H, d, F = n_heads, head_dim, mlp_hidden
    sel = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)

    u = round_bf16(adaln_ref(x, mod, n_tokens, ln_eps))   # the bf16 u the GPU quantizes
    qu, su = quantize_rows(u)
    qw, sw = quantize_rows(w_in) if w_in_q is None else w_in_q
    # rows of W_in: [q | k | v | gate | up]; k and v for every token, the
    # rest for the selected rows only (quantization is per row, so slicing
    # rows of the codes is exact)
    kv = _qlin(qu, su, qw[D:3 * D], sw[D:3 * D])
    keep = np.r_[0:D, 3 * D:3 * D + 2 * F]
    zs = _qlin(qu[sel], su[sel], qw[keep], sw[keep])
    q = zs[:, 0:D].reshape(len(sel), H, d)
    k = kv[:, 0:D].reshape(N, H, d)
    v = kv[:, D:2 * D].reshape(N, H, d)
    q = rope4_ref(head_rms_norm(q, gq, qk_eps), pos[sel], theta)
    k = rope4_ref(head_rms_norm(k, gk, qk_eps), pos, theta)
    o = attention_ref(q, k, v, 1.0 / np.sqrt(d)).reshape(len(sel), D)
    m = swiglu_ref(zs[:, D:D + F], zs[:, D + F:D + 2 * F])
    cat = round_bf16(np.concatenate([o, m], axis=1))      # [o | m] as stored in bf16
    r = fp8_linear(cat, w_out, w_out_q)

    s = stream_index(n_tokens)[sel]
    gate = np.ones_like(r) if flags & FLAG_NO_GATE else mod[s, 2, :]
    y = gate * r if flags & FLAG_NO_RESIDUAL else x[sel] + gate * r
    return {"y": y, "r": r}
