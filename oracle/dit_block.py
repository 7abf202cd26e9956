"""Plain float64 CPU oracle for the FLUX.3 Image Klein parallel DiT block forward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never calls it and
has no CPU fallback.  It imports numpy and nothing from the HIP package.

What is computed, step by step (sources are the pages' sections):

* Per-stream modulation and the parallel block: "Welcome FLUX.3 Image Klein in
  Diffusers", section "How it works": every block runs attention and a SwiGLU
  MLP side by side on one normalized input; shift, scale and gate come from
  timestep modulation set separately for text, image and reference tokens.
* Token order [image | reference | text]: same section (stage-2 streams are
  concatenated) and the miles page "FLUX 3 Image Klein", section 1 (joint
  blocks over [image | text]).
* Projections to_q, to_k, to_v, ff.linear_in, to_out.0, ff.linear_out: the
  NeMo AutoModel page, section "Image-Editing LoRA" (LoRA target modules).
* Per-head QK RMSNorm with a learnable scale: the miles page, section 3
  "Family config" (query_norm.scale / key_norm.scale).
* 4-axis RoPE (t, h, w, l), 32 of the 128 head dims per axis: "Welcome FLUX.3
  Image Klein in Diffusers", section "How it works".
* Full attention with no mask, padding attended: same section and the miles
  page, section 3 (the DiT takes no padding mask).

Readings taken where the pages are silent:
  norm = LayerNorm without affine, biased variance, eps 1e-6;
  u = LN(x) * (1 + scale) + shift; one gate per stream on the summed branch;
  no biases; W_in rows [q | k | v | gate | up]; silu on the gate half;
  W_out columns [attention | mlp]; QK RMSNorm eps 1e-6 then RoPE;
  RoPE pairs are adjacent dims (2j, 2j+1) inside each axis' 32 dims with
  omega_j = theta^(-2j/32), theta = 10000, rotation (x, y) ->
  (x cos - y sin, x sin + y cos); softmax scale 1/sqrt(d).

All arithmetic is float64.  Inputs arrive as bf16 bit patterns (uint16) and
are widened exactly.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

FLAG_NO_RESIDUAL = 1  # y = gate * r
FLAG_NO_GATE = 2      # the gate is taken as 1


def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns -> float64, exactly (bf16 is the top half of a float32)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def stream_index(n_tokens: Sequence[int]) -> np.ndarray:
    """Row i -> index of the stream whose segment contains it (segments in order)."""
    return np.repeat(np.arange(len(n_tokens)), np.asarray(n_tokens, dtype=np.int64))


def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """LayerNorm over the last axis with no affine part and the biased variance."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def adaln_ref(x: np.ndarray, mod: np.ndarray, n_tokens: Sequence[int], eps: float) -> np.ndarray:
    """Per-stream AdaLN: u = LN(x) * (1 + scale_s) + shift_s, s = the row's stream.

    x: [N, D]; mod: [S, 3, D] holding (shift, scale, gate) per stream.
    """
    s = stream_index(n_tokens)
    if s.shape[0] != x.shape[0]:
        raise ValueError("token counts do not add up to the row count")
    shift = mod[s, 0, :]
    scale = mod[s, 1, :]
    return layer_norm(x, eps) * (1.0 + scale) + shift


def head_rms_norm(q: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Per-head RMSNorm: q / sqrt(mean_e q_e^2 + eps) * g.  q: [N, H, d], g: [d]."""
    return q / np.sqrt((q ** 2).mean(axis=-1, keepdims=True) + eps) * g


def rope_omega(j: int, axis_dims: int, theta: float) -> float:
    """Frequency of pair j inside one axis: theta^(-2j / axis_dims)."""
    return float(theta) ** (-2.0 * j / axis_dims)


def rope4_ref(q: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """4-axis RoPE.  q: [N, H, d]; pos: [N, 4] integer (t, h, w, l).

    Axis a owns dims [a*d/4, (a+1)*d/4); inside it pair j is the adjacent dims
    (2j, 2j+1) and turns by angle pos_a * omega_j.
    """
    N, H, d = q.shape
    if d % 8:
        raise ValueError("head_dim must split into 4 axes of whole pairs")
    da = d // 4
    out = np.array(q, dtype=np.float64, copy=True)
    posf = np.asarray(pos, dtype=np.float64)
    for a in range(4):
        for j in range(da // 2):
            phi = posf[:, a] * rope_omega(j, da, theta)
            c = np.cos(phi)[:, None]
            s = np.sin(phi)[:, None]
            i0 = a * da + 2 * j
            x0 = q[:, :, i0]
            x1 = q[:, :, i0 + 1]
            out[:, :, i0] = x0 * c - x1 * s
            out[:, :, i0 + 1] = x0 * s + x1 * c
    return out


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax, two-pass: subtract the row max, exponentiate, divide by the row sum."""
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Full (unmasked) multi-head attention, one head at a time.

    q: [Nq, H, d] (the queries wanted), k, v: [N, H, d] (all tokens).
    o_h = softmax(q_h k_h^T * scale) v_h.
    """
    Nq, H, d = q.shape
    o = np.empty((Nq, H, v.shape[-1]), dtype=np.float64)
    for h in range(H):
        p = softmax_rows((q[:, h, :] @ k[:, h, :].T) * scale)
        o[:, h, :] = p @ v[:, h, :]
    return o


def silu(a: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def swiglu_ref(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """SwiGLU: silu(gate) * up."""
    return silu(gate) * up


def block_ref(x, mod, pos, w_in, w_out, q_scale, k_scale, n_tokens: Sequence[int],
              n_heads: int, head_dim: int, mlp_hidden: int, theta: float = 10000.0,
              ln_eps: float = 1e-6, qk_eps: float = 1e-6, flags: int = 0,
              rows: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """The parallel block forward in float64.

    Arguments may be float arrays or bf16 bit patterns (uint16, widened here).
    Shapes: x [N, D], mod [S, 3, D], pos [N, 4], w_in [3D + 2F, D],
    w_out [D, D + F], q_scale / k_scale [d].
    rows: optional sorted indices; outputs are then evaluated only at those
    rows (keys and values still come from every token).
    Returns y, r (the branch before the gate), o (attention out, [n, D]),
    m (SwiGLU out), q (after norm and RoPE, [n, H, d]) at the selected rows,
    and k (after norm and RoPE), v and u (modulated input) at every row.
    """
    def f(a):
        a = np.asarray(a)
        return widen_bf16(a) if a.dtype == np.uint16 else a.astype(np.float64)

    x, mod, w_in, w_out, gq, gk = (f(a) for a in (x, mod, w_in, w_out, q_scale, k_scale))
    pos = np.asarray(pos, dtype=np.int64)
    N, D = x.shape
    H, d, F = n_heads, head_dim, mlp_hidden
    if H * d != D or w_in.shape != (3 * D + 2 * F, D) or w_out.shape != (D, D + F):
        raise ValueError("inconsistent block shapes")
    sel = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)

    u = adaln_ref(x, mod, n_tokens, ln_eps)
    w_q, w_k, w_v = w_in[0:D], w_in[D:2 * D], w_in[2 * D:3 * D]
    w_gate, w_up = w_in[3 * D:3 * D + F], w_in[3 * D + F:3 * D + 2 * F]

    q = (u[sel] @ w_q.T).reshape(len(sel), H, d)
    k = (u @ w_k.T).reshape(N, H, d)
    v = (u @ w_v.T).reshape(N, H, d)
    q = rope4_ref(head_rms_norm(q, gq, qk_eps), pos[sel], theta)
    k = rope4_ref(head_rms_norm(k, gk, qk_eps), pos, theta)

    o = attention_ref(q, k, v, 1.0 / np.sqrt(d)).reshape(len(sel), D)
    m = swiglu_ref(u[sel] @ w_gate.T, u[sel] @ w_up.T)
    r = np.concatenate([o, m], axis=1) @ w_out.T

    s = stream_index(n_tokens)[sel]
    gate = np.ones_like(r) if flags & FLAG_NO_GATE else mod[s, 2, :]
    y = gate * r if flags & FLAG_NO_RESIDUAL else x[sel] + gate * r
    return {"y": y, "r": r, "o": o, "m": m, "q": q, "k": k, "v": v, "u": u}


def rel_l2(a, b) -> float:
    """||a - b||_2 / ||b||_2 over all elements, in float64."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))
