"""Element-wise GPU parity of the block's intermediate outputs, read back from
the documented workspace layout (include/dit.h): the AdaLN output u, q and k
after the QK RMSNorm and 4-axis RoPE of the input projection's epilogue, v,
the SwiGLU product m and the attention output o.

Each stage is checked against the oracle's definition applied to the GPU's
own (bf16) inputs of that stage, so that the bound is the stage's own
arithmetic and nothing upstream:
  u  = adaln_ref(x)                                   |du| <= 2^-8 |u| + 1e-5
  z  = u_gpu W_in^T in fp64; S = |u_gpu| |W_in|^T     fp32 accumulation of K
       exact products: |dz| <= K 2^-24 S (z itself is never stored; from
       161 to 256 tokens q and k are stored from z rounded to bf16 before the
       norm, adding 2^-8 |z|, which the bound allows up to 256 tokens)
  q  = c RoPE(RMSNorm(z_q) g_q), c = (float)(1/sqrt(128)) * (float)log2 e:
       the norm turns dz into (g / rms)(|dz_e| + |z_e| max|dz| / rms), the
       rotation mixes a pair (sqrt 2) and adds its angle error (2e-6 of the
       pair), the store rounds to bf16 (2^-8 |q|); k likewise with g_k, c = 1
  v  = z_v                                            |dv| <= |dz| + 2^-8 |v|
  m  = silu(z_gate) z_up   |dm| <= 1.1 |dz_gate| |up| + |silu(gate)| |dz_up|
                                    + (2^-8 + 1e-5) |m|
  o  = softmax(ln 2 * q_gpu k_gpu^T) v_gpu per head (the stored q carries
       log2 e, and the kernel takes exp2): the weights are rounded to bf16
       before the product with v, so |do| <= 2^-8 (sum_j p_j |v_j| + |o|)
       + 1e-5 max|v|.
Pages: "Welcome FLUX.3 Image Klein in Diffusers", "How it works" (four RoPE
axes of 32 dims, full joint attention, SwiGLU MLP); the miles page "FLUX 3
Image Klein", section 3 (query_norm / key_norm scales).
The whole chain is also compared end to end with the oracle block's own
intermediates (relative L2 <= 1e-2, the block's bound).
"""
import numpy as np
import pytest
import torch

import oracle
from flow_matching_diffusion_adaln_amd import configs, inputs, ops

from _gpu import block_config, poisoned_workspace, require_gpu, sample_rows, to_dev

pytestmark = pytest.mark.gpu

EPS = configs.QK_EPS
C_Q = float(np.float32(np.float32(1.0) / np.sqrt(np.float32(128.0)))
            * np.float32(1.4426950408889634))
LN2 = float(np.log(2.0))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    require_gpu()


def log(msg):
    print(msg, flush=True)


def bf16_view(ws, offset, n_elem):
    return ws[offset:offset + 2 * n_elem].view(torch.int16)


def read_intermediates(ws, cfg):
    N, D, F = cfg.N, cfg.width, cfg.mlp_hidden
    R = (N * D * 2 + 255) // 256 * 256
    out = {}
    for i, name in enumerate(("u", "q", "k", "v")):
        bits = bf16_view(ws, i * R, N * D).cpu().numpy().view(np.uint16)
        out[name] = oracle.widen_bf16(bits).reshape(N, D)
    bits = bf16_view(ws, 4 * R, N * (D + F)).cpu().numpy().view(np.uint16)
    cat = oracle.widen_bf16(bits).reshape(N, D + F)
    out["o"], out["m"] = cat[:, :D], cat[:, D:]
    return out


def pair_partner(D):
    e = np.arange(D)
    return e ^ 1


def qk_check(z, dz, g, gpu, c, pos, short, what):
    """RMSNorm + RoPE of z [n, D] (the input projection's q or k columns)
    against the stored values gpu [n, D]; dz: the bound on |z_gpu - z|."""
    n, D = z.shape
    H, d = D // 128, 128
    zh = z.reshape(n, H, d)
    if short:  # q and k went through bf16 before the norm
        dz = dz + 2.0 ** -8 * np.abs(z)
    dzh = dz.reshape(n, H, d)
    rms = np.sqrt((zh ** 2).mean(axis=2, keepdims=True) + EPS)
    dmax = dzh.max(axis=2, keepdims=True)
    pre = (g[None, None, :] / rms) * (dzh + np.abs(zh) * dmax / rms)
    pre = np.maximum(pre, pre[:, :, pair_partner(d)]) * np.sqrt(2.0)
    ref = oracle.rope4_ref(oracle.head_rms_norm(zh, g, EPS), pos, configs.ROPE_THETA)
    pair = np.sqrt(ref ** 2 + ref[:, :, pair_partner(d)] ** 2)
    bound = c * (pre + 2e-6 * pair + 1e-5 * pair) + 2.0 ** -8 * c * np.abs(ref) + 1e-6
    got = gpu.reshape(n, H, d)
    err = np.abs(got - c * ref)
    worst = float((err / bound).max())
    log(f"  {what}: max err/bound {worst:.3f}, max |err| {err.max():.3e}")
    assert np.all(err <= bound), what
    return ref


def check_intermediates(cfg, seed, rows=None):
    d = inputs.make_block_inputs(cfg, seed=seed)
    dv = to_dev(d)
    desc = ops.make_desc(cfg.n_tokens, cfg.width, cfg.n_heads, cfg.head_dim, cfg.mlp_hidden)
    ws = poisoned_workspace(desc)
    log(f"intermediates {cfg.name} N={cfg.N} rows={'all' if rows is None else len(rows)}")
    ops.block_fwd(dv["x"], dv["mod"], dv["pos"], dv["w_in"], dv["w_out"], dv["q_scale"],
                  dv["k_scale"], desc, workspace=ws)
    torch.cuda.synchronize()
    g = read_intermediates(ws, cfg)
    N, D, F = cfg.N, cfg.width, cfg.mlp_hidden
    sel = np.arange(N) if rows is None else np.asarray(rows)
    short = N <= 256
    w_in = oracle.widen_bf16(d["w_in"])
    gq, gk = oracle.widen_bf16(d["q_scale"]), oracle.widen_bf16(d["k_scale"])
    pos = d["pos"].astype(np.int64)

    # u: the AdaLN stage
    u_ref = oracle.adaln_ref(oracle.widen_bf16(d["x"]), oracle.widen_bf16(d["mod"]),
                             cfg.n_tokens, configs.LN_EPS)
    assert np.all(np.abs(g["u"][sel] - u_ref[sel]) <= 2.0 ** -8 * np.abs(u_ref[sel]) + 1e-5)

    # the input projection's epilogues, from the GPU's own u
    u = g["u"][sel]
    z = u @ w_in.T
    dz = 3 * D * 2.0 ** -24 * (np.abs(u) @ np.abs(w_in).T)
    q_ref = qk_check(z[:, :D], dz[:, :D], gq, g["q"][sel], C_Q, pos[sel], short, "q")
    k_ref = qk_check(z[:, D:2 * D], dz[:, D:2 * D], gk, g["k"][sel], 1.0, pos[sel], short,
                     "k")
    zv, dzv = z[:, 2 * D:3 * D], dz[:, 2 * D:3 * D]
    assert np.all(np.abs(g["v"][sel] - zv) <= dzv + 2.0 ** -8 * np.abs(zv) + 1e-6), "v"
    a, b = z[:, 3 * D:3 * D + F], z[:, 3 * D + F:]
    da, db = dz[:, 3 * D:3 * D + F], dz[:, 3 * D + F:]
    m_ref = oracle.swiglu_ref(a, b)
    silu_a = oracle.silu(a)
    bound_m = 1.1 * da * np.abs(b) + np.abs(silu_a) * db + (2.0 ** -8 + 1e-5) * np.abs(m_ref) + 1e-6
    err_m = np.abs(g["m"][sel] - m_ref)
    log(f"  m: max err/bound {float((err_m / bound_m).max()):.3f}")
    assert np.all(err_m <= bound_m), "m"

    # attention, from the GPU's own q, k, v (all keys)
    H = cfg.n_heads
    qg = g["q"][sel].reshape(len(sel), H, 128)
    kg, vg = g["k"].reshape(N, H, 128), g["v"].reshape(N, H, 128)
    o_ref = np.empty((len(sel), H, 128))
    mass = np.empty_like(o_ref)
    for h in range(H):
        p = oracle.softmax_rows((qg[:, h, :] @ kg[:, h, :].T) * LN2)
        o_ref[:, h, :] = p @ vg[:, h, :]
        mass[:, h, :] = p @ np.abs(vg[:, h, :])
    o_ref = o_ref.reshape(len(sel), D)
    bound_o = 2.0 ** -8 * (mass.reshape(len(sel), D) + np.abs(o_ref)) + 1e-5 * np.abs(vg).max()
    err_o = np.abs(g["o"][sel] - o_ref)
    log(f"  o: max err/bound {float((err_o / bound_o).max()):.3f}")
    assert np.all(err_o <= bound_o), "o"

    # end to end against the oracle block's intermediates
    ref = oracle.block_ref(d["x"], d["mod"], d["pos"], d["w_in"], d["w_out"], d["q_scale"],
                           d["k_scale"], cfg.n_tokens, cfg.n_heads, cfg.head_dim, cfg.mlp_hidden,
                           configs.ROPE_THETA, configs.LN_EPS, configs.QK_EPS, rows=rows)
    pairs = (("q", g["q"][sel] / C_Q, ref["q"].reshape(len(sel), D)),
             ("k", g["k"], ref["k"].reshape(N, D)), ("v", g["v"], ref["v"].reshape(N, D)),
             ("o", g["o"][sel], ref["o"]), ("m", g["m"][sel], ref["m"]))
    for name, got, want in pairs:
        e = oracle.rel_l2(got, want)
        log(f"  end to end {name}: relL2 {e:.3e}")
        assert e <= 1e-2, name


def test_intermediates_c1():
    # 336 tokens: 224-row tiles, norm + RoPE fused into the GEMM epilogue
    check_intermediates(configs.C1, seed=21)


def test_intermediates_c2_sampled():
    check_intermediates(configs.C2, seed=22, rows=sample_rows(configs.C2, n_random=40))


@pytest.mark.parametrize("n_tokens,cid", [((80,), 120), ((97,), 121), ((160,), 124),
                                          ((200, 56), 122)])
def test_intermediates_short_sequences(n_tokens, cid):
    # up to 160 tokens the weight-streaming projections (norm + RoPE in the
    # input projection's epilogue); at 256 every tile split along K, then the
    # fix-up stores q and k and the separate norm + RoPE pass runs
    check_intermediates(block_config(f"short{sum(n_tokens)}", n_tokens, cid), seed=23)


def test_intermediates_three_streams_with_reference():
    cfg = block_config("ref3", (256, 192, 80), 123)
    check_intermediates(cfg, seed=24)


def test_intermediates_256_row_tiles_sampled():
    # 5,601 tokens: both projections run 256-row tiles (one wave per head in
    # the q / k epilogue) with split tails
    cfg = block_config("split5601", (5441, 160), 95)
    check_intermediates(cfg, seed=25, rows=sample_rows(cfg, n_random=32))
