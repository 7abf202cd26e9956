"""Helpers shared by the GPU tests: device copies of the seeded inputs and
comparison against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from flow_matching_diffusion_adaln_amd import configs, inputs, ops


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.load_library()  # fails loudly when the HIP library is missing


def to_dev(d):
    out = {}
    for key, val in d.items():
        if val.dtype == np.uint16:
            out[key] = ops.to_device_bf16(val)
        else:
            out[key] = torch.from_numpy(np.ascontiguousarray(val)).cuda()
    return out


def widen(t):
    return oracle.widen_bf16(ops.to_host_bits(t))


def poisoned_workspace(desc):
    """A workspace whose every byte is 0xFF (bf16 NaN patterns), so that an
    output or intermediate the kernels fail to write shows up as NaN instead
    of a stale value left by an earlier call in the same memory."""
    return ops.alloc_workspace(desc).fill_(0xFF)


def run_block(dv, cfg, flags=0, y=None, workspace=None):
    desc = ops.make_desc(cfg.n_tokens, cfg.width, cfg.n_heads, cfg.head_dim, cfg.mlp_hidden,
                         flags=flags)
    if y is None:
        y = torch.full_like(dv["x"], float("nan"))
    if workspace is None:
        workspace = poisoned_workspace(desc)
    y = ops.block_fwd(dv["x"], dv["mod"], dv["pos"], dv["w_in"], dv["w_out"], dv["q_scale"],
                      dv["k_scale"], desc, y=y, workspace=workspace)
    torch.cuda.synchronize()
    return y


def oracle_block(d, cfg, rows=None, flags=0):
    return oracle.block_ref(d["x"], d["mod"], d["pos"], d["w_in"], d["w_out"], d["q_scale"],
                            d["k_scale"], cfg.n_tokens, cfg.n_heads, cfg.head_dim,
                            cfg.mlp_hidden, configs.ROPE_THETA, configs.LN_EPS, configs.QK_EPS,
                            flags=flags, rows=rows)


def sample_rows(cfg, n_random=48, seed=0):
    """Rows to check at full size: every stream's first and last rows, both
    sides of each stream boundary, the last 224- and 256-row tile edges, and a
    random spread."""
    N = cfg.N
    rows = {0, N - 1}
    e = 0
    for s in cfg.streams:
        rows.update({e, e + 1, e + s.n - 2, e + s.n - 1})
        e += s.n
    for bm in (224, 256):  # the GEMMs' two row-tile heights
        rows.update({(N // bm) * bm - 1, (N // bm) * bm})
    rng = np.random.default_rng(seed)
    rows.update(rng.choice(N, size=min(n_random, N), replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < N))


def block_config(name, n_tokens, config_id, **dims):
    """A joint-block config with the given token counts (image | [reference] | text);
    `dims` may override width, n_heads, head_dim and mlp_hidden."""
    kinds = {1: ("image",), 2: ("image", "text"), 3: ("image", "reference", "text")}[len(n_tokens)]
    streams = []
    for kind, n in zip(kinds, n_tokens):
        if kind == "text":
            streams.append(configs.Stream("text", n))
        else:
            streams.append(configs.Stream(kind, n, (1, n), 0.0 if kind == "reference" else 0.7))
    return configs.BlockConfig(name, config_id, tuple(streams), **dims)
