#!/usr/bin/env python3
"""Benchmark of the parallel DiT block forward on one MI355X.

A step is one dit_block_fwd over the 1024^2 text-to-image joint sequence
(4,096 image + 160 text tokens, width 3072, 24 x 128 heads, SwiGLU 9216,
bf16), with inputs resident in HBM.  Four weight sets (about 1 GB) rotate
between steps so the 245 MB of one block's weights is not served from the
256 MB MALL.  The timed steps record no events; a second pass of the same
steps gives per-stage times from HIP events the library records on the work
stream between its kernels.  The fp64 CPU oracle of the same block
is timed once on the host as a baseline and its output gives the parity of
the timed configuration (y, and the branch r read with the residual and gate
switched off); attention alone (dit_attn_fwd_ws) is checked at sampled query rows against
the oracle's attention on the same seeded bf16 q, k, v.  A secondary field times one guided denoise step of
the two-stage stack (c5) through dit_stack_fwd and the flow-matching sampler
at the same shapes (`--no-stack` skips both), and
blocks of the 1024^2 edit with one reference (c4, 8,352 tokens) and of the
long 2048^2 edit (2048^2 image, one 2048^2 reference, 160 text tokens;
`--no-long` skips both).  `block_fp8` times
the same block with FP8 (rowwise e4m3) projections (`--no-fp8` skips it); it
is a secondary line, not the bf16 metric.  `stage1_c3` times the two stage-1
blocks of c3 (4,096 image tokens; 80 text tokens, weight-streaming bound).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5033.2    # dense fp8 MFMA: twice the bf16 rate


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--weight-sets", type=int, default=4)
    ap.add_argument("--prewarm-blocks", type=int, default=64,
                    help="blocks run before the W warmup steps: after an idle period the "
                         "chip's power management dips the clock for about 30 blocks before "
                         "it settles (the steady state is what a denoising loop sees)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the secondary measurement of the two-stage stack with CFG (c5)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the secondary measurement of the block with FP8 projections")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the secondary measurement of the long editing sequence")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before the timed steps "
                         "(reference point for the profiler's FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def measured_traffic():
    """HBM bytes per launch of the input-projection GEMM from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs (copy-calibrated), or None when the
    GEMM source has changed since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemm_in_c2_traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.h"):
        with open(os.path.join(ROOT, "flow_matching_diffusion_adaln_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != rec.get("source_sha256_16"):
        return None
    return rec.get("traffic_bytes_per_dispatch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def cpu_baseline(d, cfg, min_seconds: float = 10.0, max_blocks: int = 8):
    """Time the fp64 oracle on the full block (one block = one step), repeated
    until at least `min_seconds` have passed (at most `max_blocks` blocks).
    Returns the first block's output, the mean seconds per block, the
    threads used, the BLAS and the number of blocks run."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] + [1])
        ref, n, t0 = None, 0, time.perf_counter()
        while n < max_blocks and (n == 0 or time.perf_counter() - t0 < min_seconds):
            out = oracle.block_ref(d["x"], d["mod"], d["pos"], d["w_in"], d["w_out"],
                                   d["q_scale"], d["k_scale"], cfg.n_tokens, cfg.n_heads,
                                   cfg.head_dim, cfg.mlp_hidden)
            ref = out if ref is None else ref
            n += 1
        sec = (time.perf_counter() - t0) / n
    blas = ",".join(sorted({i.get("internal_api", "?") for i in info})) or "?"
    return ref, sec, threads, blas, n


def stack_c5(torch, configs, ops, steps: int, warmup: int) -> dict:
    """Secondary measurement: one guided denoise step of the two-stage stack
    (5 image + 5 text stage-1 blocks, 28 joint blocks, CFG scale 4) through
    dit_stack_fwd, each block with its own random weights generated on the
    device (38 sets, 9.3 GB).  The image stage-1 blocks are shared by both
    guidance branches, so the executed FLOPs are below two full forwards.
    Timed four ways: eager, with the stage-1 text blocks on the library's
    second stream (DIT_STACK_TEXT_SIDE_STREAM), and both as replays of one
    captured HIP graph."""
    sc = configs.C5
    D, F, d = configs.WIDTH, configs.MLP_HIDDEN, configs.HEAD_DIM
    n_img, n_txt = sc.image_side * sc.image_side, sc.n_text
    gen = torch.Generator(device="cuda").manual_seed(4321)

    def rnd(shape, std):
        return (torch.randn(shape, generator=gen, device="cuda") * std).to(torch.bfloat16)

    ones = torch.ones(d, dtype=torch.bfloat16, device="cuda")
    blocks = []
    for i in range(2 * sc.n_stage1 + sc.n_joint):
        s = 1 if i < 2 * sc.n_stage1 else 2
        blocks.append({"mod": rnd((s, 3, D), 0.1 ** 0.5), "w_in": rnd((3 * D + 2 * F, D), D ** -0.5),
                       "w_out": rnd((D, D + F), (D + F) ** -0.5), "q_scale": ones, "k_scale": ones})
    cfg_img = configs.BlockConfig("img", 0, (configs.Stream("image", n_img, (sc.image_side,) * 2, sc.t),))
    cfg_txt = configs.BlockConfig("txt", 0, (configs.Stream("text", n_txt),))
    cfg_joint = configs.BlockConfig("joint", 0, (configs.Stream("image", n_img, (sc.image_side,) * 2, sc.t),
                                                 configs.Stream("text", n_txt)))
    x_img = rnd((n_img, D), 1.0)
    x_c, x_n = rnd((n_txt, D), 1.0), rnd((n_txt, D), 1.0)
    from flow_matching_diffusion_adaln_amd import inputs
    pos = torch.from_numpy(inputs.positions(cfg_joint)).cuda()
    v = torch.empty((n_img, D), dtype=torch.bfloat16, device="cuda")

    def timed(side, graph):
        """ms per denoise step: eager calls or replays of one captured call;
        side: the stage-1 text blocks on the library's second stream."""
        desc = ops.make_stack_desc(n_img, n_txt, sc.n_stage1, sc.n_stage1, sc.n_joint,
                                   sc.cfg_scale, side_stream=side)
        ws = torch.empty(ops.stack_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        call = lambda: ops.stack_fwd(desc, x_img, x_c, x_n, pos, blocks, v_img=v, workspace=ws)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                call()
            call = g.replay
            call()
            torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        del ws
        return ms

    ms = timed(False, False)
    ms_side = timed(True, False)
    ms_graph = timed(False, True)
    ms_side_graph = timed(True, True)
    flop_exec = (sc.n_stage1 * cfg_img.flop() + 2 * sc.n_stage1 * cfg_txt.flop()
                 + 2 * sc.n_joint * cfg_joint.flop())
    flop_nominal = 2 * sc.n_stage1 * (cfg_img.flop() + cfg_txt.flop()) + 2 * sc.n_joint * cfg_joint.flop()
    assert bool(torch.isfinite(v.float()).all())
    return {
        "workload": f"c5: {sc.n_stage1} image ({n_img} tokens) + {sc.n_stage1} text ({n_txt}) "
                    f"stage-1 blocks, {sc.n_joint} joint blocks ({n_img + n_txt}), CFG pair "
                    f"(scale {sc.cfg_scale}); image stage-1 shared by both branches",
        "ms_per_denoise_step": round(ms, 3),
        "ms_text_side_stream": round(ms_side, 3),
        "ms_hip_graph": round(ms_graph, 3),
        "ms_text_side_stream_hip_graph": round(ms_side_graph, 3),
        "tflops_executed": round(flop_exec / (ms * 1e-3) / 1e12, 2),
        "gflop_executed": round(flop_exec / 1e9, 1),
        "gflop_two_full_forwards": round(flop_nominal / 1e9, 1),
        "steps": steps, "warmup": warmup,
    }


def sampler_c5(torch, configs, ops, steps: int, warmup: int) -> dict:
    """The flow-matching sampler at c5 shapes (4,096 image + 160 text tokens,
    5 + 5 stage-1 and 28 joint blocks, 128-channel latent, 20,480-wide text
    features) with device-generated random weights: the step-invariant prepare,
    guided steps (CFG 4) through dit_sampler_step, and one whole unguided
    16-step generation (prepare + 16 steps)."""
    sc = configs.C5
    D, F, d = configs.WIDTH, configs.MLP_HIDDEN, configs.HEAD_DIM
    C, T = 128, 20480
    n_img, n_txt = sc.image_side * sc.image_side, sc.n_text
    gen = torch.Generator(device="cuda").manual_seed(99)

    def rnd(shape, std):
        return (torch.randn(shape, generator=gen, device="cuda") * std).to(torch.bfloat16)

    ones = torch.ones(d, dtype=torch.bfloat16, device="cuda")
    blocks = [{"w_in": rnd((3 * D + 2 * F, D), D ** -0.5), "w_out": rnd((D, D + F), (D + F) ** -0.5),
               "q_scale": ones, "k_scale": ones} for _ in range(2 * sc.n_stage1 + sc.n_joint)]
    t = {"img_in_w": rnd((D, C), C ** -0.5), "img_in_b": rnd((D,), 0.1), "ref_in_w": None,
         "ref_in_b": None, "txt_in_w": rnd((D, T), T ** -0.5), "txt_in_b": rnd((D,), 0.1),
         "t_w1": rnd((D, 256), 1 / 16), "t_b1": rnd((D,), 0.1), "t_w2": rnd((D, D), D ** -0.5),
         "t_b2": rnd((D,), 0.1),
         "mod_w": [rnd((3 * D, D), (0.1 / D) ** 0.5) for _ in range(4)],
         "mod_b": [rnd((3 * D,), 0.1) for _ in range(4)],
         "out_mod_w": rnd((2 * D, D), (0.1 / D) ** 0.5), "out_mod_b": rnd((2 * D,), 0.1),
         "out_w": rnd((C, D), D ** -0.5), "out_b": rnd((C,), 0.1)}
    from flow_matching_diffusion_adaln_amd import inputs
    cfg_joint = configs.BlockConfig("joint", 0, (configs.Stream("image", n_img, (sc.image_side,) * 2, sc.t),
                                                 configs.Stream("text", n_txt)))
    pos = torch.from_numpy(inputs.positions(cfg_joint)).cuda()
    tc, tn = rnd((n_txt, T), 1.0), rnd((n_txt, T), 1.0)
    z0 = rnd((n_img, C), 1.0)

    def model_for(scale):
        st = ops.make_stack_desc(n_img, n_txt, sc.n_stage1, sc.n_stage1, sc.n_joint, scale)
        return ops.Model(ops.make_model_desc(st, C, T), t, blocks)

    guided = model_for(sc.cfg_scale)
    ws = ops.alloc_sampler_workspace(guided.desc)
    sig = ops.flow_sigmas(50, 6.93)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ops.sampler_prepare(guided, tc, tn, None, pos, ws)
    torch.cuda.synchronize()
    prep_ms = (time.perf_counter() - t0) * 1e3
    z = z0.clone()
    for i in range(warmup):
        ops.sampler_step(guided, z, sig[i], sig[i + 1], pos, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ops.sampler_step(guided, z, sig[warmup + i], sig[warmup + i + 1], pos, ws)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / steps
    assert bool(torch.isfinite(z.float()).all())

    plain = model_for(1.0)
    sig16 = ops.flow_sigmas(16, 6.93)
    z = z0.clone()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ops.sampler_prepare(plain, tc, None, None, pos, ws)
    for i in range(16):
        ops.sampler_step(plain, z, sig16[i], sig16[i + 1], pos, ws)
    torch.cuda.synchronize()
    gen16_s = time.perf_counter() - t0
    assert bool(torch.isfinite(z.float()).all())
    return {
        "workload": f"c5 sampler: 1024^2 latent ({n_img} tokens x {C} ch), {n_txt} text tokens "
                    f"({T}-wide features), {sc.n_stage1}+{sc.n_stage1}+{sc.n_joint} blocks, "
                    f"shift 6.93",
        "prepare_ms_guided": round(prep_ms, 2),
        "ms_per_guided_step": round(step_ms, 3),
        "guided_50_step_transformer_s": round((prep_ms + 50 * step_ms) / 1e3, 3),
        "unguided_16_step_generation_s": round(gen16_s, 3),
        "steps": steps, "warmup": warmup,
    }


def block_fp8(torch, configs, ops, timing, cfg, x, mod, pos, qs, ks, weights, steps: int,
              warmup: int) -> dict:
    """The same block (same inputs, the same rotating weight sets, quantized
    rowwise to e4m3 once up front) through dit_block_fwd_fp8."""
    D, F = cfg.width, cfg.mlp_hidden
    wq = [(ops.quantize_rows_fp8(w_in), ops.quantize_rows_fp8(w_out)) for w_in, w_out in weights]
    desc = ops.make_desc(cfg.n_tokens)
    ws = ops.alloc_fp8_workspace(desc)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    def step(i, events=None):
        (wi, si), (wo, so) = wq[i % len(wq)]
        ops.block_fwd_fp8(x, mod, pos, wi, si, wo, so, qs, ks, desc, y=y, workspace=ws,
                          stream=stream, events=events)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    evs = [timing.create(ops.N_STAGES + 1) for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    st = {name: float(np.mean([timing.elapsed_ms(e[j], e[j + 1]) for e in evs]))
          for j, name in enumerate(ops.STAGES)}
    for e in evs:
        timing.destroy(e)
    assert bool(torch.isfinite(y.float()).all())
    gin = 2.0 * cfg.N * D * (3 * D + 2 * F)
    gout = 2.0 * cfg.N * (D + F) * D
    return {
        "workload": f"{cfg.name} block with FP8 (rowwise e4m3) projections",
        "dtype": "fp8 e4m3 projections, bf16 attention",
        "ms_per_block": round(ms, 4),
        "tflops": round(cfg.flop() / (ms * 1e-3) / 1e12, 2),
        "stage_ms_mean": {k: round(v, 4) for k, v in st.items()},
        "gemm_in_tflops": round(gin / (st["gemm_in"] * 1e-3) / 1e12, 2),
        "gemm_in_frac_fp8_peak": round(gin / (st["gemm_in"] * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
        "gemm_out_with_quant_tflops": round(gout / (st["gemm_out"] * 1e-3) / 1e12, 2),
        "steps": steps, "warmup": warmup,
    }


def stage1_c3(torch, configs, ops, steps: int, warmup: int) -> dict:
    """The two stage-1 blocks of c3 as independent dit_block_fwd calls: the
    4,096-token image block (MFMA-bound) and the 80-token text block, whose
    time is set by streaming its 245 MB of weights (4 rotating weight sets,
    so they come from HBM)."""
    D, F, d = configs.WIDTH, configs.MLP_HIDDEN, configs.HEAD_DIM
    gen = torch.Generator(device="cuda").manual_seed(31)

    def rnd(shape, std):
        return (torch.randn(shape, generator=gen, device="cuda") * std).to(torch.bfloat16)

    ones = torch.ones(d, dtype=torch.bfloat16, device="cuda")
    weights = [(rnd((3 * D + 2 * F, D), D ** -0.5), rnd((D, D + F), (D + F) ** -0.5))
               for _ in range(4)]
    from flow_matching_diffusion_adaln_amd import inputs
    out = {}
    for cfg in (configs.C3_IMG, configs.C3_TXT):
        x = rnd((cfg.N, D), 1.0)
        mod = rnd((1, 3, D), 0.1 ** 0.5)
        pos = torch.from_numpy(inputs.positions(cfg)).cuda()
        desc = ops.make_desc(cfg.n_tokens)
        ws = ops.alloc_workspace(desc)
        y = torch.empty_like(x)
        n = steps * 4

        def step(i):
            w_in, w_out = weights[i % 4]
            ops.block_fwd(x, mod, pos, w_in, w_out, ones, ones, desc, y=y, workspace=ws)

        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            step(i)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / n
        assert bool(torch.isfinite(y.float()).all())
        wbytes = 2.0 * ((3 * D + 2 * F) * D + D * (D + F))
        out[cfg.name] = {"N": cfg.N, "ms_per_block": round(ms, 4),
                         "tflops": round(cfg.flop() / (ms * 1e-3) / 1e12, 2),
                         "weight_gbs": round(wbytes / (ms * 1e-3) / 1e9, 1),
                         "weight_frac_hbm_peak": round(wbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    out["workload"] = ("c3: stage-1 image block (4096 tokens, t=0.9) and stage-1 text block "
                       "(80 tokens, t=0), independent calls, 4 rotating weight sets")
    out["sum_ms"] = round(out["c3_img"]["ms_per_block"] + out["c3_txt"]["ms_per_block"], 4)
    out["steps"], out["warmup"] = steps * 4, warmup
    return out


def attn_parity(torch, oracle, inputs, ops, N: int, n_rows: int = 64) -> dict:
    """Attention alone at N tokens (dit_attn_fwd_ws: the block's schedule, one
    equal share of the key tiles per CU) on seeded bf16 q, k, v (24 x 128
    heads), against the oracle's attention on the same bf16 values, at sampled
    query rows (the oracle computes each row against all N keys)."""
    d = inputs.make_attn_inputs(N, 24, 128, seed=6, logit_std=1.0)
    q, k, v = (ops.to_device_bf16(d[n]) for n in ("q", "k", "v"))
    o = ops.attn_fwd_ws(q, k, v)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, N - 1],
                                     np.random.default_rng(1).choice(N, n_rows, replace=False)]))
    qh, kh, vh = (oracle.widen_bf16(d[n]) for n in ("q", "k", "v"))
    ref = oracle.attention_ref(qh[rows], kh, vh, 128 ** -0.5)
    got = oracle.widen_bf16(ops.to_host_bits(o))[rows]
    return {"relL2_attn": oracle.rel_l2(got, ref), "attn_bound": 5e-3,
            "attn_rows_checked": int(len(rows))}


def block_secondary(torch, configs, ops, timing, cfg, steps: int, warmup: int) -> dict:
    """One block forward of another sequence (the 1024^2 edit with one
    reference, c4, or the long 2048^2 edit) with device-generated random
    weights, timed per stage with HIP events."""
    D, F, d = cfg.width, cfg.mlp_hidden, cfg.head_dim
    from flow_matching_diffusion_adaln_amd import inputs
    gen = torch.Generator(device="cuda").manual_seed(777)

    def rnd(shape, std):
        return (torch.randn(shape, generator=gen, device="cuda") * std).to(torch.bfloat16)

    x = rnd((cfg.N, D), 1.0)
    mod = rnd((cfg.n_streams, 3, D), 0.1 ** 0.5)
    w_in, w_out = rnd((3 * D + 2 * F, D), D ** -0.5), rnd((D, D + F), (D + F) ** -0.5)
    ones = torch.ones(d, dtype=torch.bfloat16, device="cuda")
    pos = torch.from_numpy(inputs.positions(cfg)).cuda()
    desc = ops.make_desc(cfg.n_tokens)
    ws = ops.alloc_workspace(desc)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    def step(events=None):
        ops.block_fwd(x, mod, pos, w_in, w_out, ones, ones, desc, y=y, workspace=ws,
                      stream=stream, events=events)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    evs = [timing.create(ops.N_STAGES + 1) for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    st = {name: float(np.mean([timing.elapsed_ms(e[j], e[j + 1]) for e in evs]))
          for j, name in enumerate(ops.STAGES)}
    for e in evs:
        timing.destroy(e)
    assert bool(torch.isfinite(y.float()).all())
    attn_tflops = cfg.attn_flop() / (st["attn"] * 1e-3) / 1e12
    return {
        "workload": f"{cfg.name}: {cfg.description}; one parallel block forward",
        "ms_per_block": round(ms, 3),
        "tflops": round(cfg.flop() / (ms * 1e-3) / 1e12, 2),
        "gflop_per_block": round(cfg.flop() / 1e9, 1),
        "attn_share_of_flop": round(cfg.attn_flop() / cfg.flop(), 3),
        "stage_ms_mean": {k: round(v, 3) for k, v in st.items()},
        "attn_tflops": round(attn_tflops, 2),
        "attn_frac_mfma_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "steps": steps, "warmup": warmup,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the block is measured on a single MI355X)", file=sys.stderr)
        return 2

    import torch

    import oracle
    from flow_matching_diffusion_adaln_amd import configs, inputs, ops, timing

    cfg = configs.CONFIGS[args.config]
    torch.cuda.set_device(0)
    ops.load_library()
    dev_name = torch.cuda.get_device_name(0)

    t_gen = time.perf_counter()
    d = inputs.make_block_inputs(cfg, seed=0)
    t_gen = time.perf_counter() - t_gen
    x = ops.to_device_bf16(d["x"])
    mod = ops.to_device_bf16(d["mod"])
    pos = torch.from_numpy(d["pos"]).cuda()
    qs, ks = ops.to_device_bf16(d["q_scale"]), ops.to_device_bf16(d["k_scale"])
    weights = [(ops.to_device_bf16(d["w_in"]), ops.to_device_bf16(d["w_out"]))]
    gen = torch.Generator(device="cuda").manual_seed(1234)
    D, F = cfg.width, cfg.mlp_hidden
    for _ in range(1, args.weight_sets):
        w_in = (torch.randn((3 * D + 2 * F, D), generator=gen, device="cuda") * D ** -0.5)
        w_out = (torch.randn((D, D + F), generator=gen, device="cuda") * (D + F) ** -0.5)
        weights.append((w_in.to(torch.bfloat16), w_out.to(torch.bfloat16)))
    desc = ops.make_desc(cfg.n_tokens)
    ws = ops.alloc_workspace(desc)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step(i, events=None):
        w_in, w_out = weights[i % len(weights)]
        ops.block_fwd(x, mod, pos, w_in, w_out, qs, ks, desc, y=y, workspace=ws,
                      stream=stream, events=events)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # pre-warm, then the W warmup steps: the timed region starts in the
    # steady state of back-to-back blocks
    for i in range(args.prewarm_blocks):
        step(i)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly K steps, no per-stage events inside it
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-stage breakdown from a separate pass of K steps with HIP events
    # recorded between the stages (on the stream the kernels run on)
    n_ev = ops.N_STAGES + 1
    evs = [timing.create(n_ev) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()

    stage_ms = np.zeros((args.steps, ops.N_STAGES))
    for i in range(args.steps):
        for s in range(ops.N_STAGES):
            stage_ms[i, s] = timing.elapsed_ms(evs[i][s], evs[i][s + 1])
    block_ms_ev = np.array([timing.elapsed_ms(e[0], e[-1]) for e in evs])
    for e in evs:
        timing.destroy(e)

    ms_per_step = wall * 1e3 / args.steps
    flop = cfg.flop()
    gemm_in_flop = 2.0 * cfg.N * D * (3 * D + 2 * F)
    gemm_out_flop = 2.0 * cfg.N * (D + F) * D
    attn_flop = cfg.attn_flop()
    st = {name: float(stage_ms[:, i].mean()) for i, name in enumerate(ops.STAGES)}
    st_med = {name: float(np.median(stage_ms[:, i])) for i, name in enumerate(ops.STAGES)}
    tflops = flop / (ms_per_step * 1e-3) / 1e12
    gemm_in_tflops = gemm_in_flop / (st["gemm_in"] * 1e-3) / 1e12

    # parity of this exact configuration (weight set 0) against the oracle:
    # y, and the branch r (read with the residual and gate switched off)
    step(0)
    torch.cuda.synchronize()
    y_set0 = oracle.widen_bf16(ops.to_host_bits(y))
    r = torch.empty_like(x)
    ops.block_fwd(x, mod, pos, weights[0][0], weights[0][1], qs, ks,
                  ops.make_desc(cfg.n_tokens, flags=ops.DIT_F_NO_RESIDUAL | ops.DIT_F_NO_GATE),
                  y=r, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    r_set0 = oracle.widen_bf16(ops.to_host_bits(r))
    del r

    result = {
        "metric": "DiT joint-block fwd TFLOP/s & ms/block, 4096 img + 160 txt tokens, bf16",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_blocks": args.prewarm_blocks,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights; 4 rotating weight sets)",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}; width {D}, {cfg.n_heads}x{cfg.head_dim} "
                        f"heads, SwiGLU {F}, one parallel block forward",
            "N": cfg.N, "n_tokens": list(cfg.n_tokens), "gflop_per_block": round(flop / 1e9, 2),
        },
        "frac_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "block_ms_events_median": round(float(np.median(block_ms_ev)), 4),
        "block_ms_events_min": round(float(np.min(block_ms_ev)), 4),
        "stage_ms_mean": {k: round(v, 4) for k, v in st.items()},
        "stage_ms_median": {k: round(v, 4) for k, v in st_med.items()},
        "attn": {
            "ms": round(st["attn"], 4),
            "tflops": round(attn_flop / (st["attn"] * 1e-3) / 1e12, 2),
            "frac_mfma_peak": round(attn_flop / (st["attn"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        },
        "gemm_out_tflops": round(gemm_out_flop / (st["gemm_out"] * 1e-3) / 1e12, 2),
        "adaln_gbs": round(4.0 * cfg.N * D / (st["adaln"] * 1e-3) / 1e9, 1),
        "roofline": {
            "kernel": "input projection: gemm_kernel<EPI_IN> (q|k|v|SwiGLU, QK RMSNorm + RoPE "
                      "epilogue) + its split-tail fix-up, timed together",
            "bound": "mfma",
            "achieved": round(gemm_in_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_in_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(),
            "traffic_unit": "bytes per launch",
            "algorithmic": f"{gemm_in_flop / 1e9:.1f} GFLOP per launch = 2 N D (3D + 2F)",
        },
        "device": dev_name,
        "input_gen_s": round(t_gen, 1),
    }

    if not args.no_stack:
        result["stack_c5"] = stack_c5(torch, configs, ops, steps=3, warmup=1)
    if not args.no_fp8:
        result["block_fp8"] = block_fp8(torch, configs, ops, timing, cfg, x, mod, pos, qs, ks,
                                        weights, args.steps, args.warmup)
    if not args.no_stack:
        result["sampler_c5"] = sampler_c5(torch, configs, ops, steps=3, warmup=1)
    if not args.no_stack:
        result["stage1_c3"] = stage1_c3(torch, configs, ops, steps=5, warmup=4)
    if not args.no_long:
        result["block_c4"] = block_secondary(torch, configs, ops, timing, configs.C4, steps=10,
                                             warmup=2)
        result["block_edit2048"] = block_secondary(torch, configs, ops, timing,
                                                   configs.EDIT_2048, steps=5, warmup=1)

    if not args.no_cpu_baseline:
        ref, sec, threads, blas, n_blocks = cpu_baseline(d, cfg)
        result["cpu_baseline"] = {
            "value": round(flop / sec / 1e12, 5),
            "unit": "TFLOP/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"the full {cfg.name} block (N={cfg.N}) through oracle.block_ref in numpy "
                      f"float64, run {n_blocks} times ({n_blocks * sec:.1f} s wall, "
                      f"{sec:.2f} s per block), BLAS {blas}, host {cpu_model()}",
            "seconds_per_block": round(sec, 3),
            "cpu_model": cpu_model(),
        }
        result["parity"] = {
            "relL2_y": oracle.rel_l2(y_set0, ref["y"]),
            "relL2_r": oracle.rel_l2(r_set0, ref["r"]),
            "bound": 1e-2,
            **attn_parity(torch, oracle, inputs, ops, cfg.N),
        }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
