"""GPU tests of the two-stage stack with classifier-free guidance
(dit_stack_fwd) against the fp64 stack oracle."""
import numpy as np
import pytest
import torch

import oracle
from _gpu import require_gpu, widen
from flow_matching_diffusion_adaln_amd import configs, inputs, ops

pytestmark = pytest.mark.gpu

D, F, d, H = configs.WIDTH, configs.MLP_HIDDEN, configs.HEAD_DIM, configs.N_HEADS
DIMS = dict(n_heads=H, head_dim=d, mlp_hidden=F)
# stacked: each block's output is bf16-rounded and fed on; the guided result
# 4 cond - 3 neg adds the two branches' errors (which are correlated: both
# share the image stage), so the bound is the block's 1e-2 times the CFG
# amplification (|4| + |3|) / |4 - 3| = 7 on the branch difference, taken
# on the result as a whole
TOL_STACK = 2e-2


def tol_full_depth(n_blocks: int, scale: float) -> float:
    """Bound for the stack at its real depth.  Each block adds an error of
    its own (the bf16 storage of u, q, k, v, o, m and of its output; about
    2e-3 of the activation, the block's measured y error) that later blocks
    carry on, so over n_blocks independent additions the relative error
    grows like sqrt(n_blocks) times that; the guided result
    s cond - (s - 1) neg takes both branches' errors with weights s and
    s - 1 (root sum of squares for independent errors) on a result about
    the size of one branch.  The bound is twice that estimate."""
    amp = float(np.hypot(scale, scale - 1.0))
    return 2.0 * np.sqrt(n_blocks) * 2e-3 * amp


def log(msg):
    print(msg, flush=True)


def block_params(seed, kind_id, n_streams, zero_gate=False):
    key = (seed, 300 + kind_id)
    mod = inputs.normal_bf16((n_streams, 3, D), np.sqrt(0.1), *key, 1)
    if zero_gate:
        mod[:, 2, :] = 0
    return {
        "mod": mod,
        "w_in": inputs.normal_bf16((3 * D + 2 * F, D), 1.0 / np.sqrt(D), *key, 2),
        "w_out": inputs.normal_bf16((D, D + F), 1.0 / np.sqrt(D + F), *key, 3),
        "q_scale": inputs.f64_to_bf16_bits(np.ones(d)),
        "k_scale": inputs.f64_to_bf16_bits(np.ones(d)),
    }


def stack_inputs(n_img_side, n_txt, n_i, n_t, n_j, seed=0, zero_gate=False):
    n_img = n_img_side * n_img_side
    cfg = configs.BlockConfig("stack", 99, (configs.Stream("image", n_img, (n_img_side, n_img_side), 0.7),
                                            configs.Stream("text", n_txt)))
    pos = inputs.positions(cfg)
    x_img = inputs.normal_bf16((n_img, D), 1.0, seed, 401)
    x_c = inputs.normal_bf16((n_txt, D), 1.0, seed, 402)
    x_n = inputs.normal_bf16((n_txt, D), 1.0, seed, 403)
    blocks = ([block_params(seed, i, 1, zero_gate) for i in range(n_i)]
              + [block_params(seed, 10 + i, 1, zero_gate) for i in range(n_t)]
              + [block_params(seed, 20 + i, 2, zero_gate) for i in range(n_j)])
    return x_img, x_c, x_n, pos, blocks


def to_dev_blocks(blocks):
    return [{k: ops.to_device_bf16(v) for k, v in b.items()} for b in blocks]


def run_stack(x_img, x_c, x_n, pos, blocks, n_i, n_t, n_j, scale, x_ref=None, n_r=0):
    n_ref = 0 if x_ref is None else x_ref.shape[0]
    desc = ops.make_stack_desc(x_img.shape[0], x_c.shape[0], n_i, n_t, n_j, scale,
                               n_ref=n_ref, n_ref_blocks=n_r)
    v = ops.stack_fwd(desc, ops.to_device_bf16(x_img), ops.to_device_bf16(x_c),
                      None if x_n is None else ops.to_device_bf16(x_n),
                      torch.from_numpy(pos).cuda(), to_dev_blocks(blocks),
                      x_ref=None if x_ref is None else ops.to_device_bf16(x_ref))
    torch.cuda.synchronize()
    return widen(v)


@pytest.mark.parametrize("scale", [4.0, 1.0])
def test_stack_cfg_parity(scale):
    require_gpu()
    n_i, n_t, n_j = 1, 1, 2
    x_img, x_c, x_n, pos, blocks = stack_inputs(16, 80, n_i, n_t, n_j)
    log(f"stack 256 img + 80 txt, blocks {n_i}+{n_t}+{n_j}, cfg {scale}")
    got = run_stack(x_img, x_c, x_n if scale != 1.0 else None, pos, blocks, n_i, n_t, n_j, scale)
    want = oracle.stack_cfg_ref(x_img, x_c, x_n, pos, blocks[:n_i], blocks[n_i:n_i + n_t],
                                blocks[n_i + n_t:], DIMS, scale)
    e = oracle.rel_l2(got, want)
    log(f"  relL2 {e:.3e}")
    assert e <= TOL_STACK


def test_stack_zero_gates_return_the_image_tokens():
    require_gpu()
    x_img, x_c, x_n, pos, blocks = stack_inputs(8, 40, 1, 1, 1, seed=3, zero_gate=True)
    got = run_stack(x_img, x_c, x_n, pos, blocks, 1, 1, 1, 4.0)
    assert np.array_equal(got, oracle.widen_bf16(x_img))


def test_stack_identical_prompts_give_the_conditional_branch():
    require_gpu()
    x_img, x_c, _, pos, blocks = stack_inputs(8, 40, 1, 1, 1, seed=4)
    a = run_stack(x_img, x_c, x_c, pos, blocks, 1, 1, 1, 4.0)
    b = run_stack(x_img, x_c, None, pos, blocks, 1, 1, 1, 1.0)
    # neg == cond bitwise, so neg + 4 (cond - neg) == cond exactly
    assert np.array_equal(a, b)


def test_stack_with_two_references_parity():
    # 256 image tokens | two 8 x 8 references (l = 1, 2) | 80 text tokens;
    # blocks: 1 image, 1 reference, 1 text, 2 joint (three-stream modulation)
    require_gpu()
    n_i, n_r, n_t, n_j = 1, 1, 1, 2
    x_img, x_c, x_n, p, _ = stack_inputs(16, 80, 0, 0, 0, seed=6)
    x_ref = inputs.normal_bf16((128, D), 1.0, 6, 404)
    pr = np.zeros((128, 4), dtype=np.int32)
    i = np.arange(128)
    pr[:, 1], pr[:, 2], pr[:, 3] = (i % 64) // 8, i % 8, 1 + i // 64
    pos = np.ascontiguousarray(np.concatenate([p[:256], pr, p[256:]]))
    blocks = ([block_params(6, 0, 1)] + [block_params(6, 5, 1)] + [block_params(6, 10, 1)]
              + [block_params(6, 20 + j, 3) for j in range(n_j)])
    log("stack 256 img + 2x64 ref + 80 txt, blocks 1+1+1+2, cfg 4.0")
    got = run_stack(x_img, x_c, x_n, pos, blocks, n_i, n_t, n_j, 4.0, x_ref=x_ref, n_r=n_r)
    want = oracle.stack_cfg_ref(x_img, x_c, x_n, pos, blocks[:1], blocks[2:3], blocks[3:],
                                DIMS, 4.0, x_ref=x_ref, ref_blocks=blocks[1:2])
    e = oracle.rel_l2(got, want)
    log(f"  relL2 {e:.3e}")
    assert e <= TOL_STACK


@pytest.mark.parametrize("scale", [1.0, 4.0])
def test_stack_full_depth_parity(scale):
    # the real depth of one denoise step: 5 image and 5 text stage-1 blocks
    # and 28 joint blocks, each with its own weights, at full width on an
    # 8 x 8 image grid and 80 text tokens
    require_gpu()
    n_i, n_t, n_j = 5, 5, 28
    x_img, x_c, x_n, pos, blocks = stack_inputs(8, 80, n_i, n_t, n_j, seed=9)
    log(f"stack 64 img + 80 txt, blocks {n_i}+{n_t}+{n_j}, cfg {scale}")
    got = run_stack(x_img, x_c, x_n if scale != 1.0 else None, pos, blocks, n_i, n_t, n_j, scale)
    want = oracle.stack_cfg_ref(x_img, x_c, x_n, pos, blocks[:n_i], blocks[n_i:n_i + n_t],
                                blocks[n_i + n_t:], DIMS, scale)
    e = oracle.rel_l2(got, want)
    # a branch runs 5 + 28 blocks (its text stage-1 and the joint blocks; the
    # image stage-1 blocks are shared by both branches)
    tol = tol_full_depth(n_t + n_j, scale)
    log(f"  relL2 {e:.3e} (bound {tol:.3e})")
    assert e <= tol


def dev_stack_args(x_img, x_c, x_n, pos, blocks):
    return (ops.to_device_bf16(x_img), ops.to_device_bf16(x_c), ops.to_device_bf16(x_n),
            torch.from_numpy(pos).cuda(), to_dev_blocks(blocks))


def test_stack_side_stream_matches_serial():
    # DIT_STACK_TEXT_SIDE_STREAM runs the stage-1 text blocks of both branches
    # on the library's second stream, beside the image blocks: the same
    # kernels on the same rows, so the result is bitwise the serial one
    require_gpu()
    n_i, n_t, n_j = 2, 2, 2
    x_img, x_c, x_n, pos, blocks = stack_inputs(16, 80, n_i, n_t, n_j, seed=10)
    xi, xc, xn, p, bl = dev_stack_args(x_img, x_c, x_n, pos, blocks)
    out = []
    for side in (False, True):
        desc = ops.make_stack_desc(256, 80, n_i, n_t, n_j, 4.0, side_stream=side)
        log(f"stack 256 img + 80 txt, blocks {n_i}+{n_t}+{n_j}, side stream {side}")
        v = torch.full((256, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        ops.stack_fwd(desc, xi, xc, xn, p, bl, v_img=v)
        torch.cuda.synchronize()
        out.append(v.cpu())
    assert torch.equal(out[0], out[1])


@pytest.mark.parametrize("side", [False, True])
def test_stack_graph_replays_match_eager(side):
    # The guided stack captured in a HIP graph through torch's capture of the
    # caller's stream (with the side stream, its fork and join events bring
    # it into the capture), replayed three times with eager launches and
    # synchronizations between the replays and a poisoned output before
    # each: every replay equals the eager result bitwise.
    require_gpu()
    n_i, n_t, n_j = 1, 1, 2
    x_img, x_c, x_n, pos, blocks = stack_inputs(8, 80, n_i, n_t, n_j, seed=11)
    xi, xc, xn, p, bl = dev_stack_args(x_img, x_c, x_n, pos, blocks)
    desc = ops.make_stack_desc(64, 80, n_i, n_t, n_j, 4.0, side_stream=side)
    ws = torch.empty(ops.stack_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    v_e = torch.empty((64, D), dtype=torch.bfloat16, device="cuda")
    v_g = torch.empty_like(v_e)
    log(f"stack graph, side stream {side}")
    ops.stack_fwd(desc, xi, xc, xn, p, bl, v_img=v_e, workspace=ws)
    torch.cuda.synchronize()
    want = v_e.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.stack_fwd(desc, xi, xc, xn, p, bl, v_img=v_g, workspace=ws)
    for r in range(3):
        v_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(v_g, want), f"replay {r}"
        # eager work between replays, on the same workspace
        ops.stack_fwd(desc, xi, xc, xn, p, bl, v_img=v_e, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(v_e, want), f"eager after replay {r}"
