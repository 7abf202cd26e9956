"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes its workspace, and rejects bad arguments on the host
before any launch (every call here fails validation or is an empty call, so
no kernel is ever enqueued)."""
import ctypes
import os
import re

import numpy as np
import pytest

from flow_matching_diffusion_adaln_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, HIP, ARG = 0, -1, -2, -3, -4, -5, -6, -7
P = 1 << 20       # fake, 16-byte aligned "device" addresses: never dereferenced
BAD = P + 8       # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        pytest.skip("libdit.so not built")
    return ops.load_library()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(ops.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout_matches_header():
    # int32 x 8 + float x 3 + uint32 = 48 bytes, no padding
    assert ctypes.sizeof(ops.BlockDesc) == 48


def test_status_strings(lib):
    for rc in (OK, NULL, SHAPE, UNSUP, ALIGN, WS, HIP, ARG):
        s = lib.dit_status_str(rc).decode()
        assert s.startswith("DIT_OK" if rc == 0 else "DIT_ERR_")
    assert lib.dit_status_str(-99).decode() == "DIT_ERR_UNKNOWN"


def ws(lib, desc):
    n = ctypes.c_size_t(0)
    rc = lib.dit_block_workspace_bytes(ctypes.byref(desc), ctypes.byref(n))
    return rc, n.value


def test_workspace_bytes(lib):
    rc, n = ws(lib, ops.make_desc([4096, 160]))
    assert rc == OK
    N, D, F = 4256, 3072, 9216
    # u, q, k, v [N, D] and [o | m] [N, D + F] in bf16, plus the fixed fp32
    # scratch of the GEMMs' split tail (two 256 x 256 tiles for each of 256
    # pieces; attention's split partials reuse it) and 1024 attention counters
    split = 2 * 256 * 256 * 256 * 4
    counters = 1024 * 4
    assert n >= 2 * (4 * N * D + N * (D + F)) + split + counters
    assert n < 2 * (4 * N * D + N * (D + F)) + split + counters + 7 * 256
    rc, n8352 = ws(lib, ops.make_desc([4096, 4096, 160]))
    assert rc == OK and n8352 > 400e6
    assert ws(lib, ops.make_desc([0]))[0] == OK


@pytest.mark.parametrize("field,value,want", [
    ("n_streams", 0, SHAPE), ("n_streams", 4, SHAPE),
    ("head_dim", 64, SHAPE),            # 24 x 64 != 3072
    ("width", 3000, SHAPE),
    ("n_heads", 0, SHAPE),
    ("mlp_hidden", 9200, UNSUP),
    ("rope_theta", 0.0, ARG), ("ln_eps", -1.0, ARG), ("qk_eps", float("nan"), ARG),
    ("flags", 4, ARG),
])
def test_desc_validation(lib, field, value, want):
    d = ops.make_desc([4096, 160])
    setattr(d, field, value)
    assert ws(lib, d)[0] == want


def test_desc_head_dim_and_tokens(lib):
    d = ops.make_desc([256, 80], width=6 * 64, n_heads=6, head_dim=64)
    assert ws(lib, d)[0] == UNSUP          # head_dim 64 is not implemented
    d = ops.make_desc([256, 80], width=2 * 128, n_heads=2)
    assert ws(lib, d)[0] == UNSUP          # heads must come in multiples of 4
    d = ops.make_desc([-1, 80])
    assert ws(lib, d)[0] == SHAPE
    d = ops.make_desc([131072, 1])
    assert ws(lib, d)[0] == SHAPE          # above DIT_MAX_TOKENS
    assert lib.dit_block_workspace_bytes(None, ctypes.byref(ctypes.c_size_t())) == NULL


def fwd(lib, desc, ptrs=None, ws_bytes=None, events=None):
    p = [P] * 9 if ptrs is None else ptrs
    if ws_bytes is None:
        ws_bytes = ws(lib, desc)[1]
    args = [ctypes.byref(desc)] + [ctypes.c_void_p(v) if v else None for v in p] + \
        [ctypes.c_size_t(ws_bytes), None]
    if events is None:
        return lib.dit_block_fwd(*args)
    return lib.dit_block_fwd_events(*args, events)


def test_block_fwd_host_errors(lib):
    d = ops.make_desc([256, 80])
    for i in range(9):
        p = [P + (1 << 30) * j for j in range(9)]
        p[i] = 0
        assert fwd(lib, d, p) == NULL, i
    for i in range(9):
        p = [P + (1 << 30) * j for j in range(9)]
        p[i] = BAD + (1 << 30) * i
        assert fwd(lib, d, p) == ALIGN, i
    p = [P + (1 << 30) * j for j in range(9)]
    assert fwd(lib, d, p, ws_bytes=ws(lib, d)[1] - 1) == WS
    # y overlapping the workspace
    p[8] = p[7]
    assert fwd(lib, d, p) == ARG
    # events array required by the events variant, and each event non-null
    p = [P + (1 << 30) * j for j in range(9)]
    ev = (ctypes.c_void_p * 6)(*([1] * 5 + [0]))
    assert fwd(lib, d, p, events=ev) == NULL


def test_empty_block_is_a_noop(lib):
    d = ops.make_desc([0, 0])
    assert fwd(lib, d, [0] * 9, ws_bytes=0) == OK


def test_attn_host_errors(lib):
    c = ctypes.c_void_p
    f = lib.dit_attn_fwd
    a, b, cc, o = c(P), c(P + (1 << 30)), c(P + (2 << 30)), c(P + (3 << 30))
    assert f(100, 24, 64, a, b, cc, o, 0.1, None) == UNSUP
    assert f(-1, 24, 128, a, b, cc, o, 0.1, None) == SHAPE
    assert f(100, 0, 128, a, b, cc, o, 0.1, None) == SHAPE
    assert f(100, 24, 128, None, b, cc, o, 0.1, None) == NULL
    assert f(100, 24, 128, c(BAD), b, cc, o, 0.1, None) == ALIGN
    assert f(100, 24, 128, a, b, cc, o, 0.0, None) == ARG
    assert f(100, 24, 128, a, b, cc, o, float("inf"), None) == ARG
    assert f(100, 24, 128, a, b, cc, c(P + 4096), 0.1, None) == ARG   # o overlaps q
    assert f(0, 24, 128, None, None, None, None, 0.1, None) == OK      # empty call


def test_attn_ws_host_errors(lib):
    c = ctypes.c_void_p
    n = ctypes.c_size_t(0)
    assert lib.dit_attn_workspace_bytes(4256, 24, 128, ctypes.byref(n)) == OK
    need = n.value
    # the split partials of up to 256 shares (two fp32 parts of 256 queries x
    # 128 dims plus row sums and maxima each) and their counters
    assert need >= 256 * 2 * 8 * 17 * 64 * 16 + 256 * 4
    assert lib.dit_attn_workspace_bytes(4256, 24, 64, ctypes.byref(n)) == UNSUP
    assert lib.dit_attn_workspace_bytes(4256, 24, 128, None) == NULL
    f = lib.dit_attn_fwd_ws
    a, b, cc, o, w = (c(P + (i << 30)) for i in range(5))
    assert f(100, 24, 128, a, b, cc, o, 0.1, None, need, None) == NULL
    assert f(100, 24, 128, a, b, cc, o, 0.1, c(BAD + (4 << 30)), need, None) == ALIGN
    assert f(100, 24, 128, a, b, cc, o, 0.1, w, need - 1, None) == WS
    assert f(100, 24, 128, a, b, cc, o, 0.1, c(P + (3 << 30) + 4096), need, None) == ARG
    assert f(100, 24, 64, a, b, cc, o, 0.1, w, need, None) == UNSUP
    assert f(0, 24, 128, None, None, None, None, 0.1, None, 0, None) == OK


def test_rope_host_errors(lib):
    c = ctypes.c_void_p
    f = lib.rope4_apply
    q, k, pos, g = c(P), c(P + (1 << 30)), c(P + (2 << 30)), c(P + (3 << 30))
    assert f(10, 24, 96, q, k, pos, 1e4, None, None, 1e-6, None) == UNSUP
    assert f(10, 24, 128, q, k, pos, 1e4, g, None, 1e-6, None) == ARG
    assert f(10, 24, 128, q, k, pos, -1.0, None, None, 1e-6, None) == ARG
    assert f(10, 24, 128, None, k, pos, 1e4, None, None, 1e-6, None) == NULL
    assert f(10, 24, 128, q, k, c(BAD), 1e4, None, None, 1e-6, None) == ALIGN
    assert f(0, 24, 128, None, None, None, 1e4, None, None, 1e-6, None) == OK


def test_adaln_host_errors(lib):
    c = ctypes.c_void_p
    f = lib.adaln_mod
    n2 = (ctypes.c_int32 * 2)(256, 80)
    x, m, o = c(P), c(P + (1 << 30)), c(P + (2 << 30))
    assert f(0, n2, 3072, x, m, o, 1e-6, None) == SHAPE
    assert f(2, None, 3072, x, m, o, 1e-6, None) == NULL
    assert f(2, n2, 3000, x, m, o, 1e-6, None) == UNSUP
    assert f(2, n2, 16384, x, m, o, 1e-6, None) == UNSUP
    assert f(2, n2, 3072, x, None, o, 1e-6, None) == NULL
    assert f(2, n2, 3072, x, m, c(BAD), 1e-6, None) == ALIGN
    assert f(2, n2, 3072, x, m, o, -1.0, None) == ARG
    bad = (ctypes.c_int32 * 2)(256, -80)
    assert f(2, bad, 3072, x, m, o, 1e-6, None) == SHAPE
    empty = (ctypes.c_int32 * 2)(0, 0)
    assert f(2, empty, 3072, None, None, None, 1e-6, None) == OK


# ------------------------------------------------------------- dit_stack_* --

def stack_ws(lib, d):
    n = ctypes.c_size_t(0)
    rc = lib.dit_stack_workspace_bytes(ctypes.byref(d), ctypes.byref(n))
    return rc, n.value


def test_stack_struct_layout():
    assert ctypes.sizeof(ops.StackDesc) == 64
    assert ctypes.sizeof(ops.BlockParams) == 40


def test_stack_workspace_bytes(lib):
    d = ops.make_stack_desc(4096, 160, 5, 5, 28, 4.0)
    rc, n = stack_ws(lib, d)
    assert rc == OK
    rc_b, nb = ws(lib, ops.make_desc([4096, 160]))
    # the block workspace at N = 4256 plus one [N, D] bf16 buffer per branch
    assert n == nb + 2 * 4256 * 3072 * 2
    assert lib.dit_stack_workspace_bytes(None, ctypes.byref(ctypes.c_size_t())) == NULL
    # with 4096 reference tokens the joint sequence is [image | reference | text]
    rc, n = stack_ws(lib, ops.make_stack_desc(4096, 160, 5, 5, 28, 4.0, n_ref=4096,
                                              n_ref_blocks=5))
    rc_b, nb = ws(lib, ops.make_desc([4096, 4096, 160]))
    assert rc == OK and n == nb + 2 * 8352 * 3072 * 2
    # the side stream's text blocks take a block workspace of their own
    rc, n_side = stack_ws(lib, ops.make_stack_desc(4096, 160, 5, 5, 28, 4.0, side_stream=True))
    rc_b, nb = ws(lib, ops.make_desc([4096, 160]))
    rc_t, nt = ws(lib, ops.make_desc([160]))
    assert rc == OK and n_side == nb + 2 * 4256 * 3072 * 2 + nt


@pytest.mark.parametrize("field,value,want", [
    ("n_img", 0, SHAPE), ("n_txt", 0, SHAPE), ("n_img_blocks", -1, SHAPE),
    ("n_joint_blocks", 2000, SHAPE), ("width", 3000, SHAPE), ("head_dim", 64, SHAPE),
    ("cfg_scale", float("nan"), ARG), ("qk_eps", -1.0, ARG), ("n_ref", -1, SHAPE),
    ("n_ref_blocks", 1, SHAPE),  # reference blocks without reference tokens
    ("n_ref", 131072, SHAPE),  # the joint sequence above DIT_MAX_TOKENS
    ("flags", 2, ARG)])  # an unknown flag bit
def test_stack_desc_validation(lib, field, value, want):
    d = ops.make_stack_desc(256, 80, 1, 1, 2, 4.0)
    setattr(d, field, value)
    assert stack_ws(lib, d)[0] == want


def stack_call(lib, d, x_img=P, x_c=P + (1 << 30), x_n=P + (2 << 30), pos=P + (3 << 30),
               blocks="ok", v=P + (4 << 30), wsp=P + (5 << 30), ws_bytes=None,
               x_ref=P + (1 << 29)):
    n_blocks = d.n_img_blocks + d.n_ref_blocks + d.n_txt_blocks + d.n_joint_blocks
    arr = (ops.BlockParams * max(n_blocks, 1))()
    for i in range(n_blocks):
        for j, name in enumerate(("mod", "w_in", "w_out", "q_scale", "k_scale")):
            setattr(arr[i], name, P + ((6 + 5 * i + j) << 30))
    if blocks == "bad_null":
        arr[n_blocks - 1].w_out = None
    elif blocks == "bad_align":
        arr[0].q_scale = BAD
    if ws_bytes is None:
        ws_bytes = stack_ws(lib, d)[1]
    c = ctypes.c_void_p
    return lib.dit_stack_fwd(ctypes.byref(d), c(x_img) if x_img else None,
                             c(x_ref) if x_ref else None, c(x_c) if x_c else None,
                             c(x_n) if x_n else None,
                             c(pos) if pos else None, None if blocks is None else arr,
                             c(v) if v else None, c(wsp) if wsp else None,
                             ctypes.c_size_t(ws_bytes), None)


def test_stack_fwd_host_errors(lib):
    d = ops.make_stack_desc(256, 80, 1, 1, 2, 4.0)
    assert stack_call(lib, d, x_img=0) == NULL
    assert stack_call(lib, d, x_n=0) == NULL          # guided: the negative branch is needed
    assert stack_call(lib, d, pos=0) == NULL
    assert stack_call(lib, d, blocks=None) == NULL
    assert stack_call(lib, d, blocks="bad_null") == NULL   # the last block is checked up front
    assert stack_call(lib, d, blocks="bad_align") == ALIGN
    assert stack_call(lib, d, x_c=BAD) == ALIGN
    assert stack_call(lib, d, ws_bytes=stack_ws(lib, d)[1] - 1) == WS
    assert stack_call(lib, d, v=P + (5 << 30)) == ARG      # output inside the workspace
    # no references: a null x_ref passes the pointer checks (stopped here by the workspace)
    assert stack_call(lib, d, x_ref=0, ws_bytes=stack_ws(lib, d)[1] - 1) == WS
    r = ops.make_stack_desc(256, 80, 1, 1, 2, 4.0, n_ref=64, n_ref_blocks=1)
    assert stack_call(lib, r, x_ref=0) == NULL
    assert stack_call(lib, r, x_ref=BAD) == ALIGN
    assert stack_call(lib, r, blocks="bad_null") == NULL


# ---- sampler ---------------------------------------------------------------------

def test_sampler_struct_layout():
    assert ctypes.sizeof(ops.ModelDesc) == 72
    assert ctypes.sizeof(ops.BlockWeights) == 32
    assert ctypes.sizeof(ops.ModelWeights) == 23 * 8


def test_flow_sigmas_match_the_oracle_and_the_pages_count(lib):
    import oracle
    for n, a in ((50, 6.93), (16, 6.93), (10, 3.0), (1, 6.93), (7, 1.0)):
        got = np.array(ops.flow_sigmas(n, a))
        want = oracle.flow_sigmas(n, a)
        assert got[0] == 1.0 and got[-1] == 0.0
        assert np.allclose(got, want, rtol=1e-15, atol=0)
    assert int((np.array(ops.flow_sigmas(50, 6.93))[:50] > 0.5).sum()) == 44
    out = (ctypes.c_double * 4)()
    assert lib.dit_flow_sigmas(0, 6.93, out) == SHAPE
    assert lib.dit_flow_sigmas(3, float("nan"), out) == ARG
    assert lib.dit_flow_sigmas(3, -1.0, out) == ARG
    assert lib.dit_flow_sigmas(3, 6.93, None) == NULL


def model_desc(n_img=256, n_ref=0, n_txt=80, blocks=(1, 0, 1, 2), scale=4.0, **kw):
    st = ops.make_stack_desc(n_img, n_txt, blocks[0], blocks[2], blocks[3], scale, n_ref=n_ref,
                             n_ref_blocks=blocks[1])
    return ops.make_model_desc(st, **kw)


def sampler_ws(lib, d):
    n = ctypes.c_size_t(0)
    rc = lib.dit_sampler_workspace_bytes(ctypes.byref(d), ctypes.byref(n))
    return rc, n.value


def test_sampler_workspace_bytes(lib):
    d = model_desc(4096, 0, 160)
    rc, n = sampler_ws(lib, d)
    assert rc == OK
    _, ns = stack_ws(lib, d.stack)
    # the stack's workspace plus prepared text rows for both prompts, the
    # timestep path, the normalized image rows and two velocity buffers
    extra = 2 * 160 * 3072 * 2 + 4 * 256 * 2 + (2 + 2 + 3 * 3 + 9 + 2) * 3072 * 2 \
        + 4096 * 3072 * 2 + 2 * 4096 * 128 * 2
    assert ns + extra <= n <= ns + extra + 20 * 256
    assert sampler_ws(lib, model_desc(latent_ch=100))[0] == UNSUP
    assert sampler_ws(lib, model_desc(text_dim=20))[0] == UNSUP
    assert sampler_ws(lib, model_desc(latent_ch=0))[0] == SHAPE
    assert sampler_ws(lib, model_desc(n_img=0))[0] == SHAPE


def fake_weights(d, null=None, bad=None):
    w = ops.ModelWeights()
    addr = [P + (40 << 30)]

    def nxt():
        addr[0] += 1 << 28
        return addr[0]
    for name in ops.MODEL_TENSORS + ("out_mod_w", "out_mod_b", "out_w", "out_b"):
        setattr(w, name, nxt())
    for g in range(ops.N_GROUPS):
        w.mod_w[g], w.mod_b[g] = nxt(), nxt()
    st = d.stack
    n = st.n_img_blocks + st.n_ref_blocks + st.n_txt_blocks + st.n_joint_blocks
    arr = (ops.BlockWeights * max(n, 1))()
    for i in range(n):
        for name in ops.BLOCK_WEIGHTS:
            setattr(arr[i], name, nxt())
    w.blocks = arr
    if null == "last_block":
        arr[n - 1].k_scale = None
    elif null is not None:
        setattr(w, null, None)
    if bad is not None:
        setattr(w, bad, BAD)
    return w, arr


def prepare_call(lib, d, w, tc=P, tn=P + (1 << 30), ref=P + (2 << 30), pos=P + (3 << 30),
                 wsp=P + (4 << 30), ws_bytes=None):
    c = ctypes.c_void_p
    if ws_bytes is None:
        ws_bytes = sampler_ws(lib, d)[1]
    return lib.dit_sampler_prepare(ctypes.byref(d), None if w is None else ctypes.byref(w),
                                   c(tc) if tc else None, c(tn) if tn else None,
                                   c(ref) if ref else None, c(pos) if pos else None,
                                   c(wsp) if wsp else None, ctypes.c_size_t(ws_bytes), None)


def step_call(lib, d, w, z=P, sigma=1.0, sigma_next=0.9, pos=P + (3 << 30), v=None,
              wsp=P + (4 << 30), ws_bytes=None):
    c = ctypes.c_void_p
    if ws_bytes is None:
        ws_bytes = sampler_ws(lib, d)[1]
    return lib.dit_sampler_step(ctypes.byref(d), None if w is None else ctypes.byref(w),
                                c(z) if z else None, sigma, sigma_next, c(pos) if pos else None,
                                c(v) if v else None, c(wsp) if wsp else None,
                                ctypes.c_size_t(ws_bytes), None)


def test_sampler_host_errors(lib):
    d = model_desc()
    w, _keep = fake_weights(d)
    small = sampler_ws(lib, d)[1] - 1
    # every error is found before anything is launched
    assert prepare_call(lib, d, None) == NULL
    assert prepare_call(lib, d, w, tc=0) == NULL
    assert prepare_call(lib, d, w, tn=0) == NULL           # guided: the negative prompt is needed
    assert prepare_call(lib, d, w, tc=BAD) == ALIGN
    assert prepare_call(lib, d, w, ws_bytes=small) == WS
    # without references ref_latent, ref_in_* and the reference group may be null
    w2, _k2 = fake_weights(d, null="ref_in_w")
    w2.mod_w[1] = None
    assert prepare_call(lib, d, w2, ref=0, ws_bytes=small) == WS
    for name in ("img_in_w", "txt_in_b", "t_w2", "out_w", "out_mod_b", "last_block"):
        wn, _kn = fake_weights(d, null=name)
        assert prepare_call(lib, d, wn) == NULL, name
        assert step_call(lib, d, wn) == NULL, name
    wb, _kb = fake_weights(d, bad="t_b1")
    assert step_call(lib, d, wb) == ALIGN
    r = model_desc(n_ref=64, blocks=(1, 1, 1, 2))
    wr, _kr = fake_weights(r, null="ref_in_b")
    assert prepare_call(lib, r, wr) == NULL
    wr, _kr = fake_weights(r)
    assert prepare_call(lib, r, wr, ref=0) == NULL
    assert step_call(lib, d, w, z=0) == NULL
    assert step_call(lib, d, w, sigma=float("inf")) == ARG
    assert step_call(lib, d, w, ws_bytes=small) == WS
    # the sampler's text blocks run once, in prepare: no side-stream flag
    ds = model_desc()
    ds.stack.flags = ops.DIT_STACK_TEXT_SIDE_STREAM
    assert sampler_ws(lib, ds)[0] == ARG
    assert step_call(lib, d, w, z=P + (4 << 30)) == ARG     # latent inside the workspace
    assert step_call(lib, d, w, v=P) == ARG                 # velocity over the latent
    assert step_call(lib, d, w, v=BAD) == ALIGN


def test_linear_and_sinusoid_host_errors(lib):
    c = ctypes.c_void_p
    assert lib.dit_linear(4, 30, 16, c(P), c(P + (1 << 30)), None, 0, c(P + (2 << 30)), None) == UNSUP
    assert lib.dit_linear(4, 32, 10, c(P), c(P + (1 << 30)), None, 0, c(P + (2 << 30)), None) == UNSUP
    assert lib.dit_linear(-1, 32, 16, c(P), c(P + (1 << 30)), None, 0, c(P + (2 << 30)), None) == SHAPE
    assert lib.dit_linear(4, 32, 16, c(P), c(P + (1 << 30)), None, 2, c(P + (2 << 30)), None) == ARG
    assert lib.dit_linear(4, 32, 16, None, c(P + (1 << 30)), None, 0, c(P + (2 << 30)), None) == NULL
    assert lib.dit_linear(4, 32, 16, c(BAD), c(P + (1 << 30)), None, 0, c(P + (2 << 30)), None) == ALIGN
    assert lib.dit_linear(4, 32, 16, c(P), c(P + (1 << 30)), None, 0, c(P + 64), None) == ARG
    assert lib.dit_linear(0, 32, 16, None, None, None, 0, None, None) == OK   # nothing to do
    t = (ctypes.c_double * 2)(0.5, float("nan"))
    assert lib.dit_time_sinusoid(0, t, c(P), None) == SHAPE
    assert lib.dit_time_sinusoid(5, t, c(P), None) == SHAPE
    assert lib.dit_time_sinusoid(2, t, c(P), None) == ARG
    assert lib.dit_time_sinusoid(1, t, None, None) == NULL
    assert lib.dit_time_sinusoid(1, t, c(BAD), None) == ALIGN


# ---- FP8 projections ---------------------------------------------------------------

def test_fp8_workspace_bytes(lib):
    d = ops.make_desc([4096, 160])
    n = ctypes.c_size_t(0)
    assert lib.dit_block_fp8_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == OK
    _, nb = ws(lib, d)
    # the bf16 block's workspace plus u and [o | m] in e4m3 and their row scales
    extra = 4256 * 3072 + 4256 * (3072 + 9216) + 2 * 4256 * 4
    assert nb + extra <= n.value <= nb + extra + 4 * 256
    assert lib.dit_block_fp8_workspace_bytes(None, ctypes.byref(n)) == NULL


def fp8_call(lib, d, ptrs=None, ws_bytes=None):
    p = [P + (i << 30) for i in range(11)] if ptrs is None else ptrs
    if ws_bytes is None:
        n = ctypes.c_size_t(0)
        lib.dit_block_fp8_workspace_bytes(ctypes.byref(d), ctypes.byref(n))
        ws_bytes = n.value
    c = [ctypes.c_void_p(v) if v else None for v in p]
    return lib.dit_block_fwd_fp8(ctypes.byref(d), *c[:10], c[10], ctypes.c_size_t(ws_bytes),
                                 None)


def test_fp8_host_errors(lib):
    d = ops.make_desc([256, 80])
    good = [P + (i << 30) for i in range(11)]
    for i in range(11):  # x, mod, pos, w_in8, w_in_scale, w_out8, w_out_scale, q/k scale, y, ws
        bad = list(good)
        bad[i] = 0
        assert fp8_call(lib, d, bad) == NULL, i
        bad[i] = BAD
        assert fp8_call(lib, d, bad) == ALIGN, i
    n = ctypes.c_size_t(0)
    lib.dit_block_fp8_workspace_bytes(ctypes.byref(d), ctypes.byref(n))
    assert fp8_call(lib, d, ws_bytes=n.value - 1) == WS
    over = list(good)
    over[9] = good[10]                                   # y inside the workspace
    assert fp8_call(lib, d, over) == ARG
    assert fp8_call(lib, ops.make_desc([256, 80], width=3000)) == SHAPE
    assert fp8_call(lib, ops.make_desc([0])) == OK       # nothing to do
    c = ctypes.c_void_p
    assert lib.dit_quantize_rows_fp8(4, 12, c(P), c(P + (1 << 30)), c(P + (2 << 30)), None) == UNSUP
    assert lib.dit_quantize_rows_fp8(-1, 16, c(P), c(P + (1 << 30)), c(P + (2 << 30)), None) == SHAPE
    assert lib.dit_quantize_rows_fp8(4, 16, None, c(P + (1 << 30)), c(P + (2 << 30)), None) == NULL
    assert lib.dit_quantize_rows_fp8(4, 16, c(P), c(BAD), c(P + (2 << 30)), None) == ALIGN
    assert lib.dit_quantize_rows_fp8(4, 16, c(P), c(P + 64), c(P + (2 << 30)), None) == ARG
    assert lib.dit_quantize_rows_fp8(0, 16, None, None, None, None) == OK


def test_struct_layouts_match_a_c_compiler(tmp_path):
    # sizes and field offsets of every struct in include/dit.h, as gcc lays
    # them out, against the ctypes mirrors the binding passes by pointer
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    rocm_inc = "/opt/rocm/include"
    if gcc is None or not os.path.exists(os.path.join(rocm_inc, "hip", "hip_runtime_api.h")):
        pytest.skip("gcc or the HIP headers are not available")
    structs = {"dit_block_desc": ops.BlockDesc, "dit_stack_desc": ops.StackDesc,
               "dit_block_params": ops.BlockParams, "dit_model_desc": ops.ModelDesc,
               "dit_block_weights": ops.BlockWeights, "dit_model_weights": ops.ModelWeights}
    lines = ["#define __HIP_PLATFORM_AMD__ 1", "#include <stdio.h>", "#include <stddef.h>",
             '#include "dit.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    r = subprocess.run([gcc, "-std=c11", "-I", os.path.dirname(HEADER), "-I", rocm_inc,
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True,
                               check=True).stdout.splitlines():
        name, field, val = line.split()
        got[(name, field)] = int(val)
    for cname, cls in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert got[(cname, fname)] == getattr(cls, fname).offset, (cname, fname)


def test_noalloc_scratch_and_host_errors(lib):
    n = ctypes.c_size_t(0)
    assert lib.dit_block_noalloc_scratch_bytes(ctypes.byref(n)) == OK
    assert lib.dit_block_noalloc_scratch_bytes(None) == NULL
    # the scratch holds exactly the workspace of the largest sequence it serves
    assert ws(lib, ops.make_desc([ops.NOALLOC_MAX_TOKENS]))[1] == n.value
    assert ws(lib, ops.make_desc([4096, 256]))[1] <= n.value
    text = open(HEADER).read()
    assert re.search(r"#define DIT_NOALLOC_MAX_TOKENS %d\b" % ops.NOALLOC_MAX_TOKENS, text)

    def call(desc, ptrs):
        args = [ctypes.byref(desc)] + [ctypes.c_void_p(v) if v else None for v in ptrs] + [None]
        return lib.dit_block_fwd_noalloc(*args)

    p = [P + (1 << 30) * j for j in range(8)]
    # one token too many (or a wider block that no longer fits) is refused
    # before the device is touched
    assert call(ops.make_desc([ops.NOALLOC_MAX_TOKENS + 1]), p) == WS
    assert call(ops.make_desc([4096, 257]), p) == WS
    assert call(ops.make_desc([4096], width=4096, n_heads=32), p) == WS
    for i in range(8):
        q = list(p)
        q[i] = 0
        assert call(ops.make_desc([256, 80]), q) == NULL, i
        q[i] = BAD + (1 << 30) * i
        assert call(ops.make_desc([256, 80]), q) == ALIGN, i
    # shape errors and the empty call come first, as in dit_block_fwd
    assert call(ops.make_desc([256, 80], head_dim=64, n_heads=48), p) == UNSUP
    assert call(ops.make_desc([0, 0]), [0] * 8) == OK
