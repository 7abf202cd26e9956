"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes its workspace, and rejects bad arguments on the host
before any launch (every call here fails validation or is an empty call, so
no kernel is ever enqueued)."""
import ctypes
import os
import re

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
    # scratch of the GEMMs' split tail (two 256 x 256 tiles for each of 256 pieces)
    split = 2 * 256 * 256 * 256 * 4
    assert n >= 2 * (4 * N * D + N * (D + F)) + split
    assert n < 2 * (4 * N * D + N * (D + F)) + split + 6 * 256
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
    assert ctypes.sizeof(ops.StackDesc) == 60
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


@pytest.mark.parametrize("field,value,want", [
    ("n_img", 0, SHAPE), ("n_txt", 0, SHAPE), ("n_img_blocks", -1, SHAPE),
    ("n_joint_blocks", 2000, SHAPE), ("width", 3000, SHAPE), ("head_dim", 64, SHAPE),
    ("cfg_scale", float("nan"), ARG), ("qk_eps", -1.0, ARG), ("n_ref", -1, SHAPE),
    ("n_ref_blocks", 1, SHAPE),  # reference blocks without reference tokens
    ("n_ref", 131072, SHAPE)])  # the joint sequence above DIT_MAX_TOKENS
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
