"""ctypes binding of libdit.so (argument marshalling only).

Every function takes torch tensors that already live on the GPU, checks
their dtype, shape and contiguity, and passes raw device pointers and sizes
to the C ABI declared in include/dit.h.  All computation happens in the HIP
kernels; if the library is missing the binding raises, there is no fallback.
PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

from . import configs

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdit.so")

DIT_F_NO_RESIDUAL = 1
DIT_F_NO_GATE = 2
N_STAGES = 5
STAGES = ("adaln", "gemm_in", "rope", "attn", "gemm_out")
EXPORTS = ("dit_block_workspace_bytes", "dit_block_fwd", "dit_block_fwd_events", "dit_attn_fwd",
           "rope4_apply", "adaln_mod", "dit_stack_workspace_bytes", "dit_stack_fwd",
           "dit_flow_sigmas", "dit_sampler_workspace_bytes", "dit_sampler_prepare",
           "dit_sampler_step", "dit_linear", "dit_time_sinusoid", "dit_quantize_rows_fp8",
           "dit_block_fp8_workspace_bytes", "dit_block_fwd_fp8", "dit_block_fwd_fp8_events",
           "dit_block_fwd_noalloc", "dit_block_noalloc_scratch_bytes", "dit_attn_workspace_bytes",
           "dit_attn_fwd_ws", "dit_status_str")
NOALLOC_MAX_TOKENS = 4352
N_GROUPS = 4        # block groups with their own modulation: stage-1 image, reference, text; joint
TIME_DIM = 256


class BlockDesc(ctypes.Structure):
    _fields_ = [
        ("n_streams", ctypes.c_int32),
        ("n_tokens", ctypes.c_int32 * 3),
        ("width", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("mlp_hidden", ctypes.c_int32),
        ("rope_theta", ctypes.c_float),
        ("ln_eps", ctypes.c_float),
        ("qk_eps", ctypes.c_float),
        ("flags", ctypes.c_uint32),
    ]


class StackDesc(ctypes.Structure):
    _fields_ = [
        ("n_img", ctypes.c_int32),
        ("n_ref", ctypes.c_int32),
        ("n_txt", ctypes.c_int32),
        ("n_img_blocks", ctypes.c_int32),
        ("n_ref_blocks", ctypes.c_int32),
        ("n_txt_blocks", ctypes.c_int32),
        ("n_joint_blocks", ctypes.c_int32),
        ("width", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("mlp_hidden", ctypes.c_int32),
        ("rope_theta", ctypes.c_float),
        ("ln_eps", ctypes.c_float),
        ("qk_eps", ctypes.c_float),
        ("cfg_scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
    ]


DIT_STACK_TEXT_SIDE_STREAM = 1


class BlockParams(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in ("mod", "w_in", "w_out", "q_scale", "k_scale")]


class ModelDesc(ctypes.Structure):
    _fields_ = [("stack", StackDesc), ("latent_ch", ctypes.c_int32), ("text_dim", ctypes.c_int32)]


BLOCK_WEIGHTS = ("w_in", "w_out", "q_scale", "k_scale")


class BlockWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in BLOCK_WEIGHTS]


MODEL_TENSORS = ("img_in_w", "img_in_b", "ref_in_w", "ref_in_b", "txt_in_w", "txt_in_b",
                 "t_w1", "t_b1", "t_w2", "t_b2")


class ModelWeights(ctypes.Structure):
    _fields_ = ([(name, ctypes.c_void_p) for name in MODEL_TENSORS]
                + [("mod_w", ctypes.c_void_p * N_GROUPS), ("mod_b", ctypes.c_void_p * N_GROUPS)]
                + [(name, ctypes.c_void_p) for name in ("out_mod_w", "out_mod_b", "out_w", "out_b")]
                + [("blocks", ctypes.POINTER(BlockWeights))])


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libdit.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    desc_p = ctypes.POINTER(BlockDesc)
    lib.dit_block_workspace_bytes.argtypes = [desc_p, ctypes.POINTER(sz)]
    lib.dit_block_fwd.argtypes = [desc_p] + [vp] * 8 + [vp, sz, vp]
    lib.dit_block_fwd_events.argtypes = [desc_p] + [vp] * 8 + [vp, sz, vp, ctypes.POINTER(vp)]
    lib.dit_attn_fwd.argtypes = [i32, i32, i32, vp, vp, vp, vp, f32, vp]
    lib.rope4_apply.argtypes = [i32, i32, i32, vp, vp, vp, f32, vp, vp, f32, vp]
    lib.adaln_mod.argtypes = [i32, ctypes.POINTER(i32), i32, vp, vp, vp, f32, vp]
    stack_p = ctypes.POINTER(StackDesc)
    lib.dit_stack_workspace_bytes.argtypes = [stack_p, ctypes.POINTER(sz)]
    lib.dit_stack_fwd.argtypes = [stack_p, vp, vp, vp, vp, vp, ctypes.POINTER(BlockParams), vp, vp,
                                  sz, vp]
    model_p, weights_p = ctypes.POINTER(ModelDesc), ctypes.POINTER(ModelWeights)
    f64 = ctypes.c_double
    lib.dit_flow_sigmas.argtypes = [i32, f64, ctypes.POINTER(f64)]
    lib.dit_sampler_workspace_bytes.argtypes = [model_p, ctypes.POINTER(sz)]
    lib.dit_sampler_prepare.argtypes = [model_p, weights_p, vp, vp, vp, vp, vp, sz, vp]
    lib.dit_sampler_step.argtypes = [model_p, weights_p, vp, f64, f64, vp, vp, vp, sz, vp]
    lib.dit_linear.argtypes = [i32, i32, i32, vp, vp, vp, i32, vp, vp]
    lib.dit_time_sinusoid.argtypes = [i32, ctypes.POINTER(f64), vp, vp]
    lib.dit_quantize_rows_fp8.argtypes = [i32, i32, vp, vp, vp, vp]
    lib.dit_block_fp8_workspace_bytes.argtypes = [desc_p, ctypes.POINTER(sz)]
    lib.dit_block_fwd_fp8.argtypes = [desc_p] + [vp] * 10 + [vp, sz, vp]
    lib.dit_block_fwd_fp8_events.argtypes = [desc_p] + [vp] * 10 + [vp, sz, vp,
                                                                   ctypes.POINTER(vp)]
    lib.dit_block_fwd_noalloc.argtypes = [desc_p] + [vp] * 8 + [vp]
    lib.dit_block_noalloc_scratch_bytes.argtypes = [ctypes.POINTER(sz)]
    lib.dit_attn_workspace_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
    lib.dit_attn_fwd_ws.argtypes = [i32, i32, i32, vp, vp, vp, vp, f32, vp, sz, vp]
    lib.dit_status_str.argtypes = [ctypes.c_int]
    lib.dit_status_str.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name != "dit_status_str":
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


class DitError(RuntimeError):
    def __init__(self, rc: int):
        self.rc = rc
        super().__init__(load_library().dit_status_str(rc).decode())


def _check(rc: int) -> None:
    if rc != 0:
        raise DitError(rc)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _bf16(t: torch.Tensor, shape, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_desc(n_tokens: Sequence[int], width: int = configs.WIDTH, n_heads: int = configs.N_HEADS,
              head_dim: int = configs.HEAD_DIM, mlp_hidden: int = configs.MLP_HIDDEN,
              rope_theta: float = configs.ROPE_THETA, ln_eps: float = configs.LN_EPS,
              qk_eps: float = configs.QK_EPS, flags: int = 0) -> BlockDesc:
    d = BlockDesc()
    d.n_streams = len(n_tokens)
    for i, n in enumerate(n_tokens):
        d.n_tokens[i] = int(n)
    d.width, d.n_heads, d.head_dim, d.mlp_hidden = width, n_heads, head_dim, mlp_hidden
    d.rope_theta, d.ln_eps, d.qk_eps, d.flags = rope_theta, ln_eps, qk_eps, flags
    return d


def workspace_bytes(desc: BlockDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().dit_block_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def alloc_workspace(desc: BlockDesc, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_bytes(desc), 1), dtype=torch.uint8, device=device)


def block_fwd(x, mod, pos, w_in, w_out, q_scale, k_scale, desc: BlockDesc, y=None,
              workspace=None, stream=None, events=None) -> torch.Tensor:
    """y = dit_block_fwd(...).  events: optional list of DIT_N_STAGES + 1 raw hipEvent_t."""
    N = sum(desc.n_tokens[i] for i in range(desc.n_streams))
    D, F, d = desc.width, desc.mlp_hidden, desc.head_dim
    _bf16(x, (N, D), "x")
    _bf16(mod, (desc.n_streams, 3, D), "mod")
    if pos.dtype != torch.int32 or tuple(pos.shape) != (N, 4) or not pos.is_cuda \
            or not pos.is_contiguous():
        raise ValueError("pos must be a contiguous int32 [N, 4] GPU tensor")
    _bf16(w_in, (3 * D + 2 * F, D), "w_in")
    _bf16(w_out, (D, D + F), "w_out")
    _bf16(q_scale, (d,), "q_scale")
    _bf16(k_scale, (d,), "k_scale")
    if y is None:
        y = torch.empty_like(x)
    _bf16(y, (N, D), "y")
    if workspace is None:
        workspace = alloc_workspace(desc, x.device)
    lib = load_library()
    args = [ctypes.byref(desc), _ptr(x), _ptr(mod), _ptr(pos), _ptr(w_in), _ptr(w_out),
            _ptr(q_scale), _ptr(k_scale), _ptr(y), _ptr(workspace),
            ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(stream)]
    if events is None:
        _check(lib.dit_block_fwd(*args))
    else:
        arr = (ctypes.c_void_p * (N_STAGES + 1))(*events)
        _check(lib.dit_block_fwd_events(*args, arr))
    return y


def noalloc_scratch_bytes() -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().dit_block_noalloc_scratch_bytes(ctypes.byref(n)))
    return n.value


def block_fwd_noalloc(x, mod, pos, w_in, w_out, q_scale, k_scale, desc: BlockDesc, y=None,
                      stream=None) -> torch.Tensor:
    """y = dit_block_fwd_noalloc(...): the block with the library's own per-GPU
    scratch instead of a workspace argument (y is allocated here when not given)."""
    N = sum(desc.n_tokens[i] for i in range(desc.n_streams))
    D, F, d = desc.width, desc.mlp_hidden, desc.head_dim
    _bf16(x, (N, D), "x")
    _bf16(mod, (desc.n_streams, 3, D), "mod")
    if pos.dtype != torch.int32 or tuple(pos.shape) != (N, 4) or not pos.is_cuda \
            or not pos.is_contiguous():
        raise ValueError("pos must be a contiguous int32 [N, 4] GPU tensor")
    _bf16(w_in, (3 * D + 2 * F, D), "w_in")
    _bf16(w_out, (D, D + F), "w_out")
    _bf16(q_scale, (d,), "q_scale")
    _bf16(k_scale, (d,), "k_scale")
    if y is None:
        y = torch.empty_like(x)
    _bf16(y, (N, D), "y")
    _check(load_library().dit_block_fwd_noalloc(
        ctypes.byref(desc), _ptr(x), _ptr(mod), _ptr(pos), _ptr(w_in), _ptr(w_out),
        _ptr(q_scale), _ptr(k_scale), _ptr(y), _stream(stream)))
    return y


def attn_fwd(q, k, v, o=None, softmax_scale: Optional[float] = None, stream=None):
    """o = dit_attn_fwd(q, k, v); q, k, v, o bf16 [N, H, d]."""
    N, H, d = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _bf16(t, (N, H, d), n)
    if o is None:
        o = torch.empty_like(q)
    _bf16(o, (N, H, d), "o")
    scale = d ** -0.5 if softmax_scale is None else softmax_scale
    _check(load_library().dit_attn_fwd(N, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                       ctypes.c_float(scale), _stream(stream)))
    return o


def attn_workspace_bytes(n_tokens: int, n_heads: int, head_dim: int = configs.HEAD_DIM) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().dit_attn_workspace_bytes(n_tokens, n_heads, head_dim, ctypes.byref(n)))
    return n.value


def attn_fwd_ws(q, k, v, o=None, softmax_scale: Optional[float] = None, workspace=None,
                stream=None):
    """o = dit_attn_fwd_ws(q, k, v): attention with the work split over the CUs
    (the block's schedule); q, k, v, o bf16 [N, H, d]."""
    N, H, d = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _bf16(t, (N, H, d), n)
    if o is None:
        o = torch.empty_like(q)
    _bf16(o, (N, H, d), "o")
    if workspace is None:
        workspace = torch.empty(attn_workspace_bytes(N, H, d), dtype=torch.uint8, device=q.device)
    scale = d ** -0.5 if softmax_scale is None else softmax_scale
    _check(load_library().dit_attn_fwd_ws(
        N, H, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), ctypes.c_float(scale), _ptr(workspace),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(stream)))
    return o


def rope4_apply(q, k, pos, theta: float = configs.ROPE_THETA, q_scale=None, k_scale=None,
                qk_eps: float = configs.QK_EPS, stream=None):
    """In place: optional QK RMSNorm, then 4-axis RoPE on q and k ([N, H, d] bf16)."""
    N, H, d = q.shape
    _bf16(q, (N, H, d), "q")
    _bf16(k, (N, H, d), "k")
    if pos.dtype != torch.int32 or tuple(pos.shape) != (N, 4) or not pos.is_cuda \
            or not pos.is_contiguous():
        raise ValueError("pos must be a contiguous int32 [N, 4] GPU tensor")
    if q_scale is not None:
        _bf16(q_scale, (d,), "q_scale")
    if k_scale is not None:
        _bf16(k_scale, (d,), "k_scale")
    _check(load_library().rope4_apply(N, H, d, _ptr(q), _ptr(k), _ptr(pos), ctypes.c_float(theta),
                                      _ptr(q_scale), _ptr(k_scale), ctypes.c_float(qk_eps),
                                      _stream(stream)))
    return q, k


def adaln_mod(x, mod, n_tokens: Sequence[int], out=None, eps: float = configs.LN_EPS,
              stream=None):
    """out = LN(x) * (1 + scale_s) + shift_s per stream; x [N, W] bf16, mod [S, 3, W]."""
    N, W = x.shape
    _bf16(x, (N, W), "x")
    _bf16(mod, (len(n_tokens), 3, W), "mod")
    if out is None:
        out = torch.empty_like(x)
    _bf16(out, (N, W), "out")
    counts = (ctypes.c_int32 * len(n_tokens))(*[int(n) for n in n_tokens])
    _check(load_library().adaln_mod(len(n_tokens), counts, W, _ptr(x), _ptr(mod), _ptr(out),
                                    ctypes.c_float(eps), _stream(stream)))
    return out


def to_device_bf16(bits, device="cuda") -> torch.Tensor:
    """uint16 bf16 bit patterns (numpy) -> bfloat16 GPU tensor, bytes unchanged."""
    import numpy as np
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def to_host_bits(t: torch.Tensor):
    """bfloat16 GPU tensor -> uint16 numpy bit patterns."""
    import numpy as np
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def make_stack_desc(n_img: int, n_txt: int, n_img_blocks: int, n_txt_blocks: int,
                    n_joint_blocks: int, cfg_scale: float, n_ref: int = 0, n_ref_blocks: int = 0,
                    width: int = configs.WIDTH, n_heads: int = configs.N_HEADS,
                    head_dim: int = configs.HEAD_DIM,
                    mlp_hidden: int = configs.MLP_HIDDEN, side_stream: bool = False) -> StackDesc:
    """side_stream: run the stage-1 text blocks on the library's second stream
    (DIT_STACK_TEXT_SIDE_STREAM)."""
    d = StackDesc()
    d.n_img, d.n_ref, d.n_txt = n_img, n_ref, n_txt
    d.n_img_blocks, d.n_ref_blocks = n_img_blocks, n_ref_blocks
    d.n_txt_blocks, d.n_joint_blocks = n_txt_blocks, n_joint_blocks
    d.width, d.n_heads, d.head_dim, d.mlp_hidden = width, n_heads, head_dim, mlp_hidden
    d.rope_theta, d.ln_eps, d.qk_eps = configs.ROPE_THETA, configs.LN_EPS, configs.QK_EPS
    d.cfg_scale = cfg_scale
    d.flags = DIT_STACK_TEXT_SIDE_STREAM if side_stream else 0
    return d


def stack_workspace_bytes(desc: StackDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().dit_stack_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def stack_fwd(desc: StackDesc, x_img, x_txt_cond, x_txt_neg, pos, blocks, v_img=None,
              workspace=None, stream=None, x_ref=None) -> torch.Tensor:
    """v_img = dit_stack_fwd(...).  blocks: sequence of dicts with keys mod,
    w_in, w_out, q_scale, k_scale (image blocks, then reference, text and
    joint blocks); x_ref is required when desc.n_ref > 0."""
    D, F, d = desc.width, desc.mlp_hidden, desc.head_dim
    N = desc.n_img + desc.n_ref + desc.n_txt
    _bf16(x_img, (desc.n_img, D), "x_img")
    if desc.n_ref > 0:
        if x_ref is None:
            raise ValueError("x_ref is required when n_ref > 0")
        _bf16(x_ref, (desc.n_ref, D), "x_ref")
    _bf16(x_txt_cond, (desc.n_txt, D), "x_txt_cond")
    if x_txt_neg is not None:
        _bf16(x_txt_neg, (desc.n_txt, D), "x_txt_neg")
    if pos.dtype != torch.int32 or tuple(pos.shape) != (N, 4) or not pos.is_cuda \
            or not pos.is_contiguous():
        raise ValueError("pos must be a contiguous int32 [n_img + n_ref + n_txt, 4] GPU tensor")
    n_stage1 = desc.n_img_blocks + desc.n_ref_blocks + desc.n_txt_blocks
    n_blocks = n_stage1 + desc.n_joint_blocks
    if len(blocks) != n_blocks:
        raise ValueError(f"expected {n_blocks} blocks, got {len(blocks)}")
    s_joint = 3 if desc.n_ref > 0 else 2
    arr = (BlockParams * max(n_blocks, 1))()
    for i, b in enumerate(blocks):
        s = 1 if i < n_stage1 else s_joint
        _bf16(b["mod"], (s, 3, D), f"blocks[{i}].mod")
        _bf16(b["w_in"], (3 * D + 2 * F, D), f"blocks[{i}].w_in")
        _bf16(b["w_out"], (D, D + F), f"blocks[{i}].w_out")
        _bf16(b["q_scale"], (d,), f"blocks[{i}].q_scale")
        _bf16(b["k_scale"], (d,), f"blocks[{i}].k_scale")
        for name in ("mod", "w_in", "w_out", "q_scale", "k_scale"):
            setattr(arr[i], name, b[name].data_ptr())
    if v_img is None:
        v_img = torch.empty((desc.n_img, D), dtype=torch.bfloat16, device=x_img.device)
    _bf16(v_img, (desc.n_img, D), "v_img")
    if workspace is None:
        workspace = torch.empty(stack_workspace_bytes(desc), dtype=torch.uint8,
                                device=x_img.device)
    _check(load_library().dit_stack_fwd(
        ctypes.byref(desc), _ptr(x_img), _ptr(x_ref), _ptr(x_txt_cond), _ptr(x_txt_neg),
        ctypes.c_void_p(pos.data_ptr()), arr, _ptr(v_img), _ptr(workspace),
        ctypes.c_size_t(workspace.numel()), _stream(stream)))
    return v_img


# ---- flow-matching sampler ------------------------------------------------------

def flow_sigmas(n_steps: int, alpha: float = 6.93):
    """The n_steps + 1 sigmas of the shifted schedule (dit_flow_sigmas), as a list."""
    out = (ctypes.c_double * (n_steps + 1))()
    _check(load_library().dit_flow_sigmas(n_steps, ctypes.c_double(alpha), out))
    return list(out)


def make_model_desc(stack: StackDesc, latent_ch: int = 128, text_dim: int = 20480) -> ModelDesc:
    d = ModelDesc()
    d.stack = stack
    d.latent_ch, d.text_dim = latent_ch, text_dim
    return d


def sampler_workspace_bytes(desc: ModelDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().dit_sampler_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


class Model:
    """Device weights of the model around the blocks, marshalled once into the
    C structs.  tensors: dict with the MODEL_TENSORS names plus out_mod_w,
    out_mod_b, out_w, out_b and lists mod_w, mod_b (N_GROUPS each);
    blocks: list of dicts with the BLOCK_WEIGHTS names (groups in order
    image, reference, text, joint).  ref_in_* and the reference group's
    modulation may be None without references."""

    def __init__(self, desc: ModelDesc, tensors, blocks):
        st = desc.stack
        D, F, d, C, T = st.width, st.mlp_hidden, st.head_dim, desc.latent_ch, desc.text_dim
        refs = st.n_ref > 0
        shapes = {"img_in_w": (D, C), "img_in_b": (D,), "ref_in_w": (D, C), "ref_in_b": (D,),
                  "txt_in_w": (D, T), "txt_in_b": (D,), "t_w1": (D, TIME_DIM), "t_b1": (D,),
                  "t_w2": (D, D), "t_b2": (D,), "out_mod_w": (2 * D, D), "out_mod_b": (2 * D,),
                  "out_w": (C, D), "out_b": (C,)}
        w = ModelWeights()
        for name, shape in shapes.items():
            t = tensors.get(name)
            if t is None and name.startswith("ref_in") and not refs:
                continue
            _bf16(t, shape, name)
            setattr(w, name, t.data_ptr())
        for g in range(N_GROUPS):
            if tensors["mod_w"][g] is None and g == 1 and not refs:
                continue
            _bf16(tensors["mod_w"][g], (3 * D, D), f"mod_w[{g}]")
            _bf16(tensors["mod_b"][g], (3 * D,), f"mod_b[{g}]")
            w.mod_w[g] = tensors["mod_w"][g].data_ptr()
            w.mod_b[g] = tensors["mod_b"][g].data_ptr()
        n_blocks = st.n_img_blocks + st.n_ref_blocks + st.n_txt_blocks + st.n_joint_blocks
        if len(blocks) != n_blocks:
            raise ValueError(f"expected {n_blocks} blocks, got {len(blocks)}")
        self._blocks = (BlockWeights * max(n_blocks, 1))()
        for i, b in enumerate(blocks):
            _bf16(b["w_in"], (3 * D + 2 * F, D), f"blocks[{i}].w_in")
            _bf16(b["w_out"], (D, D + F), f"blocks[{i}].w_out")
            _bf16(b["q_scale"], (d,), f"blocks[{i}].q_scale")
            _bf16(b["k_scale"], (d,), f"blocks[{i}].k_scale")
            for name in BLOCK_WEIGHTS:
                setattr(self._blocks[i], name, b[name].data_ptr())
        w.blocks = self._blocks
        self.weights = w
        self.desc = desc
        self._keep = (tensors, blocks)  # the device memory the pointers refer to


def _pos_check(pos, n):
    if pos.dtype != torch.int32 or tuple(pos.shape) != (n, 4) or not pos.is_cuda \
            or not pos.is_contiguous():
        raise ValueError(f"pos must be a contiguous int32 [{n}, 4] GPU tensor")


def alloc_sampler_workspace(desc: ModelDesc, device="cuda") -> torch.Tensor:
    return torch.empty(sampler_workspace_bytes(desc), dtype=torch.uint8, device=device)


def sampler_prepare(model: Model, txt_cond, txt_neg, ref_latent, pos, workspace, stream=None):
    st, desc = model.desc.stack, model.desc
    _bf16(txt_cond, (st.n_txt, desc.text_dim), "txt_cond")
    if txt_neg is not None:
        _bf16(txt_neg, (st.n_txt, desc.text_dim), "txt_neg")
    if ref_latent is not None:
        _bf16(ref_latent, (st.n_ref, desc.latent_ch), "ref_latent")
    _pos_check(pos, st.n_img + st.n_ref + st.n_txt)
    _check(load_library().dit_sampler_prepare(
        ctypes.byref(desc), ctypes.byref(model.weights), _ptr(txt_cond), _ptr(txt_neg),
        _ptr(ref_latent), ctypes.c_void_p(pos.data_ptr()), _ptr(workspace),
        ctypes.c_size_t(workspace.numel()), _stream(stream)))


def sampler_step(model: Model, z, sigma: float, sigma_next: float, pos, workspace, v_out=None,
                 stream=None):
    """In place: z <- z + (sigma_next - sigma) * guided velocity (dit_sampler_step)."""
    st, desc = model.desc.stack, model.desc
    _bf16(z, (st.n_img, desc.latent_ch), "z")
    if v_out is not None:
        _bf16(v_out, (st.n_img, desc.latent_ch), "v_out")
    _pos_check(pos, st.n_img + st.n_ref + st.n_txt)
    _check(load_library().dit_sampler_step(
        ctypes.byref(desc), ctypes.byref(model.weights), _ptr(z), ctypes.c_double(sigma),
        ctypes.c_double(sigma_next), ctypes.c_void_p(pos.data_ptr()), _ptr(v_out),
        _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(stream)))
    return z


def linear(x, w, b=None, act: int = 0, y=None, stream=None) -> torch.Tensor:
    """y = act(x w^T + b) (dit_linear); x [M, K], w [N, K], b [N]."""
    M, K = x.shape
    N = w.shape[0]
    _bf16(x, (M, K), "x")
    _bf16(w, (N, K), "w")
    if b is not None:
        _bf16(b, (N,), "b")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _bf16(y, (M, N), "y")
    _check(load_library().dit_linear(M, N, K, _ptr(x), _ptr(w), _ptr(b), act, _ptr(y),
                                     _stream(stream)))
    return y


def time_sinusoid(ts, out=None, stream=None) -> torch.Tensor:
    """out [len(ts), 256]: the timestep sinusoids (dit_time_sinusoid)."""
    n = len(ts)
    arr = (ctypes.c_double * max(n, 1))(*ts)
    if out is None:
        out = torch.empty((n, TIME_DIM), dtype=torch.bfloat16, device="cuda")
    _check(load_library().dit_time_sinusoid(n, arr, _ptr(out), _stream(stream)))
    return out


# ---- FP8 projections ---------------------------------------------------------------

def quantize_rows_fp8(x, q=None, scale=None, stream=None):
    """(codes uint8 [M, K], scales float32 [M]) of bf16 x [M, K] (dit_quantize_rows_fp8)."""
    M, K = x.shape
    _bf16(x, (M, K), "x")
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    if q.dtype != torch.uint8 or tuple(q.shape) != (M, K) or not q.is_contiguous():
        raise ValueError("q must be a contiguous uint8 [M, K] tensor")
    if scale.dtype != torch.float32 or tuple(scale.shape) != (M,):
        raise ValueError("scale must be a float32 [M] tensor")
    _check(load_library().dit_quantize_rows_fp8(M, K, _ptr(x), _ptr(q), _ptr(scale),
                                                _stream(stream)))
    return q, scale


def block_fp8_workspace_bytes(desc: BlockDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().dit_block_fp8_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def alloc_fp8_workspace(desc: BlockDesc, device="cuda") -> torch.Tensor:
    return torch.empty(max(block_fp8_workspace_bytes(desc), 1), dtype=torch.uint8, device=device)


def _fp8_weight(q, s, shape, name):
    if q.dtype != torch.uint8 or tuple(q.shape) != tuple(shape) or not q.is_cuda \
            or not q.is_contiguous():
        raise ValueError(f"{name} must be a contiguous uint8 {tuple(shape)} GPU tensor")
    if s.dtype != torch.float32 or tuple(s.shape) != (shape[0],) or not s.is_contiguous():
        raise ValueError(f"{name} scales must be a contiguous float32 [{shape[0]}] tensor")


def block_fwd_fp8(x, mod, pos, w_in8, w_in_scale, w_out8, w_out_scale, q_scale, k_scale,
                  desc: BlockDesc, y=None, workspace=None, stream=None, events=None):
    """y = dit_block_fwd_fp8(...): the block with FP8 projections; the weights
    as returned by quantize_rows_fp8."""
    N = sum(desc.n_tokens[i] for i in range(desc.n_streams))
    D, F, d = desc.width, desc.mlp_hidden, desc.head_dim
    _bf16(x, (N, D), "x")
    _bf16(mod, (desc.n_streams, 3, D), "mod")
    _pos_check(pos, N)
    _fp8_weight(w_in8, w_in_scale, (3 * D + 2 * F, D), "w_in8")
    _fp8_weight(w_out8, w_out_scale, (D, D + F), "w_out8")
    _bf16(q_scale, (d,), "q_scale")
    _bf16(k_scale, (d,), "k_scale")
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_fp8_workspace(desc, x.device)
    args = [ctypes.byref(desc), _ptr(x), _ptr(mod), ctypes.c_void_p(pos.data_ptr()),
            _ptr(w_in8), _ptr(w_in_scale), _ptr(w_out8), _ptr(w_out_scale), _ptr(q_scale),
            _ptr(k_scale), _ptr(y), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
            _stream(stream)]
    lib = load_library()
    if events is None:
        _check(lib.dit_block_fwd_fp8(*args))
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        _check(lib.dit_block_fwd_fp8_events(*args, arr))
    return y
