"""ctypes binding of liblwm_attn.so with the C ABI's names (argument marshalling only).

Each function takes torch tensors already on the GPU in the ``[B, L, H, D]`` layout (feature
stride 1), passes their pointers, sizes and strides to the C entry point of the same name and
enqueues the work on ``torch.cuda.current_stream()``.  Outputs that are not passed in are
allocated with ``torch.empty``.  Nothing here computes any part of the method: if the library
is missing or a call fails, a ``LwmError`` is raised; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LWM_ATTN_LIB", os.path.join(_HERE, "liblwm_attn.so"))

LWM_BF16, LWM_FP32 = 0, 1
LAYOUTS = {"half": 0, "interleaved": 1}
STATUS = {0: "LWM_OK", -1: "LWM_ERR_INVALID_ARG", -2: "LWM_ERR_UNSUPPORTED", -3: "LWM_ERR_WORKSPACE", -4: "LWM_ERR_HIP"}


class LwmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Tensor4(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("B", ctypes.c_int64), ("L", ctypes.c_int64), ("H", ctypes.c_int64), ("D", ctypes.c_int64),
                ("sB", ctypes.c_int64), ("sL", ctypes.c_int64), ("sH", ctypes.c_int64)]


class RopeArgs(ctypes.Structure):
    _fields_ = [("theta", ctypes.c_double), ("layout", ctypes.c_int32), ("restart", ctypes.c_int32),
                ("q_pos_offset", ctypes.c_int64), ("k_pos_offset", ctypes.c_int64)]


_lib = None
EXPORTS = ["lwm_abi_version", "lwm_last_error", "lwm_rope_apply", "lwm_blockattn_fwd",
           "lwm_blockattn_bwd_workspace_size", "lwm_blockattn_bwd", "lwm_blockattn_fwd_rope",
           "lwm_blockattn_bwd_rope", "lwm_ring_step", "lwm_ring_step_bwd",
           "lwm_blockwise_ffn_workspace_size", "lwm_blockwise_ffn", "lwm_profile_enable", "lwm_profile_reset", "lwm_profile_count", "lwm_profile_get"]


def lib() -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m ring_causal_attention_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, F64, VP = (ctypes.POINTER(Tensor4), ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_double, ctypes.c_void_p)
    L.lwm_abi_version.restype = ctypes.c_int
    L.lwm_abi_version.argtypes = []
    L.lwm_last_error.restype = ctypes.c_char_p
    L.lwm_last_error.argtypes = []
    L.lwm_rope_apply.restype = ctypes.c_int
    L.lwm_rope_apply.argtypes = [P, P, VP, VP, I64, F64, I32, I32, VP]
    L.lwm_blockattn_fwd.restype = ctypes.c_int
    L.lwm_blockattn_fwd.argtypes = [P, P, P, VP, VP, I64, I64, I32, F32, P, VP, VP]
    L.lwm_blockattn_bwd_workspace_size.restype = ctypes.c_size_t
    L.lwm_blockattn_bwd_workspace_size.argtypes = [I64, I64, I64, I64, I64]
    L.lwm_blockattn_bwd.restype = ctypes.c_int
    L.lwm_blockattn_bwd.argtypes = [P, P, P, P, VP, P, VP, VP, I64, I64, I32, F32, P, P, P, VP, ctypes.c_size_t, VP]
    R = ctypes.POINTER(RopeArgs)
    L.lwm_blockattn_fwd_rope.restype = ctypes.c_int
    L.lwm_blockattn_fwd_rope.argtypes = [P, P, P, VP, VP, I64, I64, I32, F32, R, P, VP, P, P, VP]
    L.lwm_blockattn_bwd_rope.restype = ctypes.c_int
    L.lwm_blockattn_bwd_rope.argtypes = [P, P, P, P, VP, P, VP, VP, I64, I64, I32, F32, R, P, P, P, VP,
                                         ctypes.c_size_t, VP]
    L.lwm_ring_step.restype = ctypes.c_int
    L.lwm_ring_step.argtypes = [P, P, P, VP, VP, I64, I64, I32, F32, P, VP, P, VP]
    L.lwm_ring_step_bwd.restype = ctypes.c_int
    L.lwm_ring_step_bwd.argtypes = [P, P, P, P, VP, P, VP, VP, I64, I64, I32, F32, P, P, P, VP, ctypes.c_size_t, VP]
    L.lwm_blockwise_ffn_workspace_size.restype = ctypes.c_size_t
    L.lwm_blockwise_ffn_workspace_size.argtypes = [I64, I64, I64]
    L.lwm_blockwise_ffn.restype = ctypes.c_int
    L.lwm_blockwise_ffn.argtypes = [VP, I64, I64, I64, VP, VP, I64, VP, I64, I64, VP, I64, I64, VP, ctypes.c_size_t, VP]
    L.lwm_profile_enable.restype = ctypes.c_int
    L.lwm_profile_enable.argtypes = [I32]
    L.lwm_profile_reset.restype = ctypes.c_int
    L.lwm_profile_reset.argtypes = []
    L.lwm_profile_count.restype = ctypes.c_int
    L.lwm_profile_count.argtypes = []
    L.lwm_profile_get.restype = ctypes.c_int
    L.lwm_profile_get.argtypes = [I32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(F64), ctypes.POINTER(I64)]
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise LwmError(status, lib().lwm_last_error().decode(errors="replace"))


def tensor4(t: torch.Tensor | None) -> Tensor4 | None:
    """Describe a [B, L, H, D] tensor (feature stride 1) for the ABI."""
    if t is None:
        return None
    if t.dim() != 4:
        raise ValueError(f"expected a [B, L, H, D] tensor, got shape {tuple(t.shape)}")
    if t.dtype == torch.bfloat16:
        dt = LWM_BF16
    elif t.dtype == torch.float32:
        dt = LWM_FP32
    else:
        raise ValueError(f"unsupported dtype {t.dtype}")
    B, L, H, D = t.shape
    if t.numel() == 0:  # no element is addressed: describe it with contiguous strides
        return Tensor4(t.data_ptr(), dt, 0, B, L, H, D, L * H * D, H * D, D)
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError("the feature dimension must be contiguous")
    return Tensor4(t.data_ptr(), dt, 0, B, L, H, D, t.stride(0), t.stride(1), t.stride(2))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ref(s):
    return None if s is None else ctypes.byref(s)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _seg(s):
    if s is None:
        return None
    if s.dtype != torch.int32 or not s.is_contiguous():
        raise ValueError("segment ids / positions must be contiguous int32 [B, L]")
    return s


def lwm_abi_version() -> int:
    return lib().lwm_abi_version()


def lwm_rope_apply(x, y=None, pos=None, seg=None, pos_offset=0, theta=10000.0, layout="half", inverse=False):
    """RoPE of x into y (default: a new tensor; pass y=x for in place).  Returns y."""
    y = torch.empty_like(x) if y is None else y
    _check(lib().lwm_rope_apply(_ref(tensor4(x)), _ref(tensor4(y)), _ptr(_seg(pos)), _ptr(_seg(seg)), int(pos_offset),
                                float(theta), LAYOUTS[layout], int(bool(inverse)), _stream(x)))
    return y


def lwm_blockattn_fwd(q, k, v, seg_q=None, seg_k=None, q_offset=0, k_offset=0, causal=True, scale=0.0,
                      o=None, lse=None, want_lse=True):
    """Forward; returns (o, lse) with lse float32 [B, H, Lq] (None if want_lse is False)."""
    B, Lq, H, _ = q.shape
    o = torch.empty_like(q) if o is None else o
    if lse is None and want_lse:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    _check(lib().lwm_blockattn_fwd(_ref(tensor4(q)), _ref(tensor4(k)), _ref(tensor4(v)), _ptr(_seg(seg_q)),
                                   _ptr(_seg(seg_k)), int(q_offset), int(k_offset), int(bool(causal)), float(scale),
                                   _ref(tensor4(o)), _ptr(lse), _stream(q)))
    return o, lse


def lwm_blockattn_bwd_workspace_size(B, H, Lq, Lk, D) -> int:
    return int(lib().lwm_blockattn_bwd_workspace_size(B, H, Lq, Lk, D))


def lwm_blockattn_bwd(q, k, v, o, lse, dout, seg_q=None, seg_k=None, q_offset=0, k_offset=0, causal=True,
                      scale=0.0, dq=None, dk=None, dv=None, workspace=None):
    """Backward; returns (dq, dk, dv) w.r.t. the operands given (the rotated Q', K')."""
    B, Lq, H, D = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = lwm_blockattn_bwd_workspace_size(B, H, Lq, k.shape[1], D)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib().lwm_blockattn_bwd(_ref(tensor4(q)), _ref(tensor4(k)), _ref(tensor4(v)), _ref(tensor4(o)), _ptr(lse),
                                   _ref(tensor4(dout)), _ptr(_seg(seg_q)), _ptr(_seg(seg_k)), int(q_offset),
                                   int(k_offset), int(bool(causal)), float(scale), _ref(tensor4(dq)),
                                   _ref(tensor4(dk)), _ref(tensor4(dv)), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(q)))
    return dq, dk, dv


def rope_args(theta, layout="half", restart=False, q_pos_offset=0, k_pos_offset=0) -> RopeArgs:
    """The RoPE descriptor of the fused entry points (positions restart per segment if restart)."""
    return RopeArgs(float(theta), LAYOUTS[layout], int(bool(restart)), int(q_pos_offset), int(k_pos_offset))


def lwm_blockattn_fwd_rope(q, k, v, theta, seg_q=None, seg_k=None, q_offset=0, k_offset=0, causal=True, scale=0.0,
                           layout="half", restart=False, q_pos_offset=0, k_pos_offset=0, o=None, lse=None,
                           q_rot=None, k_rot=None, want_q_rot=True):
    """Forward from the pre-RoPE q, k (RoPE inside the call); returns (o, lse, q_rot, k_rot).
    q_rot is None when want_q_rot is False and no buffer is given."""
    B, Lq, H, _ = q.shape
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device) if lse is None else lse
    k_rot = torch.empty_like(k) if k_rot is None else k_rot
    if q_rot is None and want_q_rot:
        q_rot = torch.empty_like(q)
    ra = rope_args(theta, layout, restart, q_pos_offset, k_pos_offset)
    _check(lib().lwm_blockattn_fwd_rope(_ref(tensor4(q)), _ref(tensor4(k)), _ref(tensor4(v)), _ptr(_seg(seg_q)),
                                        _ptr(_seg(seg_k)), int(q_offset), int(k_offset), int(bool(causal)),
                                        float(scale), ctypes.byref(ra), _ref(tensor4(o)), _ptr(lse),
                                        _ref(tensor4(q_rot)), _ref(tensor4(k_rot)), _stream(q)))
    return o, lse, q_rot, k_rot


def lwm_blockattn_bwd_rope(q_rot, k_rot, v, o, lse, dout, theta, seg_q=None, seg_k=None, q_offset=0, k_offset=0,
                           causal=True, scale=0.0, layout="half", restart=False, q_pos_offset=0, k_pos_offset=0,
                           dq=None, dk=None, dv=None, workspace=None):
    """Backward with the inverse RoPE inside the call; returns (dq, dk, dv) w.r.t. the pre-RoPE Q, K."""
    B, Lq, H, D = q_rot.shape
    dq = torch.empty_like(q_rot) if dq is None else dq
    dk = torch.empty_like(k_rot) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = torch.empty(lwm_blockattn_bwd_workspace_size(B, H, Lq, k_rot.shape[1], D), dtype=torch.uint8,
                                device=q_rot.device)
    ra = rope_args(theta, layout, restart, q_pos_offset, k_pos_offset)
    _check(lib().lwm_blockattn_bwd_rope(_ref(tensor4(q_rot)), _ref(tensor4(k_rot)), _ref(tensor4(v)),
                                        _ref(tensor4(o)), _ptr(lse), _ref(tensor4(dout)), _ptr(_seg(seg_q)),
                                        _ptr(_seg(seg_k)), int(q_offset), int(k_offset), int(bool(causal)),
                                        float(scale), ctypes.byref(ra), _ref(tensor4(dq)), _ref(tensor4(dk)),
                                        _ref(tensor4(dv)), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(q_rot)))
    return dq, dk, dv


def lwm_ring_step(q, k_shard, v_shard, o_acc, lse_acc, seg_q=None, seg_k=None, q_offset=0, k_offset=0,
                  causal=True, scale=0.0, o_final=None):
    """Fold one KV shard into (o_acc float32 [B, Lq, H, D], lse_acc float32 [B, H, Lq]) in place."""
    _check(lib().lwm_ring_step(_ref(tensor4(q)), _ref(tensor4(k_shard)), _ref(tensor4(v_shard)), _ptr(_seg(seg_q)),
                               _ptr(_seg(seg_k)), int(q_offset), int(k_offset), int(bool(causal)), float(scale),
                               _ref(tensor4(o_acc)), _ptr(lse_acc), _ref(tensor4(o_final)), _stream(q)))
    return o_acc, lse_acc


def lwm_ring_step_bwd(q, k_shard, v_shard, o, lse, dout, dq_acc, dk_acc, dv_acc, seg_q=None, seg_k=None,
                      q_offset=0, k_offset=0, causal=True, scale=0.0, workspace=None):
    """Add one KV shard's share of the gradients into dq_acc (float32, like q) and dk_acc,
    dv_acc (float32, like k_shard), in place; o and lse are the forward's results over all shards."""
    B, Lq, H, D = q.shape
    need = lwm_blockattn_bwd_workspace_size(B, H, Lq, k_shard.shape[1], D)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib().lwm_ring_step_bwd(_ref(tensor4(q)), _ref(tensor4(k_shard)), _ref(tensor4(v_shard)), _ref(tensor4(o)),
                                   _ptr(lse), _ref(tensor4(dout)), _ptr(_seg(seg_q)), _ptr(_seg(seg_k)), int(q_offset),
                                   int(k_offset), int(bool(causal)), float(scale), _ref(tensor4(dq_acc)),
                                   _ref(tensor4(dk_acc)), _ref(tensor4(dv_acc)), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(q)))
    return dq_acc, dk_acc, dv_acc


def _matrix(t, name):
    if t.dtype != torch.bfloat16 or t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name}: expected a bf16 matrix with contiguous rows, got {t.dtype} {tuple(t.shape)}")
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def lwm_blockwise_ffn_workspace_size(rows, d_ff, chunk) -> int:
    return int(lib().lwm_blockwise_ffn_workspace_size(rows, d_ff, chunk))


def lwm_blockwise_ffn(x, w_gate, w_up, w_down, chunk=8192, y=None, workspace=None):
    """y = (silu(x W_gate^T) * (x W_up^T)) W_down^T over chunks of `chunk` rows; x [rows, d_model],
    w_gate / w_up [d_ff, d_model], w_down [d_model, d_ff] (nn.Linear layout).  Returns y."""
    rows, d_model = x.shape
    d_ff = w_gate.shape[0]
    if tuple(w_gate.shape) != (d_ff, d_model) or tuple(w_up.shape) != (d_ff, d_model) \
            or tuple(w_down.shape) != (d_model, d_ff):
        raise ValueError("weight shapes do not match x")
    if w_gate.stride(0) != w_up.stride(0):
        raise ValueError("w_gate and w_up must share a row stride")
    y = torch.empty((rows, d_model), dtype=x.dtype, device=x.device) if y is None else y
    if workspace is None:
        workspace = torch.empty(lwm_blockwise_ffn_workspace_size(rows, d_ff, chunk), dtype=torch.uint8,
                                device=x.device)
    _check(lib().lwm_blockwise_ffn(_ptr(x), rows, d_model, _matrix(x, "x"), _ptr(w_gate), _ptr(w_up),
                                   _matrix(w_gate, "w_gate"), _ptr(w_down), _matrix(w_down, "w_down"), d_ff, _ptr(y),
                                   _matrix(y, "y"), int(chunk), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(x)))
    return y


def lwm_profile_enable(on: bool = True):
    _check(lib().lwm_profile_enable(int(bool(on))))


def lwm_profile_reset():
    _check(lib().lwm_profile_reset())


def lwm_profile_read() -> dict:
    """{kernel name: (total milliseconds, launches)} since the last reset (waits for the events)."""
    L = lib()
    out = {}
    for i in range(L.lwm_profile_count()):
        name, ms, n = ctypes.c_char_p(), ctypes.c_double(), ctypes.c_int64()
        _check(L.lwm_profile_get(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(n)))
        out[name.value.decode()] = (ms.value, n.value)
    return out
