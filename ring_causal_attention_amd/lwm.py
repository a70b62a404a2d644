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
           "lwm_blockattn_bwd_workspace_size", "lwm_blockattn_bwd_workspace_size_ds", "lwm_blockattn_bwd", "lwm_blockattn_bwd_noalloc", "lwm_blockattn_fwd_rope",
           "lwm_blockattn_bwd_rope", "lwm_ring_step", "lwm_ring_step_bwd",
           "lwm_blockwise_ffn_workspace_size", "lwm_blockwise_ffn", "lwm_profile_enable", "lwm_profile_reset", "lwm_profile_count", "lwm_profile_get",
           "lwm_probe_mfma_bf16"]


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
    L.lwm_blockattn_bwd_workspace_size_ds.restype = ctypes.c_size_t
    L.lwm_blockattn_bwd_workspace_size_ds.argtypes = [I64, I64, I64, I64, I64, I64, I64, I32, I64]
    L.lwm_blockattn_bwd.restype = ctypes.c_int
    L.lwm_blockattn_bwd.argtypes = [P, P, P, P, VP, P, VP, VP, I64, I64, I32, F32, P, P, P, VP, ctypes.c_size_t, VP]
    L.lwm_blockattn_bwd_noalloc.restype = ctypes.c_int
    L.lwm_blockattn_bwd_noalloc.argtypes = [P, P, P, P, VP, P, VP, VP, I64, I64, I32, F32, P, P, P, VP]
    R = ctypes.POINTER(RopeArgs)
    L.lwm_blockattn_fwd_rope.restype = ctypes.c_int
    L.lwm_blockattn_fwd_rope.argtypes = [P, P, P, VP, VP, I64, I64, I32, F32, R, P, VP, P, P, VP]
    L.lwm_blockattn_bwd_rope.restype = ctypes.c_int
    L.lwm_blockattn_bwd_rope.argtypes = [P, P, P, P, VP, P, VP, VP, I64, I64, I32, F32, R, P, P, P, VP,
                                         ctypes.c_size_t, VP]
    L.lwm_ring_step.restype = ctypes.c_int
    L.lwm_ring_step.argtypes = [P, P, P, VP, VP, I64, I64, I32, F32, P, VP, P, VP]
    L.lwm_ring_step_bwd.restype = ctypes.c_int
    L.lwm_ring_step_bwd.argtypes = [P, P, P, P, VP, P, VP, VP, I64, I64, I32, F32, P, P, P, VP, ctypes.c_size_t, I32,
                                    VP]
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
    L.lwm_probe_mfma_bf16.restype = ctypes.c_int
    L.lwm_probe_mfma_bf16.argtypes = [VP, VP, I32, I32, VP]
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise LwmError(status, lib().lwm_last_error().decode(errors="replace"))


def _on_device(t: torch.Tensor, name: str, device) -> None:
    """Device memory only, and on the device of the call's first operand: the library takes raw
    pointers and cannot tell host memory, or another GPU's, from its own."""
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor, got one on {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, but the call's tensors are on {device}")


def tensor4(t: torch.Tensor | None, name: str = "tensor", device=None) -> Tensor4 | None:
    """Describe a [B, L, H, D] GPU tensor (feature stride 1) for the ABI."""
    if t is None:
        return None
    if t.dim() != 4:
        raise ValueError(f"{name}: expected a [B, L, H, D] tensor, got shape {tuple(t.shape)}")
    if t.dtype == torch.bfloat16:
        dt = LWM_BF16
    elif t.dtype == torch.float32:
        dt = LWM_FP32
    else:
        raise ValueError(f"{name}: unsupported dtype {t.dtype}")
    _on_device(t, name, device)
    B, L, H, D = t.shape
    if t.numel() == 0:  # no element is addressed: describe it with contiguous strides
        return Tensor4(t.data_ptr(), dt, 0, B, L, H, D, L * H * D, H * D, D)
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError(f"{name}: the feature dimension must be contiguous")
    return Tensor4(t.data_ptr(), dt, 0, B, L, H, D, t.stride(0), t.stride(1), t.stride(2))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ref(s):
    return None if s is None else ctypes.byref(s)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _seg(s, B, L, device, name="segment ids"):
    """Segment ids or positions: contiguous int32 [B, L] on the call's device (or None)."""
    if s is None:
        return None
    if s.dtype != torch.int32 or not s.is_contiguous():
        raise ValueError(f"{name}: must be contiguous int32 [B, L]")
    if tuple(s.shape) != (B, L):
        raise ValueError(f"{name}: shape {tuple(s.shape)}, expected {(B, L)}")
    _on_device(s, name, device)
    return s


def _rows(t, B, H, L, device, name):
    """Per-row float32 [B, H, L] (lse, lse_acc): contiguous, on the call's device (or None)."""
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous float32 [B, H, L]")
    if tuple(t.shape) != (B, H, L):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {(B, H, L)}")
    _on_device(t, name, device)
    return t


def _workspace(ws, device):
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("workspace: must be a contiguous 1-D uint8 tensor")
    _on_device(ws, "workspace", device)
    return ws


def lwm_abi_version() -> int:
    return lib().lwm_abi_version()


def lwm_rope_apply(x, y=None, pos=None, seg=None, pos_offset=0, theta=10000.0, layout="half", inverse=False):
    """RoPE of x into y (default: a new tensor; pass y=x for in place).  Returns y."""
    y = torch.empty_like(x) if y is None else y
    B, L = x.shape[0], x.shape[1]
    dv = x.device
    _check(lib().lwm_rope_apply(_ref(tensor4(x, "x", dv)), _ref(tensor4(y, "y", dv)), _ptr(_seg(pos, B, L, dv, "pos")),
                                _ptr(_seg(seg, B, L, dv, "seg")), int(pos_offset), float(theta), LAYOUTS[layout],
                                int(bool(inverse)), _stream(x)))
    return y


def lwm_blockattn_fwd(q, k, v, seg_q=None, seg_k=None, q_offset=0, k_offset=0, causal=True, scale=0.0,
                      o=None, lse=None, want_lse=True):
    """Forward; returns (o, lse) with lse float32 [B, H, Lq] (None if want_lse is False)."""
    B, Lq, H, _ = q.shape
    o = torch.empty_like(q) if o is None else o
    if lse is None and want_lse:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    dv, Lk = q.device, k.shape[1]
    _check(lib().lwm_blockattn_fwd(_ref(tensor4(q, "q", dv)), _ref(tensor4(k, "k", dv)), _ref(tensor4(v, "v", dv)),
                                   _ptr(_seg(seg_q, B, Lq, dv, "seg_q")), _ptr(_seg(seg_k, B, Lk, dv, "seg_k")),
                                   int(q_offset), int(k_offset), int(bool(causal)), float(scale),
                                   _ref(tensor4(o, "o", dv)), _ptr(_rows(lse, B, H, Lq, dv, "lse")), _stream(q)))
    return o, lse


def lwm_blockattn_bwd_workspace_size(B, H, Lq, Lk, D) -> int:
    return int(lib().lwm_blockattn_bwd_workspace_size(B, H, Lq, Lk, D))


def lwm_blockattn_bwd_workspace_size_ds(B, H, Lq, Lk, D, heads_per_pass, q_offset=0, k_offset=0, causal=True) -> int:
    return int(lib().lwm_blockattn_bwd_workspace_size_ds(B, H, Lq, Lk, D, int(q_offset), int(k_offset),
                                                         int(bool(causal)), heads_per_pass))


# Most device memory the binding gives the stored dS when it allocates a backward workspace itself
# (it allocates only the slots of the pairs per pass it picks).
DS_BUDGET_BYTES = 80 << 30


# Fewest (batch, head) pairs per pass for which the binding picks the stored-dS backward: with
# fewer, each pass's launches leave too much of the chip idle at their ends (measured on a packed
# row of 65536 tokens: 8 pairs per pass slower than recomputing, 16 faster).
DS_MIN_HEADS = 16


def default_ds_heads(B, H, Lq, Lk, D, budget=DS_BUDGET_BYTES, q_offset=0, k_offset=0, causal=True) -> int:
    """(batch, head) pairs per pass of the stored-dS backward whose slots fit in ``budget`` bytes:
    all B*H if they fit, else the largest multiple of 8; 0 (the recomputing path) when fewer than
    min(B*H, DS_MIN_HEADS) fit."""
    slot = (lwm_blockattn_bwd_workspace_size_ds(B, H, Lq, Lk, D, 1, q_offset, k_offset, causal)
            - lwm_blockattn_bwd_workspace_size(B, H, Lq, Lk, D))
    if slot <= 0:
        return 0
    bh = B * H
    g = min(bh, budget // slot)
    if g < bh:
        g -= g % 8
    return g if g >= min(bh, DS_MIN_HEADS) else 0


def bwd_workspace(B, H, Lq, Lk, D, device, ds_heads=None, q_offset=0, k_offset=0, causal=True):
    """A backward workspace for a call with these sizes, offsets and causal flag: with room for
    the stored dS of ``ds_heads`` pairs per pass (None: ``default_ds_heads``; 0: none, the
    recomputing path).  Sized with causal=False it suits any offsets."""
    heads = (default_ds_heads(B, H, Lq, Lk, D, q_offset=q_offset, k_offset=k_offset, causal=causal)
             if ds_heads is None else int(ds_heads))
    size = (lwm_blockattn_bwd_workspace_size_ds(B, H, Lq, Lk, D, heads, q_offset, k_offset, causal) if heads > 0
            else lwm_blockattn_bwd_workspace_size(B, H, Lq, Lk, D))
    return torch.empty(size, dtype=torch.uint8, device=device)


def lwm_blockattn_bwd(q, k, v, o, lse, dout, seg_q=None, seg_k=None, q_offset=0, k_offset=0, causal=True,
                      scale=0.0, dq=None, dk=None, dv=None, workspace=None, ds_heads=None):
    """Backward; returns (dq, dk, dv) w.r.t. the operands given (the rotated Q', K').  Without a
    ``workspace`` one is allocated with room for ``ds_heads`` (see ``bwd_workspace``)."""
    B, Lq, H, D = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = bwd_workspace(B, H, Lq, k.shape[1], D, q.device, ds_heads, q_offset, k_offset, causal)
    d, Lk = q.device, k.shape[1]
    _check(lib().lwm_blockattn_bwd(_ref(tensor4(q, "q", d)), _ref(tensor4(k, "k", d)), _ref(tensor4(v, "v", d)),
                                   _ref(tensor4(o, "o", d)), _ptr(_rows(lse, B, H, Lq, d, "lse")),
                                   _ref(tensor4(dout, "dout", d)), _ptr(_seg(seg_q, B, Lq, d, "seg_q")),
                                   _ptr(_seg(seg_k, B, Lk, d, "seg_k")), int(q_offset), int(k_offset),
                                   int(bool(causal)), float(scale), _ref(tensor4(dq, "dq", d)),
                                   _ref(tensor4(dk, "dk", d)), _ref(tensor4(dv, "dv", d)),
                                   _ptr(_workspace(workspace, d)), workspace.numel(), _stream(q)))
    return dq, dk, dv


def lwm_blockattn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, seg_q=None, seg_k=None, q_offset=0, k_offset=0,
                              causal=True, scale=0.0):
    """lwm_blockattn_bwd with the library's static per-GPU workspace: the caller passes every
    output (nothing is allocated here or in the call).  Returns (dq, dk, dv)."""
    B, Lq, H, D = q.shape
    d, Lk = q.device, k.shape[1]
    _check(lib().lwm_blockattn_bwd_noalloc(_ref(tensor4(q, "q", d)), _ref(tensor4(k, "k", d)),
                                           _ref(tensor4(v, "v", d)), _ref(tensor4(o, "o", d)),
                                           _ptr(_rows(lse, B, H, Lq, d, "lse")), _ref(tensor4(dout, "dout", d)),
                                           _ptr(_seg(seg_q, B, Lq, d, "seg_q")), _ptr(_seg(seg_k, B, Lk, d, "seg_k")),
                                           int(q_offset), int(k_offset), int(bool(causal)), float(scale),
                                           _ref(tensor4(dq, "dq", d)), _ref(tensor4(dk, "dk", d)),
                                           _ref(tensor4(dv, "dv", d)), _stream(q)))
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
    d, Lk = q.device, k.shape[1]
    _check(lib().lwm_blockattn_fwd_rope(_ref(tensor4(q, "q", d)), _ref(tensor4(k, "k", d)), _ref(tensor4(v, "v", d)),
                                        _ptr(_seg(seg_q, B, Lq, d, "seg_q")), _ptr(_seg(seg_k, B, Lk, d, "seg_k")),
                                        int(q_offset), int(k_offset), int(bool(causal)), float(scale),
                                        ctypes.byref(ra), _ref(tensor4(o, "o", d)),
                                        _ptr(_rows(lse, B, H, Lq, d, "lse")), _ref(tensor4(q_rot, "q_rot", d)),
                                        _ref(tensor4(k_rot, "k_rot", d)), _stream(q)))
    return o, lse, q_rot, k_rot


def lwm_blockattn_bwd_rope(q_rot, k_rot, v, o, lse, dout, theta, seg_q=None, seg_k=None, q_offset=0, k_offset=0,
                           causal=True, scale=0.0, layout="half", restart=False, q_pos_offset=0, k_pos_offset=0,
                           dq=None, dk=None, dv=None, workspace=None, ds_heads=None):
    """Backward with the inverse RoPE inside the call; returns (dq, dk, dv) w.r.t. the pre-RoPE Q, K."""
    B, Lq, H, D = q_rot.shape
    dq = torch.empty_like(q_rot) if dq is None else dq
    dk = torch.empty_like(k_rot) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = bwd_workspace(B, H, Lq, k_rot.shape[1], D, q_rot.device, ds_heads, q_offset, k_offset, causal)
    ra = rope_args(theta, layout, restart, q_pos_offset, k_pos_offset)
    d, Lk = q_rot.device, k_rot.shape[1]
    _check(lib().lwm_blockattn_bwd_rope(_ref(tensor4(q_rot, "q_rot", d)), _ref(tensor4(k_rot, "k_rot", d)),
                                        _ref(tensor4(v, "v", d)), _ref(tensor4(o, "o", d)),
                                        _ptr(_rows(lse, B, H, Lq, d, "lse")), _ref(tensor4(dout, "dout", d)),
                                        _ptr(_seg(seg_q, B, Lq, d, "seg_q")), _ptr(_seg(seg_k, B, Lk, d, "seg_k")),
                                        int(q_offset), int(k_offset), int(bool(causal)), float(scale),
                                        ctypes.byref(ra), _ref(tensor4(dq, "dq", d)), _ref(tensor4(dk, "dk", d)),
                                        _ref(tensor4(dv, "dv", d)), _ptr(_workspace(workspace, d)),
                                        workspace.numel(), _stream(q_rot)))
    return dq, dk, dv


def lwm_ring_step(q, k_shard, v_shard, o_acc, lse_acc, seg_q=None, seg_k=None, q_offset=0, k_offset=0,
                  causal=True, scale=0.0, o_final=None):
    """Fold one KV shard into (o_acc float32 [B, Lq, H, D], lse_acc float32 [B, H, Lq]) in place."""
    B, Lq, H, _ = q.shape
    d, Lk = q.device, k_shard.shape[1]
    if lse_acc is None:
        raise ValueError("lse_acc: required")
    _check(lib().lwm_ring_step(_ref(tensor4(q, "q", d)), _ref(tensor4(k_shard, "k_shard", d)),
                               _ref(tensor4(v_shard, "v_shard", d)), _ptr(_seg(seg_q, B, Lq, d, "seg_q")),
                               _ptr(_seg(seg_k, B, Lk, d, "seg_k")), int(q_offset), int(k_offset), int(bool(causal)),
                               float(scale), _ref(tensor4(o_acc, "o_acc", d)),
                               _ptr(_rows(lse_acc, B, H, Lq, d, "lse_acc")), _ref(tensor4(o_final, "o_final", d)),
                               _stream(q)))
    return o_acc, lse_acc


RING_BWD_REUSE_WORKSPACE = 1


def lwm_ring_step_bwd(q, k_shard, v_shard, o, lse, dout, dq_acc, dk_acc, dv_acc, seg_q=None, seg_k=None,
                      q_offset=0, k_offset=0, causal=True, scale=0.0, workspace=None, reuse_workspace=False,
                      ds_heads=None):
    """Add one KV shard's share of the gradients into dq_acc (float32, like q) and dk_acc,
    dv_acc (float32, like k_shard), in place; o and lse are the forward's results over all shards.
    ``reuse_workspace``: the workspace already holds this query block's delta and rescaled lse
    from an earlier step of the same ring (same q, o, lse, dout), so that pass is skipped.
    Without a ``workspace`` one is allocated with room for ``ds_heads`` (see ``bwd_workspace``)."""
    B, Lq, H, D = q.shape
    if workspace is None:
        if reuse_workspace:
            raise ValueError("reuse_workspace needs the workspace an earlier step of the ring wrote")
        workspace = bwd_workspace(B, H, Lq, k_shard.shape[1], D, q.device, ds_heads, q_offset, k_offset, causal)
    d, Lk = q.device, k_shard.shape[1]
    _check(lib().lwm_ring_step_bwd(_ref(tensor4(q, "q", d)), _ref(tensor4(k_shard, "k_shard", d)),
                                   _ref(tensor4(v_shard, "v_shard", d)), _ref(tensor4(o, "o", d)),
                                   _ptr(_rows(lse, B, H, Lq, d, "lse")), _ref(tensor4(dout, "dout", d)),
                                   _ptr(_seg(seg_q, B, Lq, d, "seg_q")), _ptr(_seg(seg_k, B, Lk, d, "seg_k")),
                                   int(q_offset), int(k_offset), int(bool(causal)), float(scale),
                                   _ref(tensor4(dq_acc, "dq_acc", d)), _ref(tensor4(dk_acc, "dk_acc", d)),
                                   _ref(tensor4(dv_acc, "dv_acc", d)), _ptr(_workspace(workspace, d)),
                                   workspace.numel(), RING_BWD_REUSE_WORKSPACE if reuse_workspace else 0,
                                   _stream(q)))
    return dq_acc, dk_acc, dv_acc


def _matrix(t, name, device=None):
    if t.dtype != torch.bfloat16 or t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name}: expected a bf16 matrix with contiguous rows, got {t.dtype} {tuple(t.shape)}")
    _on_device(t, name, device)
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
    d = x.device
    _matrix(w_up, "w_up", d)
    _check(lib().lwm_blockwise_ffn(_ptr(x), rows, d_model, _matrix(x, "x", d), _ptr(w_gate), _ptr(w_up),
                                   _matrix(w_gate, "w_gate", d), _ptr(w_down), _matrix(w_down, "w_down", d), d_ff,
                                   _ptr(y), _matrix(y, "y", d), int(chunk), _ptr(_workspace(workspace, d)),
                                   workspace.numel(), _stream(x)))
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


def lwm_probe_mfma_bf16(src: torch.Tensor, iters: int, sink: torch.Tensor | None = None) -> torch.Tensor:
    """Matrix-core rate probe: ``src`` is a bf16 GPU tensor of blocks * 256 * 128 values; one
    launch of blocks = src.numel() // 32768 workgroups, each wave ``iters`` rounds of four
    32x32x16 bf16 MFMAs on register-resident operands read from ``src``.  Returns ``sink``
    (float32, one value per lane)."""
    _on_device(src, "src", None)
    if src.dtype != torch.bfloat16 or not src.is_contiguous() or src.numel() % (256 * 128) or src.numel() == 0:
        raise ValueError("src: expected a contiguous bf16 GPU tensor of blocks * 256 * 128 values")
    blocks = src.numel() // (256 * 128)
    if sink is None:
        sink = torch.empty(blocks * 256, dtype=torch.float32, device=src.device)
    _on_device(sink, "sink", src.device)
    if sink.dtype != torch.float32 or not sink.is_contiguous() or sink.numel() != blocks * 256:
        raise ValueError(f"sink: expected a contiguous float32 GPU tensor of {blocks * 256} values")
    _check(lib().lwm_probe_mfma_bf16(_ptr(src), _ptr(sink), blocks, int(iters), _stream(src)))
    return sink
