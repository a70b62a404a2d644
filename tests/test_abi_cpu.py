"""The C-ABI library on the host: it loads, exports every declared symbol, and rejects bad
arguments with the documented status before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

from ring_causal_attention_amd import lwm

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lwm_attn.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lwm_[a-z0-9_]+)\s*\(", text)))


def _lib():
    if not os.path.exists(lwm.LIB_PATH):
        pytest.skip("library not built (run __graft_entry__.build())")
    return lwm.lib()


def test_exports_every_declared_symbol():
    L = _lib()
    names = declared_functions()
    assert set(names) == set(lwm.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n
    assert L.lwm_abi_version() == 4
    assert L.lwm_last_error() == b""


def t4(ptr=16, dtype=0, B=1, L=8, H=2, D=128, sB=None, sL=None, sH=None):
    sH = D if sH is None else sH
    sL = H * D if sL is None else sL
    sB = L * H * D if sB is None else sB
    return lwm.Tensor4(ptr, dtype, 0, B, L, H, D, sB, sL, sH)


def fwd(q=None, k=None, v=None, o=None, seg_q=None, seg_k=None, qo=0, ko=0, causal=1, scale=0.0):
    L = _lib()
    q, k, v, o = q or t4(), k or t4(), v or t4(), o or t4()
    st = L.lwm_blockattn_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), seg_q, seg_k, qo, ko, causal, scale,
                             ctypes.byref(o), None, None)
    return st, L.lwm_last_error().decode()


@pytest.mark.parametrize("kwargs,status,needle", [
    ({"q": t4(ptr=0)}, -1, "NULL"),
    ({"q": t4(ptr=8)}, -1, "aligned"),
    ({"q": t4(D=64), "k": t4(D=64), "v": t4(D=64), "o": t4(D=64)}, -2, "128"),
    ({"k": t4(H=3), "v": t4(H=3)}, -1, "mismatch"),
    ({"v": t4(L=9)}, -1, "mismatch"),
    ({"o": t4(L=9)}, -1, "mismatch"),
    ({"q": t4(dtype=1)}, -2, "mixed"),
    ({"q": t4(dtype=7)}, -2, "dtype"),
    ({"q": t4(sL=255)}, -1, "multiples"),
    ({"seg_q": 16}, -1, "both"),
    ({"qo": -1}, -1, "offsets"),
    ({"causal": 2}, -1, "causal"),
    ({"scale": -1.0}, -1, "scale"),
    ({"scale": float("nan")}, -1, "scale"),
])
def test_forward_validation(kwargs, status, needle):
    st, msg = fwd(**kwargs)
    assert st == status and needle in msg, (st, msg)


def test_backward_and_ring_validation():
    L = _lib()
    q = t4()
    r = ctypes.byref
    ws = L.lwm_blockattn_bwd_workspace_size(1, 2, 8, 8, 128)
    assert ws >= 1 * 2 * 8 * 4 and ws % 256 == 0
    st = L.lwm_blockattn_bwd(r(q), r(q), r(q), r(q), 16, r(q), None, None, 0, 0, 1, 0.0, r(q), r(q), r(q), 256, ws - 1, None)
    assert st == -3 and "workspace" in L.lwm_last_error().decode()
    st = L.lwm_blockattn_bwd(r(q), r(q), r(q), r(q), None, r(q), None, None, 0, 0, 1, 0.0, r(q), r(q), r(q), 256, ws, None)
    assert st == -1 and "lse" in L.lwm_last_error().decode()
    f = t4(dtype=1)
    st = L.lwm_blockattn_bwd(r(f), r(f), r(f), r(f), 16, r(f), None, None, 0, 0, 1, 0.0, r(f), r(f), r(f), 256, ws, None)
    assert st == -2
    oacc = t4(dtype=0)
    st = L.lwm_ring_step(r(q), r(q), r(q), None, None, 0, 0, 1, 0.0, r(oacc), 16, None, None)
    assert st == -1 and "float32" in L.lwm_last_error().decode()
    oacc = t4(dtype=1, L=9)
    st = L.lwm_ring_step(r(q), r(q), r(q), None, None, 0, 0, 1, 0.0, r(oacc), 16, None, None)
    assert st == -1


def test_ring_backward_validation():
    L = _lib()
    r = ctypes.byref
    q = t4()
    acc = t4(dtype=1)
    ws = L.lwm_blockattn_bwd_workspace_size(1, 2, 8, 8, 128)
    args = lambda dqa, dka, dva, lse=16, nbytes=ws: (r(q), r(q), r(q), r(q), lse, r(q), None, None, 0, 0, 1, 0.0,
                                                    r(dqa), r(dka), r(dva), 256, nbytes, None)
    st = L.lwm_ring_step_bwd(*args(q, acc, acc))  # bf16 accumulator
    assert st == -1 and "float32" in L.lwm_last_error().decode()
    st = L.lwm_ring_step_bwd(*args(acc, t4(dtype=1, L=9), acc))
    assert st == -1 and "mismatch" in L.lwm_last_error().decode()
    st = L.lwm_ring_step_bwd(*args(acc, acc, acc, nbytes=ws - 1))
    assert st == -3 and "workspace" in L.lwm_last_error().decode()
    st = L.lwm_ring_step_bwd(*args(acc, acc, acc, lse=None))
    assert st == -1 and "lse" in L.lwm_last_error().decode()
    assert L.lwm_ring_step_bwd(r(q), r(q), r(q), r(q), 16, r(q), 16, None, 0, 0, 1, 0.0, r(acc), r(acc), r(acc),
                               256, ws, None) == -1


def test_rope_validation():
    L = _lib()
    r = ctypes.byref
    x = t4()
    for args, status in [((r(x), r(x), None, None, 0, 0.0, 0, 0, None), -1),
                         ((r(x), r(x), None, None, 0, 1e4, 5, 0, None), -1),
                         ((r(x), r(t4(L=4)), None, None, 0, 1e4, 0, 0, None), -1),
                         ((r(t4(D=24)), r(t4(D=24)), None, None, 0, 1e4, 0, 0, None), -2),
                         ((r(x), r(x), None, None, 0, 1e4, 0, 3, None), -1)]:
        assert L.lwm_rope_apply(*args) == status, args


def test_fused_rope_validation():
    """The fused-RoPE entry points check the RoPE descriptor and the extra outputs before any launch."""
    L = _lib()
    r = ctypes.byref
    q = t4()
    good = lwm.RopeArgs(1e6, 0, 0, 0, 0)

    def fwd_rope(rope=good, q_rot=None, k_rot=q, seg=None, dtype=0, qp=16):
        x = t4(dtype=dtype, ptr=qp)
        st = L.lwm_blockattn_fwd_rope(r(x), r(t4(dtype=dtype)), r(t4(dtype=dtype)), seg, seg, 0, 0, 1, 0.0,
                                      None if rope is None else r(rope), r(t4(dtype=dtype)), None,
                                      None if q_rot is None else r(q_rot), None if k_rot is None else r(k_rot), None)
        return st, L.lwm_last_error().decode()

    for kwargs, status, needle in [
        ({"rope": None}, -1, "rope is NULL"),
        ({"rope": lwm.RopeArgs(0.0, 0, 0, 0, 0)}, -1, "theta"),
        ({"rope": lwm.RopeArgs(float("inf"), 0, 0, 0, 0)}, -1, "theta"),
        ({"rope": lwm.RopeArgs(1e6, 2, 0, 0, 0)}, -1, "layout"),
        ({"rope": lwm.RopeArgs(1e6, 0, 2, 0, 0)}, -1, "restart"),
        ({"rope": lwm.RopeArgs(1e6, 0, 1, 0, 0)}, -1, "restart = 1 needs"),
        ({"rope": lwm.RopeArgs(1e6, 0, 0, 1 << 41, 0)}, -1, "offsets"),
        ({"k_rot": None}, -1, "k_rot"),
        ({"k_rot": t4(L=9)}, -1, "mismatch"),
        ({"q_rot": t4(ptr=16)}, -1, "overlap"),
        ({"q_rot": t4(H=3)}, -1, "mismatch"),
        ({"dtype": 1, "k_rot": t4(dtype=1)}, -2, "bf16"),
    ]:
        st, msg = fwd_rope(**kwargs)
        assert st == status and needle in msg, (kwargs, st, msg)
    # in-place key rotation (k_rot == k) needs the same strides
    st, msg = fwd_rope(k_rot=t4(sH=256, sL=512, sB=4096))
    assert st == -1 and "strides" in msg, (st, msg)
    ws = L.lwm_blockattn_bwd_workspace_size(1, 2, 8, 8, 128)

    def bwd_rope(rope=good, seg=None, nbytes=ws, dk=q):
        return L.lwm_blockattn_bwd_rope(r(q), r(q), r(q), r(q), 16, r(q), seg, seg, 0, 0, 1, 0.0,
                                        None if rope is None else r(rope), r(q), r(dk), r(q), 256, nbytes, None)

    assert bwd_rope(rope=None) == -1 and "rope" in L.lwm_last_error().decode()
    assert bwd_rope(rope=lwm.RopeArgs(1e6, 0, 1, 0, 0)) == -1 and "restart" in L.lwm_last_error().decode()
    assert bwd_rope(nbytes=ws - 1) == -3
    assert bwd_rope(dk=t4(L=9)) == -1 and "mismatch" in L.lwm_last_error().decode()


def test_ffn_validation():
    L = _lib()
    ws = L.lwm_blockwise_ffn_workspace_size(300, 96, 128)
    assert ws >= 128 * 96 * 2 and ws % 256 == 0
    assert L.lwm_blockwise_ffn_workspace_size(100, 96, 128) >= 100 * 96 * 2

    def call(rows=300, d_model=64, ldx=64, x=256, wg=256, wu=256, ldw=64, wd=256, ldwd=96, d_ff=96, y=256, ldy=64,
             chunk=128, ws_ptr=256, nbytes=ws):
        st = L.lwm_blockwise_ffn(x, rows, d_model, ldx, wg, wu, ldw, wd, ldwd, d_ff, y, ldy, chunk, ws_ptr, nbytes,
                                 None)
        return st, L.lwm_last_error().decode()

    for kwargs, status, needle in [
        ({"x": None}, -1, "NULL"),
        ({"wu": 264}, -1, "aligned"),
        ({"d_model": 48, "ldx": 48, "ldw": 48, "ldy": 48}, -2, "multiples of 32"),
        ({"d_ff": 0}, -2, "multiples of 32"),
        ({"ldx": 32}, -1, "below"),
        ({"ldwd": 100}, -1, "multiple of 8"),
        ({"ldy": 1 << 22}, -2, "8 MiB"),
        ({"chunk": 0}, -1, "chunk"),
        ({"rows": -1}, -1, "rows"),
        ({"nbytes": ws - 1}, -3, "workspace"),
        ({"ws_ptr": 128}, -3, "aligned"),
    ]:
        st, msg = call(**kwargs)
        assert st == status and needle in msg, (kwargs, st, msg)
    # rows = 0 is a no-op that touches no pointer
    assert call(rows=0, x=None, wg=None, wu=None, wd=None, y=None, ws_ptr=None, nbytes=0)[0] == 0
