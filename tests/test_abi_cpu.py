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
    assert L.lwm_abi_version() == 8
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
    args = lambda dqa, dka, dva, lse=16, nbytes=ws, flags=0: (r(q), r(q), r(q), r(q), lse, r(q), None, None, 0, 0, 1,
                                                             0.0, r(dqa), r(dka), r(dva), 256, nbytes, flags, None)
    st = L.lwm_ring_step_bwd(*args(q, acc, acc))  # bf16 accumulator
    assert st == -1 and "float32" in L.lwm_last_error().decode()
    st = L.lwm_ring_step_bwd(*args(acc, t4(dtype=1, L=9), acc))
    assert st == -1 and "mismatch" in L.lwm_last_error().decode()
    st = L.lwm_ring_step_bwd(*args(acc, acc, acc, nbytes=ws - 1))
    assert st == -3 and "workspace" in L.lwm_last_error().decode()
    st = L.lwm_ring_step_bwd(*args(acc, acc, acc, lse=None))
    assert st == -1 and "lse" in L.lwm_last_error().decode()
    assert L.lwm_ring_step_bwd(r(q), r(q), r(q), r(q), 16, r(q), 16, None, 0, 0, 1, 0.0, r(acc), r(acc), r(acc),
                               256, ws, 0, None) == -1
    for flags in (2, -1):
        st = L.lwm_ring_step_bwd(*args(acc, acc, acc, flags=flags))
        assert st == -1 and "flags" in L.lwm_last_error().decode()


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


def test_grid_bound_covers_key_tiles():
    """Launch grids are (query or key tiles of 128) x B x H workgroups: a short query block against a
    very long key side is refused on the host, like a long query side (no int overflow on device)."""
    L = _lib()
    r = ctypes.byref
    big_h = 65535
    q = t4(B=65535, L=1, H=big_h, sL=big_h * 128, sB=big_h * 128)
    k = t4(B=65535, L=1 << 20, H=big_h, sL=big_h * 128, sB=(1 << 20) * big_h * 128)
    ws = L.lwm_blockattn_bwd_workspace_size(65535, big_h, 1, 1 << 20, 128)
    st = L.lwm_blockattn_bwd(r(q), r(k), r(k), r(q), 16, r(q), None, None, 0, 0, 1, 0.0, r(q), r(k), r(k), 256, ws,
                             None)
    assert st == -2 and "grid too large" in L.lwm_last_error().decode(), L.lwm_last_error()
    st = L.lwm_blockattn_fwd(r(q), r(k), r(k), None, None, 0, 0, 1, 0.0, r(q), None, None)
    assert st == -2 and "grid too large" in L.lwm_last_error().decode()
    # the same sizes with a small batch pass the grid bound: the call gets as far as a later check
    # (a negative scale) and is refused there.  No call in this file may pass every check: its
    # descriptors point at address 16, and a launch on a machine with a GPU would fault it.
    q1 = t4(B=1, L=1, H=2)
    k1 = t4(B=1, L=1 << 20, H=2)
    st = L.lwm_blockattn_fwd(r(q1), r(k1), r(k1), None, None, 0, 0, 1, -1.0, r(q1), None, None)
    assert st == -1 and "scale" in L.lwm_last_error().decode(), L.lwm_last_error()


def test_binding_rejects_host_and_misshapen_tensors():
    """The Python binding refuses CPU tensors and misshapen lse / segment ids / workspace before any
    call into the library (a raw host pointer would reach the GPU otherwise)."""
    import torch
    _lib()
    q = torch.zeros((1, 8, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        lwm.lwm_blockattn_fwd(q, q, q, o=q.clone(), want_lse=False)
    with pytest.raises(ValueError, match="GPU tensor"):
        lwm.lwm_rope_apply(q, theta=1e4)
    # the argument checks every entry point applies (shape and dtype before the device)
    dev = torch.device("cuda", 0)
    with pytest.raises(ValueError, match="lse: shape"):
        lwm._rows(torch.zeros((1, 2, 7)), 1, 2, 8, dev, "lse")
    with pytest.raises(ValueError, match="lse: must be contiguous float32"):
        lwm._rows(torch.zeros((1, 2, 8), dtype=torch.float64), 1, 2, 8, dev, "lse")
    with pytest.raises(ValueError, match="lse_acc: must be contiguous"):
        lwm._rows(torch.zeros((1, 8, 2)).transpose(1, 2), 1, 2, 8, dev, "lse_acc")
    with pytest.raises(ValueError, match="GPU tensor"):
        lwm._rows(torch.zeros((1, 2, 8)), 1, 2, 8, dev, "lse")
    with pytest.raises(ValueError, match="seg_k: shape"):
        lwm._seg(torch.zeros((1, 7), dtype=torch.int32), 1, 8, dev, "seg_k")
    with pytest.raises(ValueError, match="int32"):
        lwm._seg(torch.zeros((1, 8), dtype=torch.int64), 1, 8, dev, "seg")
    with pytest.raises(ValueError, match="GPU tensor"):
        lwm._seg(torch.zeros((1, 8), dtype=torch.int32), 1, 8, dev, "seg")
    with pytest.raises(ValueError, match="workspace"):
        lwm._workspace(torch.zeros(4096, dtype=torch.float32), dev)
    with pytest.raises(ValueError, match="GPU tensor"):
        lwm._workspace(torch.zeros(4096, dtype=torch.uint8), dev)
    with pytest.raises(ValueError, match="x: expected a bf16 matrix"):
        lwm._matrix(torch.zeros((4, 64)), "x", dev)


def test_noalloc_backward_size_limit():
    """The allocation-free backward refuses B*H*Lq beyond its static workspace on the host."""
    L = _lib()
    r = ctypes.byref
    q = t4(B=1, L=1 << 16, H=33, sL=33 * 128, sB=(1 << 16) * 33 * 128)
    st = L.lwm_blockattn_bwd_noalloc(r(q), r(q), r(q), r(q), 16, r(q), None, None, 0, 0, 1, 0.0, r(q), r(q), r(q),
                                     None)
    assert st == -2 and "static workspace" in L.lwm_last_error().decode()


@pytest.mark.parametrize("src,sink,blocks,iters,needle", [
    (None, 16, 4, 64, "NULL"),
    (16, None, 4, 64, "NULL"),
    (8, 16, 4, 64, "aligned"),
    (16, 2, 4, 64, "aligned"),
    (16, 16, 0, 64, "blocks"),
    (16, 16, 4097, 64, "blocks"),
    (16, 16, 4, 0, "iters"),
    (16, 16, 4, 12, "iters"),
    (16, 16, 4, (1 << 24) + 8, "iters"),
])
def test_mfma_probe_validation(src, sink, blocks, iters, needle):
    """The matrix-core rate probe checks its arguments on the host and launches nothing otherwise."""
    L = _lib()
    st = L.lwm_probe_mfma_bf16(src, sink, blocks, iters, None)
    assert st == -1 and needle in L.lwm_last_error().decode()


def test_mfma_probe_binding_rejects_host_and_misshapen_tensors():
    import torch
    with pytest.raises(ValueError, match="GPU tensor"):
        lwm.lwm_probe_mfma_bf16(torch.zeros(256 * 128, dtype=torch.bfloat16), 8)


def ds_blocks_brute(Lq, Lk, q_offset, k_offset, causal):
    """Blocks of one stored-dS slot, summed key block by key block: each keeps the 64-query blocks
    from its first causally visible query block on (all of them without the causal mask)."""
    nqb, nkb = -(-Lq // 256) * 256 // 64, -(-Lk // 64)
    total = 0
    for kb in range(nkb):
        lo = min(max(kb + (k_offset - q_offset) // 64, 0), nqb) if causal else 0
        # lo is the block of the first query q with q_offset + q >= k_offset + 64 kb
        first = max(0, k_offset + 64 * kb - q_offset) if causal else 0
        assert lo == min(first // 64, nqb)
        total += nqb - lo
    return total


def test_stored_ds_workspace_size():
    """lwm_blockattn_bwd_workspace_size_ds: the two float32 rows per query, then one slot of 64 x 64
    bf16 blocks per (batch, head) pair of a pass, holding a key block's query blocks from its first
    causally visible one on."""
    L = _lib()
    cases = [(300, 500, 0, 0, 1), (300, 500, 0, 0, 0), (256, 7, 0, 0, 1), (1000, 1000, 180, 0, 1),
             (400, 380, 0, 100, 1), (300, 600, 10000, 9800, 1), (260, 200, 5000, 0, 1), (64, 640, 0, 300, 1),
             (32768, 32768, 0, 0, 1), (16384, 16384, 16384 * 40, 16384 * 40, 1), (16384, 16384, 0, 16384, 1),
             (65536, 65536, 0, 0, 1), (1, 1, 0, 0, 1), (1, 1, 0, 63, 1), (5, 64, 64, 0, 1)]
    for Lq, Lk, qo, ko, causal in cases:
        base = L.lwm_blockattn_bwd_workspace_size(2, 3, Lq, Lk, 128)
        slot = ds_blocks_brute(Lq, Lk, qo, ko, causal) * 8192
        for heads in (1, 4, 100):
            got = L.lwm_blockattn_bwd_workspace_size_ds(2, 3, Lq, Lk, 128, qo, ko, causal, heads)
            want = base + min(heads, 6) * slot if slot else base
            assert got == want, (Lq, Lk, qo, ko, causal, heads, got, want)
    # a causal square slot keeps the blocks on and after the diagonal: 8 + 7 + ... + 1 of 8 x 8
    assert ds_blocks_brute(300, 500, 0, 0, 1) == 36 and ds_blocks_brute(300, 500, 0, 0, 0) == 64
    assert ds_blocks_brute(256, 7, 0, 0, 1) == 4  # 256 queries = 4 blocks, one key block
    assert ds_blocks_brute(16384, 16384, 0, 16384, 1) == 0  # keys all after the queries
    for args in ((2, 3, 300, 500, 128, 0, 0, 1, 0), (2, 3, 300, 500, 128, 0, 0, 1, -5),
                 (2, 3, 300, 0, 128, 0, 0, 1, 4), (1, 1, (1 << 21) + 1, 64, 128, 0, 0, 1, 1),
                 (1, 1, 64, 64, 128, -1, 0, 1, 1), (1, 1, 64, 64, 128, 0, (1 << 40) + 1, 1, 1),
                 (1, 1, 16384, 16384, 128, 0, 16384, 1, 1)):
        assert L.lwm_blockattn_bwd_workspace_size_ds(*args) == L.lwm_blockattn_bwd_workspace_size(*args[:5]), args
    assert L.lwm_blockattn_bwd_workspace_size_ds(0, 3, 300, 500, 128, 0, 0, 1, 4) == 256
    assert L.lwm_blockattn_bwd_workspace_size_ds(64, 64, 1 << 21, 1 << 31, 128, 0, 0, 0, 4096) == 2**64 - 1


def test_default_stored_ds_heads():
    """The binding's choice of pairs per pass for the workspaces it allocates (up to 80 GiB of dS)."""
    assert lwm.DS_BUDGET_BYTES == 80 << 30
    assert lwm.default_ds_heads(1, 32, 32768, 32768, 128) == 32  # causal slots of about 1 GiB
    assert lwm.default_ds_heads(1, 32, 32768, 32768, 128, causal=False) == 32  # 2 GiB each
    assert lwm.default_ds_heads(1, 32, 65536, 65536, 128) == 16  # 4.3 GB slots: 19, then a multiple of 8
    assert lwm.default_ds_heads(1, 32, 65536, 65536, 128, causal=False) == 0  # 8 GiB slots: 8, under 16
    assert lwm.default_ds_heads(1, 4, 1 << 20, 1 << 20, 128) == 0  # not one slot fits
    slot = lwm.lwm_blockattn_bwd_workspace_size_ds(1, 1, 4096, 4096, 128, 1) - \
        lwm.lwm_blockattn_bwd_workspace_size(1, 1, 4096, 4096, 128)
    assert slot == 64 * 65 // 2 * 8192
    assert lwm.default_ds_heads(1, 12, 4096, 4096, 128, budget=12 * slot) == 12
    assert lwm.default_ds_heads(1, 12, 4096, 4096, 128, budget=11 * slot) == 0
    assert lwm.default_ds_heads(1, 40, 4096, 4096, 128, budget=39 * slot) == 32
    assert lwm.default_ds_heads(1, 4, 4096, 4096, 128, budget=4 * slot) == 4
    assert lwm.default_ds_heads(1, 4, 4096, 4096, 128, budget=3 * slot) == 0
    assert lwm.default_ds_heads(2, 8, 4096, 4096, 128, budget=16 * slot) == 16
