"""Host-side checks of libtxl.so that need no GPU: it loads, exports every
function include/txl.h declares, and rejects bad arguments before launching
anything (only failing calls are made here, so nothing reaches the device)."""
import ctypes
import os
import re

import pytest

import transformer_xl_relative_rel_amd as txl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "txl.h")

OK, EINVAL, EUNSUP, EALIAS, EWS = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(txl_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = txl.lib()
    names = declared_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(txl.EXPORTED)


def test_version_and_status_strings():
    lib = txl.lib()
    assert lib.txl_version().decode().count(".") == 2
    for s in range(6):
        assert lib.txl_status_string(s).decode()


def _desc(B=2, H=2, L=8, M=4, dh=64, dtype=txl.BF16):
    d = txl.RelAttnDesc()
    assert txl.lib().txl_relattn_desc_init(ctypes.byref(d), B, H, L, M, dh, dtype) == OK
    return d


def test_desc_init_packs_dense_strides():
    d = _desc(B=3, H=5, L=7, M=9, dh=32)
    K = 16
    assert list(d.q_stride) == [5 * 7 * 32, 7 * 32, 32]
    assert list(d.k_stride) == [5 * K * 32, K * 32, 32]
    assert list(d.r_stride) == [K * 32, 32]
    assert abs(d.scale - 32 ** -0.5) < 1e-7


FAKE = 1 << 30  # 16-byte aligned addresses, 1 GiB apart, never dereferenced


def _fwd(d, q=FAKE, k=FAKE * 2, v=FAKE * 3, r=FAKE * 4, u=FAKE * 5, vb=FAKE * 6, out=FAKE * 7, lse=0, ws=0,
         ws_bytes=0):
    vp = ctypes.c_void_p
    return txl.lib().txl_relattn_fwd(ctypes.byref(d) if d is not None else None, vp(q), vp(k), vp(v), vp(r), vp(u),
                                     vp(vb), vp(out), vp(lse), vp(ws), ws_bytes, vp(0))


def test_relattn_rejects_bad_arguments():
    lib = txl.lib()
    assert _fwd(None) == EINVAL
    for field, val in (("L", 0), ("B", 0), ("M", -1), ("dtype", 7)):
        d = _desc()
        setattr(d, field, val)
        assert _fwd(d) == EINVAL, field
    assert _fwd(_desc(dh=48)) == EUNSUP
    assert _fwd(_desc(dh=16, dtype=txl.BF16)) == EUNSUP
    assert _fwd(_desc(dh=128, dtype=txl.F32)) == EUNSUP
    assert b"dh" in lib.txl_last_error()
    assert _fwd(_desc(), q=0) == EINVAL
    assert _fwd(_desc(), k=FAKE * 2 + 8) == EINVAL          # misaligned base
    d = _desc()
    d.q_stride[2] = 65                                       # row breaks 16-byte alignment
    assert _fwd(d) == EINVAL
    d = _desc()
    d.k_stride[2] = 32                                       # rows would overlap
    assert _fwd(d) == EINVAL


def test_relattn_rejects_aliasing():
    d = _desc(B=1, H=1, L=8, M=0, dh=64)
    assert _fwd(d, out=FAKE) == EALIAS                       # out == q
    assert _fwd(d, out=FAKE + 64) == EALIAS                  # partial overlap with q
    assert _fwd(d, lse=FAKE * 3 + 16) == EALIAS              # lse inside v


def test_split_plan_needs_workspace():
    d = _desc(B=1, H=16, L=128, M=1600, dh=64)               # long memory: split automatically
    n = ctypes.c_size_t(0)
    assert txl.lib().txl_relattn_workspace_size(ctypes.byref(d), ctypes.byref(n)) == OK
    assert n.value > 0
    assert _fwd(d) == EWS
    assert _fwd(d, ws=FAKE * 16 + 16, ws_bytes=n.value) == EWS  # misaligned
    assert _fwd(d, ws=FAKE * 16, ws_bytes=n.value - 1) == EWS
    d3 = _desc(B=8, H=16, L=512, M=512, dh=64)               # enough blocks: no split
    assert txl.lib().txl_relattn_workspace_size(ctypes.byref(d3), ctypes.byref(n)) == OK
    assert n.value == 0
    d3.splits = 4
    assert txl.lib().txl_relattn_workspace_size(ctypes.byref(d3), ctypes.byref(n)) == OK
    assert n.value >= 4 * 8 * 16 * 512 * 64 * 4


def _mem(mem=FAKE, M_cur=8, h=FAKE * 2, L=8, new=FAKE * 3, mem_len=8, ext=0, B=2, d=32, dtype=txl.BF16,
         mem_bs=None, h_bs=None, new_bs=None):
    vp = ctypes.c_void_p
    mem_bs = M_cur * d if mem_bs is None else mem_bs
    h_bs = L * d if h_bs is None else h_bs
    new_bs = mem_len * d if new_bs is None else new_bs
    got = ctypes.c_int(-1)
    s = txl.lib().txl_mem_update(vp(mem), M_cur, vp(h), L, vp(new), mem_len, ext, B, d, dtype, mem_bs, h_bs, new_bs,
                                 ctypes.byref(got), vp(0))
    return s


def test_mem_update_rejects_bad_arguments():
    assert _mem(mem=0) == EINVAL                 # M_cur > 0 needs mem
    assert _mem(d=4) == EINVAL                   # 8-byte rows
    assert _mem(B=0) == EINVAL
    assert _mem(mem_len=-1) == EINVAL
    assert _mem(h=FAKE * 2 + 2) == EINVAL        # misaligned
    assert _mem(new=FAKE) == EALIAS              # in place over mem
    assert _mem(new=FAKE * 2 + 64) == EALIAS     # overlaps h
    assert _mem(h_bs=8) == EINVAL                # batch stride smaller than a batch row
    vp = ctypes.c_void_p
    arr = (vp * 1)(vp(FAKE))
    got = ctypes.c_int()
    assert txl.lib().txl_mem_update_batched(0, arr, 1, arr, 1, arr, 1, 0, 1, 32, txl.BF16, 32, 32, 32,
                                            ctypes.byref(got), vp(0)) == EINVAL
    assert txl.lib().txl_mem_update_batched(65, arr, 1, arr, 1, arr, 1, 0, 1, 32, txl.BF16, 32, 32, 32,
                                            ctypes.byref(got), vp(0)) == EINVAL


def _fwd_mem(d, out=FAKE * 7, lse=0, mem=FAKE * 8, h=FAKE * 9, new=FAKE * 10, M_cur=8, L=8, mem_len=8, B=2, dm=32):
    vp = ctypes.c_void_p
    got = ctypes.c_int(-1)
    return txl.lib().txl_relattn_fwd_mem_update(
        ctypes.byref(d), vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), vp(FAKE * 4), vp(FAKE * 5), vp(FAKE * 6), vp(out),
        vp(lse), vp(0), 0, vp(mem), M_cur, vp(h), L, vp(new), mem_len, 0, B, dm, txl.BF16, M_cur * dm, L * dm,
        mem_len * dm, ctypes.byref(got), vp(0))


def test_fused_mem_update_rejects_bad_arguments():
    d = _desc(B=1, H=1, L=8, M=0, dh=64)
    assert _fwd_mem(d, out=FAKE) == EALIAS              # the attention's own checks
    assert _fwd_mem(d, mem=0) == EINVAL                 # the memory update's own checks
    assert _fwd_mem(d, new=FAKE * 8 + 16) == EALIAS     # in place over mem
    # the two run together: the copy must not write what the attention reads or writes ...
    assert _fwd_mem(d, new=FAKE * 3 + 64) == EALIAS     # new_mem inside v
    assert _fwd_mem(d, new=FAKE * 7 + 64) == EALIAS     # new_mem inside out
    assert _fwd_mem(d, new=FAKE * 5) == EALIAS          # new_mem over u
    # ... nor read what the attention writes
    assert _fwd_mem(d, h=FAKE * 7 + 32) == EALIAS       # h inside out
    assert _fwd_mem(d, lse=FAKE * 8 + 64) == EALIAS     # lse inside mem
    assert b"overlaps" in txl.lib().txl_last_error()


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(txl, "_lib", None)
    monkeypatch.setattr(txl, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        txl.lib()


def _bwd(d, ws=FAKE * 20, ws_bytes=1 << 40, **kw):
    vp = ctypes.c_void_p
    ptr = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, r=FAKE * 4, u=FAKE * 5, vb=FAKE * 6, out=FAKE * 7, lse=FAKE * 8,
               dout=FAKE * 9, dq=FAKE * 10, dk=FAKE * 11, dv=FAKE * 12, dr=FAKE * 13, du=FAKE * 14, dvb=FAKE * 15)
    ptr.update(kw)
    order = ("q", "k", "v", "r", "u", "vb", "out", "lse", "dout", "dq", "dk", "dv", "dr", "du", "dvb")
    return txl.lib().txl_relattn_bwd(ctypes.byref(d) if d is not None else None, *[vp(ptr[x]) for x in order],
                                     vp(ws), ctypes.c_size_t(ws_bytes), vp(0))


def test_relattn_bwd_rejects_bad_arguments():
    """Every check of txl_relattn_bwd runs on the host and fails before any launch."""
    lib = txl.lib()
    assert _bwd(None) == EINVAL
    assert _bwd(_desc(dh=32)) == EUNSUP                       # the backward is bf16 with dh = 64 only
    assert _bwd(_desc(dh=64, dtype=txl.F32)) == EUNSUP
    assert b"dh = 64" in lib.txl_last_error()
    for name in ("q", "lse", "dout", "dq", "dr", "du", "dvb"):
        assert _bwd(_desc(), **{name: 0}) == EINVAL, name
    assert _bwd(_desc(), dq=FAKE * 10 + 8) == EINVAL           # misaligned output
    assert _bwd(_desc(), ws=0) == EWS
    assert _bwd(_desc(), ws_bytes=16) == EWS
    assert _bwd(_desc(), ws=FAKE * 20 + 64) == EWS            # workspace must be 256-byte aligned
    assert _bwd(_desc(), dq=FAKE) == EALIAS                    # dq on top of q
    assert _bwd(_desc(), dk=FAKE * 10) == EALIAS               # two outputs overlap
    n = ctypes.c_size_t(0)
    assert lib.txl_relattn_bwd_workspace_size(ctypes.byref(_desc()), ctypes.byref(n)) == OK and n.value > 0
    assert lib.txl_relattn_bwd_workspace_size(ctypes.byref(_desc(dh=128)), ctypes.byref(n)) == EUNSUP


def test_fused_mem_update_writes_no_length_on_failure():
    """A failing call writes nothing, M_new included, also when the failure is
    found by the fused path's own checks (a 2 GiB memory row)."""
    vp = ctypes.c_void_p
    d = _desc(B=1, H=1, L=160, M=0, dh=64)        # bf16 throughput kernel: the copy rides on it
    d.splits = 1
    dm = 1 << 30                                   # one bf16 row of 2 GiB
    got = ctypes.c_int(-1)
    s = txl.lib().txl_relattn_fwd_mem_update(
        ctypes.byref(d), vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), vp(FAKE * 4), vp(FAKE * 5), vp(FAKE * 6),
        vp(FAKE * 7), vp(0), vp(0), 0, vp(0), 0, vp(FAKE * 9), 1, vp(FAKE * 12), 1, 0, 1, dm, txl.BF16, 0, dm, dm,
        ctypes.byref(got), vp(0))
    assert s == EUNSUP
    assert got.value == -1
    got.value = -1
    assert _fwd_mem(_desc(B=1, H=1, L=8, M=0, dh=64), out=FAKE) == EALIAS and got.value == -1


def test_fused_mem_update_rejects_new_mem_over_mem_valid():
    d = _desc(B=2, H=1, L=8, M=0, dh=64)
    d.mem_valid = FAKE * 10 + 4                      # the kernel reads it while the copy writes new_mem
    assert _fwd_mem(d) == EALIAS
    d.mem_valid = FAKE * 7 + 4                       # and the attention's out must not cover it either
    assert _fwd(d) == EALIAS


def test_mem_update_len():
    lib = txl.lib()
    n = ctypes.c_int(-1)
    # end = M_cur + max(0, L - ext_len), beg = max(0, end - mem_len), M_new = end - beg
    for M_cur, L, mem_len, ext, want in ((0, 8, 8, 0, 8), (8, 8, 8, 0, 8), (3, 4, 16, 0, 7), (5, 10, 4, 3, 4),
                                         (5, 2, 16, 3, 5), (0, 0, 5, 0, 0), (7, 9, 0, 0, 0)):
        assert lib.txl_mem_update_len(M_cur, L, mem_len, ext, ctypes.byref(n)) == OK
        assert n.value == want, (M_cur, L, mem_len, ext)
    assert lib.txl_mem_update_len(-1, 1, 1, 0, ctypes.byref(n)) == EINVAL
    assert lib.txl_mem_update_len(1, 1, 1, 0, None) == EINVAL


def test_layer_fwd_needs_a_context():
    vp = ctypes.c_void_p
    ld = txl.LayerDesc(1, 8, 64, 1, 64, 128, 1e-5, 0, 0, None)
    lw = txl.LayerWeights(*[FAKE * (i + 1) for i in range(len(txl.LAYER_KEYS))])
    s = txl.lib().txl_layer_fwd(vp(0), ctypes.byref(ld), ctypes.byref(lw), vp(FAKE * 20), vp(0), 0, vp(FAKE * 21),
                                vp(FAKE * 22), vp(FAKE * 23), vp(FAKE * 24), ctypes.c_size_t(1 << 40), vp(0))
    assert s == EINVAL
    assert b"ctx" in txl.lib().txl_last_error()
    assert txl.lib().txl_context_destroy(vp(0)) == OK
