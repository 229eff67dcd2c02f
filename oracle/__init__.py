"""Oracle: plain scalar CPU reference for Transformer-XL relative attention.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
benchmark's CPU-baseline leg are the only users.  The HIP library never
imports, links or calls anything here, and nothing here imports the HIP
library.  The arithmetic lives in ``txl_oracle.c`` (IEEE double, one scalar
at a time); this module marshals numpy arrays into it and adds the
multi-segment driver, which is a plain loop over the C functions.

Sources (web pages, cited by title and section / class):
  [SRC] "Transformer-XL模型 核心源码阅读笔记" (source-reading notes,
        blog.csdn.net/ACM_hades/article/details/104742528)
  [XL]  "Transformer-XL" (textbook notes, zty624.github.io, DL notebooks,
        ch4_transformer/xl)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "txl_oracle.c")
_LIB = os.path.join(_HERE, "libtxl_oracle.so")
_lock = threading.Lock()
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_U8 = ctypes.POINTER(ctypes.c_ubyte)
_VP = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (portable -O2, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-Wall", "-Wextra", "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_native = None


def _load_native():
    """The same C source built with -O2 -march=native (no fast-math, no FP
    contraction) for this host, used only to time the oracle as a CPU
    baseline.  Built per host into the temporary directory (the code is
    specific to the CPU it was built on), once per process."""
    global _native
    with _lock:
        if _native is not None:
            return _native
        import hashlib
        import tempfile
        model = ""
        try:
            model = next((l for l in open("/proc/cpuinfo") if l.startswith("model name")), "")
        except OSError:
            pass
        tag = hashlib.sha256((model + open(_SRC).read()).encode()).hexdigest()[:16]
        path = os.path.join(tempfile.gettempdir(), f"txl_oracle_native_{tag}_{os.getpid()}.so")
        cmd = ["gcc", "-O2", "-march=native", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-Wall", "-Wextra", "-Wno-unused-parameter", _SRC, "-o", path, "-lm"]
        subprocess.run(cmd, check=True)
        lib = ctypes.CDLL(path)
        lib.txo_relattn_fwd_range.argtypes = [_I, _I, _I, _I, _I, ctypes.c_double, _I,
                                              _D, _D, _D, _D, _D, _D, _D, _D, _I, _I]
        lib.txo_relattn_fwd_range.restype = _I
        os.unlink(path)   # the mapping stays valid
        _native = lib
        return lib


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.txo_visible_mask.argtypes = [_I, _I, _U8]
        lib.txo_visible_mask_same_length.argtypes = [_I, _I, _I, _U8]
        lib.txo_rel_shift.argtypes = [_I, _I, _D, _D]
        lib.txo_relattn_scores.argtypes = [_I, _I, _I, ctypes.c_double, _I, _D, _D, _D, _D, _D, _D]
        lib.txo_relattn_fwd_range.argtypes = [_I, _I, _I, _I, _I, ctypes.c_double, _I,
                                              _D, _D, _D, _D, _D, _D, _D, _D, _I, _I]
        lib.txo_relattn_row.argtypes = [_I, _I, _I, _I, ctypes.c_double, _I, _I, _I,
                                        _D, _D, _D, _D, _D, _D, _D, _D]
        lib.txo_relattn_fwd_vis_range.argtypes = [_I, _I, _I, _I, _I, ctypes.c_double, _I,
                                                  ctypes.POINTER(_I)] + [_D] * 8 + [_I, _I]
        lib.txo_relattn_row_vis.argtypes = [_I, _I, _I, _I, ctypes.c_double, _I, _I, _I, _I, _I] + [_D] * 8
        lib.txo_relattn_bwd_range.argtypes = [_I, _I, _I, _I, _I, ctypes.c_double, _I,
                                              ctypes.POINTER(_I)] + [_D] * 13 + [_I, _I]
        lib.txo_mem_update.argtypes = [_VP, _I, _VP, _I, _VP, _I, _I, _I, _I, _I, _I64, _I64, _I64]
        lib.txo_pos_emb.argtypes = [_I, _I, _I, _D]
        lib.txo_linear.argtypes = [_I, _I, _I, _D, _D, _D, _D]
        lib.txo_layer_norm.argtypes = [_I, _I, _D, _D, _D, ctypes.c_double, _D]
        lib.txo_layer_fwd.argtypes = [_I] * 7 + [_D] * 15 + [ctypes.c_double, _D]
        lib.txo_layer_fwd_ex.argtypes = [_I] * 9 + [ctypes.POINTER(_I)] + [_D] * 15 + [ctypes.c_double, _D]
        for name in ("txo_visible_mask", "txo_visible_mask_same_length", "txo_rel_shift",
                     "txo_relattn_scores", "txo_relattn_fwd_range", "txo_relattn_row",
                     "txo_relattn_fwd_vis_range", "txo_relattn_row_vis", "txo_relattn_bwd_range",
                     "txo_mem_update", "txo_pos_emb", "txo_linear", "txo_layer_norm", "txo_layer_fwd",
                     "txo_layer_fwd_ex"):
            getattr(lib, name).restype = _I
        _lib = lib
        return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(_D)


def _check(rc: int, what: str) -> int:
    if rc < 0:
        raise ValueError(f"oracle {what} failed with code {rc}")
    return rc


def visible_mask(L: int, M: int) -> np.ndarray:
    """[L, M+L] bool, True = visible ([SRC] MemTransformerLM._forward mask)."""
    out = np.zeros((L, M + L), dtype=np.uint8)
    _check(_load().txo_visible_mask(L, M, out.ctypes.data_as(_U8)), "visible_mask")
    return out.astype(bool)


def visible_mask_same_length(L: int, M_cur: int, mem_len: int) -> np.ndarray:
    """[L, M_cur+L] bool for the same_length option of [SRC] _forward."""
    out = np.zeros((L, M_cur + L), dtype=np.uint8)
    _check(_load().txo_visible_mask_same_length(L, M_cur, mem_len, out.ctypes.data_as(_U8)),
           "visible_mask_same_length")
    return out.astype(bool)


def rel_shift(x) -> np.ndarray:
    """The literal pad / reshape / slice of [SRC] RelMultiHeadAttn._rel_shift on [L, K]."""
    x = _f64(x)
    L, K = x.shape
    y = np.empty_like(x)
    _check(_load().txo_rel_shift(L, K, _p(x), _p(y)), "rel_shift")
    return y


def relattn_scores(q, k, r, u, vb, M: int, scale: float | None = None, literal: bool = False) -> np.ndarray:
    """Scores of one head: q [L, dh], k, r [M+L, dh], u, vb [dh] -> [L, M+L], -inf where masked."""
    q, k, r, u, vb = map(_f64, (q, k, r, u, vb))
    L, dh = q.shape
    K = M + L
    assert k.shape == (K, dh) and r.shape == (K, dh) and u.shape == (dh,) and vb.shape == (dh,)
    S = np.empty((L, K), dtype=np.float64)
    _check(_load().txo_relattn_scores(L, M, dh, 0.0 if scale is None else scale, int(literal),
                                      _p(q), _p(k), _p(r), _p(u), _p(vb), _p(S)), "relattn_scores")
    return S


def relattn_fwd(q, k, v, r, u, vb, scale: float | None = None, literal: bool = False,
                threads: int = 1, bh_range: tuple[int, int] | None = None,
                same_length: int = 0, mem_valid=None, native: bool = False):
    """Relative attention over all heads.

    q [B, H, L, dh]; k, v [B, H, M+L, dh]; r [H, M+L, dh]; u, vb [H, dh].
    Returns (out [B, H, L, dh], lse [B, H, L]) in float64.  ``threads`` > 1
    splits the independent (b, h) heads across Python threads (the C call
    releases the GIL); ``bh_range`` restricts the work to a slice of the
    flattened (b, h) index (the other rows of the result stay zero).
    ``same_length`` > 0 applies the same_length mask of [SRC]
    MemTransformerLM._forward with that mem_len; ``mem_valid`` ([B] ints in
    [0, M]) hides the oldest M - mem_valid[b] memory rows of batch row b
    (per-row memory reset).  Both use the direct score form.  ``native`` runs
    the same code built for this host's CPU (-march=native; timing only).
    """
    q, k, v, r, u, vb = map(_f64, (q, k, v, r, u, vb))
    B, H, L, dh = q.shape
    K = k.shape[2]
    M = K - L
    assert M >= 0 and k.shape == (B, H, K, dh) and v.shape == (B, H, K, dh)
    assert r.shape == (H, K, dh) and u.shape == (H, dh) and vb.shape == (H, dh)
    out = np.zeros((B, H, L, dh), dtype=np.float64)
    lse = np.zeros((B, H, L), dtype=np.float64)
    variant = same_length > 0 or mem_valid is not None
    assert not (native and (variant or literal)), "the native build serves the direct, unmasked form"
    lib = _load_native() if native else _load()
    lo, hi = (0, B * H) if bh_range is None else bh_range
    sc = 0.0 if scale is None else float(scale)
    args = (_p(q), _p(k), _p(v), _p(r), _p(u), _p(vb), _p(out), _p(lse))
    assert not (variant and literal), "the mask variants use the direct form"
    mv = None
    if mem_valid is not None:
        mv = np.ascontiguousarray(np.asarray(mem_valid, dtype=np.int32))
        assert mv.shape == (B,)

    def run(a, b):
        if variant:
            mvp = mv.ctypes.data_as(ctypes.POINTER(_I)) if mv is not None else None
            _check(lib.txo_relattn_fwd_vis_range(B, H, L, M, dh, sc, int(same_length), mvp, *args, a, b),
                   "relattn_fwd_vis")
        else:
            _check(lib.txo_relattn_fwd_range(B, H, L, M, dh, sc, int(literal), *args, a, b), "relattn_fwd")

    if threads <= 1 or hi - lo <= 1:
        run(lo, hi)
    else:
        n = min(threads, hi - lo)
        cuts = [lo + (hi - lo) * t // n for t in range(n + 1)]
        ts = [threading.Thread(target=run, args=(cuts[t], cuts[t + 1])) for t in range(n)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
    return out, lse


def relattn_bwd(q, k, v, r, u, vb, dout, scale: float | None = None, threads: int = 1,
                bh_range: tuple[int, int] | None = None, same_length: int = 0, mem_valid=None):
    """Gradients of relattn_fwd's output (see txo_relattn_bwd_range).

    Shapes as relattn_fwd; dout [B, H, L, dh] is the upstream gradient of out.
    Returns a dict of float64 arrays: dq [B, H, L, dh], dk, dv [B, H, K, dh],
    dr [H, K, dh], du, dvb [H, dh].  dr, du and dvb are the sums over the
    batch rows (in b order) of the per-head contributions.  ``bh_range``
    restricts the work to a slice of the flattened (b, h) index: heads outside
    it contribute nothing (their dq, dk, dv stay zero).
    """
    q, k, v, r, u, vb, dout = map(_f64, (q, k, v, r, u, vb, dout))
    B, H, L, dh = q.shape
    K = k.shape[2]
    M = K - L
    assert M >= 0 and k.shape == (B, H, K, dh) and v.shape == (B, H, K, dh) and dout.shape == q.shape
    assert r.shape == (H, K, dh) and u.shape == (H, dh) and vb.shape == (H, dh)
    dq = np.zeros((B, H, L, dh))
    dk = np.zeros((B, H, K, dh))
    dv = np.zeros((B, H, K, dh))
    dr_bh = np.zeros((B, H, K, dh))
    du_bh = np.zeros((B, H, dh))
    dvb_bh = np.zeros((B, H, dh))
    lo, hi = (0, B * H) if bh_range is None else bh_range
    sc = 0.0 if scale is None else float(scale)
    mv = None
    if mem_valid is not None:
        mv = np.ascontiguousarray(np.asarray(mem_valid, dtype=np.int32))
        assert mv.shape == (B,)
    mvp = mv.ctypes.data_as(ctypes.POINTER(_I)) if mv is not None else None
    lib = _load()

    def run(a, b):
        _check(lib.txo_relattn_bwd_range(B, H, L, M, dh, sc, int(same_length), mvp, _p(q), _p(k), _p(v), _p(r),
                                         _p(u), _p(vb), _p(dout), _p(dq), _p(dk), _p(dv), _p(dr_bh), _p(du_bh),
                                         _p(dvb_bh), a, b), "relattn_bwd")

    if threads <= 1 or hi - lo <= 1:
        run(lo, hi)
    else:
        n = min(threads, hi - lo)
        cuts = [lo + (hi - lo) * t // n for t in range(n + 1)]
        ts = [threading.Thread(target=run, args=(cuts[t], cuts[t + 1])) for t in range(n)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
    dr, du, dvb = np.zeros((H, K, dh)), np.zeros((H, dh)), np.zeros((H, dh))
    for b in range(B):
        dr += dr_bh[b]
        du += du_bh[b]
        dvb += dvb_bh[b]
    return {"dq": dq, "dk": dk, "dv": dv, "dr": dr, "du": du, "dvb": dvb}


def relattn_row(q, k, v, r, u, vb, b: int, h: int, i: int, scale: float | None = None,
                same_length: int = 0, mem_valid: int | None = None):
    """Output row out[b, h, i, :] and lse[b, h, i], computed alone (for sampled checks).
    ``same_length`` and ``mem_valid`` (this row's valid memory count) as in relattn_fwd."""
    q, k, v, r, u, vb = map(_f64, (q, k, v, r, u, vb))
    B, H, L, dh = q.shape
    M = k.shape[2] - L
    row = np.empty(dh, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    sc = 0.0 if scale is None else scale
    if same_length > 0 or mem_valid is not None:
        mvb = M if mem_valid is None else int(mem_valid)
        _check(_load().txo_relattn_row_vis(H, L, M, dh, sc, int(same_length), mvb, b, h, i,
                                           _p(q), _p(k), _p(v), _p(r), _p(u), _p(vb), _p(row), _p(lse)),
               "relattn_row_vis")
    else:
        _check(_load().txo_relattn_row(H, L, M, dh, sc, b, h, i,
                                       _p(q), _p(k), _p(v), _p(r), _p(u), _p(vb), _p(row), _p(lse)),
               "relattn_row")
    return row, float(lse[0])


def mem_update(mem: np.ndarray | None, h: np.ndarray, mem_len: int, ext_len: int = 0) -> np.ndarray:
    """[SRC] _update_mems on raw bytes: mem [B, M_cur, d] (or None), h [B, L, d] -> [B, M_new, d]."""
    h = np.ascontiguousarray(h)
    B, L, d = h.shape
    if mem is None:
        mem = np.zeros((B, 0, d), dtype=h.dtype)
    mem = np.ascontiguousarray(mem)
    assert mem.dtype == h.dtype and mem.shape[0] == B and mem.shape[2] == d
    M_cur = mem.shape[1]
    end = M_cur + max(0, L - ext_len)
    M_new = end - max(0, end - mem_len)
    new = np.zeros((B, M_new, d), dtype=h.dtype)
    es = h.dtype.itemsize
    rc = _load().txo_mem_update(mem.ctypes.data, M_cur, h.ctypes.data, L, new.ctypes.data, mem_len, ext_len,
                                B, d, es, M_cur * d, L * d, M_new * d)
    assert _check(rc, "mem_update") == M_new
    return new


def pos_emb(K: int, demb: int, clamp_len: int = 0) -> np.ndarray:
    """[SRC] PositionalEmbedding at positions K-1 .. 0 -> [K, demb]."""
    out = np.empty((K, demb), dtype=np.float64)
    _check(_load().txo_pos_emb(K, demb, clamp_len, _p(out)), "pos_emb")
    return out


def linear(x, W, bias=None) -> np.ndarray:
    x, W = _f64(x), _f64(W)
    N, i = x.shape
    o = W.shape[0]
    y = np.empty((N, o), dtype=np.float64)
    b = None if bias is None else _f64(bias)
    _check(_load().txo_linear(N, i, o, _p(x), _p(W), _p(b), _p(y)), "linear")
    return y


def layer_norm(x, g, b, eps: float = 1e-5) -> np.ndarray:
    x, g, b = _f64(x), _f64(g), _f64(b)
    N, d = x.shape
    y = np.empty_like(x)
    _check(_load().txo_layer_norm(N, d, _p(x), _p(g), _p(b), eps, _p(y)), "layer_norm")
    return y


LAYER_KEYS = ("W_qkv", "W_r", "W_o", "ln1_g", "ln1_b", "W1", "b1", "W2", "b2", "ln2_g", "ln2_b")


def layer_fwd(h_in, mem, w: dict, u, vb, n_head: int, d_head: int, eps: float = 1e-5, clamp_len: int = 0,
              same_length: int = 0, mem_valid=None) -> np.ndarray:
    """One post-LN decoder layer (see txo_layer_fwd_ex).  h_in [B, L, d]; mem [B, M_cur, d] or None.
    clamp_len / same_length as in [SRC] MemTransformerLM (0 = off); mem_valid [B] ints in
    [0, M_cur] keeps only the newest mem_valid[b] memory rows of row b."""
    h_in = _f64(h_in)
    B, L, d = h_in.shape
    M_cur = 0 if mem is None else mem.shape[1]
    memd = None if (mem is None or M_cur == 0) else _f64(mem)
    ws = [_f64(w[key]) for key in LAYER_KEYS]
    d_inner = ws[5].shape[0]
    out = np.empty_like(h_in)
    mv = None
    if mem_valid is not None:
        mv = np.ascontiguousarray(np.asarray(mem_valid, dtype=np.int32))
        assert mv.shape == (B,)
    mvp = mv.ctypes.data_as(ctypes.POINTER(_I)) if mv is not None else None
    _check(_load().txo_layer_fwd_ex(B, L, M_cur, d, n_head, d_head, d_inner, int(clamp_len), int(same_length), mvp,
                                    _p(h_in), _p(memd), *[_p(a) for a in ws], _p(_f64(u)), _p(_f64(vb)), eps,
                                    _p(out)),
           "layer_fwd")
    return out


def stack_segment(x, mems, layers: list[dict], u, vb, n_head: int, d_head: int, mem_len: int,
                  eps: float = 1e-5):
    """One segment through the layer stack, as [SRC] MemTransformerLM._forward.

    x [B, L, d] (the embedded segment); mems: list of len(layers)+1 arrays
    [B, M_cur, d] (M_cur may be 0).  hids[0] = x, hids[n+1] = layer_n(hids[n],
    mems[n]); then every mems[n] <- Tail of [mems[n]; hids[n]] ([SRC]
    _update_mems with ext_len = 0).  Returns (hids[-1], new_mems).
    """
    hids = [_f64(x)]
    for n, w in enumerate(layers):
        hids.append(layer_fwd(hids[n], mems[n], w, u, vb, n_head, d_head, eps))
    new_mems = [mem_update(_f64(m), hh, mem_len) for m, hh in zip(mems, hids)]
    return hids[-1], new_mems
