"""MI355X-native Transformer-XL segment-recurrent relative attention.

A thin binding over the C ABI of ``libtxl.so`` (declared in include/txl.h).
It only marshals arguments: torch supplies device memory and the current
stream, every step of the computation runs in the library's HIP kernels.
If the library is not built, every call raises; there is no fallback.
"""
from __future__ import annotations

import atexit
import ctypes
import os

__all__ = [
    "TxlError", "lib", "lib_path", "relattn_fwd", "relattn_fwd_noalloc", "relattn_fwd_mem_update", "relattn_workspace_size", "relattn_bwd",
    "relattn_bwd_workspace_size", "mem_update", "mem_update_batched", "stack_segment",
    "layer_fwd", "layer_workspace_size", "Context", "context", "LAYER_KEYS", "F32", "BF16", "EXPORTED",
]

F32, BF16 = 0, 1
_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libtxl.so")
_lib = None

# Every function declared in include/txl.h.
EXPORTED = ("txl_version", "txl_status_string", "txl_last_error", "txl_relattn_desc_init",
            "txl_relattn_workspace_size", "txl_relattn_fwd", "txl_relattn_fwd_noalloc", "txl_relattn_fwd_mem_update",
            "txl_relattn_bwd_workspace_size", "txl_relattn_bwd",
            "txl_mem_update", "txl_mem_update_len", "txl_mem_update_batched",
            "txl_context_create", "txl_context_destroy", "txl_layer_workspace_size", "txl_layer_fwd")

# Weight names of one decoder layer, in the order of txl_layer_weights.
LAYER_KEYS = ("W_qkv", "W_r", "W_o", "ln1_g", "ln1_b", "W1", "b1", "W2", "b2", "ln2_g", "ln2_b")


class TxlError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"txl status {status}: {msg}")
        self.status = status


class RelAttnDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("L", ctypes.c_int), ("M", ctypes.c_int),
                ("dh", ctypes.c_int), ("dtype", ctypes.c_int), ("scale", ctypes.c_float), ("splits", ctypes.c_int),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3), ("v_stride", ctypes.c_int64 * 3),
                ("o_stride", ctypes.c_int64 * 3), ("r_stride", ctypes.c_int64 * 2),
                ("mem_valid", ctypes.c_void_p), ("window", ctypes.c_int)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("L", ctypes.c_int), ("d_model", ctypes.c_int), ("n_head", ctypes.c_int),
                ("d_head", ctypes.c_int), ("d_inner", ctypes.c_int), ("ln_eps", ctypes.c_float),
                ("clamp_len", ctypes.c_int), ("same_length", ctypes.c_int), ("mem_valid", ctypes.c_void_p)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in LAYER_KEYS]


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load libtxl.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(transformer_xl_relative_rel_amd/build.py)")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    dp = ctypes.POINTER(RelAttnDesc)
    L.txl_version.restype = ctypes.c_char_p
    L.txl_status_string.argtypes = [i]
    L.txl_status_string.restype = ctypes.c_char_p
    L.txl_last_error.restype = ctypes.c_char_p
    L.txl_relattn_desc_init.argtypes = [dp, i, i, i, i, i, i]
    L.txl_relattn_workspace_size.argtypes = [dp, ctypes.POINTER(sz)]
    L.txl_relattn_fwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.txl_relattn_fwd_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.txl_relattn_fwd_mem_update.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, i, vp, i, vp, i, i, i,
                                             i, i, i64, i64, i64, ctypes.POINTER(i), vp]
    L.txl_relattn_bwd_workspace_size.argtypes = [dp, ctypes.POINTER(sz)]
    L.txl_relattn_bwd.argtypes = [dp] + [vp] * 16 + [sz, vp]
    L.txl_mem_update.argtypes = [vp, i, vp, i, vp, i, i, i, i, i, i64, i64, i64, ctypes.POINTER(i), vp]
    L.txl_mem_update_batched.argtypes = [i, ctypes.POINTER(vp), i, ctypes.POINTER(vp), i, ctypes.POINTER(vp), i, i,
                                         i, i, i, i64, i64, i64, ctypes.POINTER(i), vp]
    ldp = ctypes.POINTER(LayerDesc)
    L.txl_layer_workspace_size.argtypes = [ldp, i, ctypes.POINTER(sz)]
    L.txl_layer_fwd.argtypes = [vp, ldp, ctypes.POINTER(LayerWeights), vp, vp, i, vp, vp, vp, vp, sz, vp]
    L.txl_mem_update_len.argtypes = [i, i, i, i, ctypes.POINTER(i)]
    L.txl_context_create.argtypes = [ctypes.POINTER(vp)]
    L.txl_context_destroy.argtypes = [vp]
    for name in ("txl_relattn_desc_init", "txl_relattn_workspace_size", "txl_relattn_fwd", "txl_relattn_fwd_noalloc",
                 "txl_relattn_fwd_mem_update",
                 "txl_relattn_bwd_workspace_size", "txl_relattn_bwd", "txl_mem_update", "txl_mem_update_len",
                 "txl_mem_update_batched", "txl_context_create", "txl_context_destroy", "txl_layer_workspace_size",
                 "txl_layer_fwd"):
        getattr(L, name).restype = i
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise TxlError(status, lib().txl_last_error().decode())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _desc(q, k, r_k, out, v, scale, splits) -> RelAttnDesc:
    B, H, L, dh = q.shape
    K = k.shape[2]
    d = RelAttnDesc()
    _check(lib().txl_relattn_desc_init(ctypes.byref(d), B, H, L, K - L, dh, _dtype_code(q)))
    d.scale = 0.0 if scale is None else float(scale)
    d.splits = int(splits)
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", out)):
        if t.stride(-1) != 1:
            raise ValueError(f"{name[0]}: the last axis must be contiguous")
        getattr(d, name)[:] = list(t.stride()[:3])
    if r_k.stride(-1) != 1:
        raise ValueError("r_k: the last axis must be contiguous")
    d.r_stride[:] = list(r_k.stride()[:2])
    return d


def relattn_workspace_size(q, k, splits: int = 0) -> int:
    """Workspace bytes txl_relattn_fwd needs for these shapes."""
    import torch
    B, H, L, dh = q.shape
    d = RelAttnDesc()
    _check(lib().txl_relattn_desc_init(ctypes.byref(d), B, H, L, k.shape[2] - L, dh, _dtype_code(q)))
    d.splits = int(splits)
    n = ctypes.c_size_t(0)
    _check(lib().txl_relattn_workspace_size(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def relattn_fwd(q, k, v, r_k, u, vb, *, scale: float | None = None, out=None, lse=None, want_lse: bool = False,
                splits: int = 0, workspace=None, stream=None, window: int = 0, mem_valid=None):
    """Relative attention forward (txl_relattn_fwd).

    q [B, H, L, dh]; k, v [B, H, M+L, dh]; r_k [H, M+L, dh] (row c = relative
    position M+L-1-c); u, vb [H, dh] float32.  bf16 or float32 tensors on one
    device; strided views are accepted when the last axis is contiguous.
    ``window`` > 0 limits query i to keys j >= i + M + 1 - window (same_length);
    ``mem_valid`` (int32 [B] on the device) keeps only the newest mem_valid[b]
    memory rows of batch row b.
    Returns out (and lse [B, H, L] float32 when ``want_lse`` or ``lse`` is given).
    """
    d, out, lse, workspace, ws_bytes = _fwd_args(q, k, v, r_k, u, vb, scale, out, lse, want_lse, splits, workspace,
                                                 window, mem_valid)
    _check(lib().txl_relattn_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(r_k), _ptr(u), _ptr(vb), _ptr(out),
                                 _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))
    return (out, lse) if lse is not None else out


def relattn_fwd_noalloc(q, k, v, r_k, u, vb, out, lse=None, *, scale: float | None = None, splits: int = 0,
                        stream=None, window: int = 0, mem_valid=None):
    """relattn_fwd through txl_relattn_fwd_noalloc: no device allocation in the
    library or here (out, and lse if wanted, are the caller's); a key-split
    workspace comes from the library's static scratch."""
    import torch
    for t in (u, vb) + ((lse,) if lse is not None else ()):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("u, vb and lse must be contiguous float32")
    d = _desc(q, k, r_k, out, v, scale, splits)
    d.window = int(window)
    if mem_valid is not None:
        if mem_valid.dtype != torch.int32 or not mem_valid.is_contiguous() or mem_valid.numel() != q.shape[0]:
            raise ValueError("mem_valid must be a contiguous int32 tensor of B entries")
        d.mem_valid = mem_valid.data_ptr()
    _check(lib().txl_relattn_fwd_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(r_k), _ptr(u), _ptr(vb),
                                         _ptr(out), _ptr(lse), _stream(stream)))
    return (out, lse) if lse is not None else out


def _fwd_args(q, k, v, r_k, u, vb, scale, out, lse, want_lse, splits, workspace, window, mem_valid):
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    for t in (u, vb) + ((lse,) if lse is not None else ()):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("u, vb and lse must be contiguous float32")
    d = _desc(q, k, r_k, out, v, scale, splits)
    d.window = int(window)
    if mem_valid is not None:
        if mem_valid.dtype != torch.int32 or not mem_valid.is_contiguous() or mem_valid.numel() != q.shape[0]:
            raise ValueError("mem_valid must be a contiguous int32 tensor of B entries")
        d.mem_valid = mem_valid.data_ptr()
    need = ctypes.c_size_t(0)
    _check(lib().txl_relattn_workspace_size(ctypes.byref(d), ctypes.byref(need)))
    if need.value and workspace is None:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return d, out, lse, workspace, ws_bytes


def relattn_fwd_mem_update(q, k, v, r_k, u, vb, mem, h, mem_len: int, ext_len: int = 0, *, new_mem=None,
                           scale: float | None = None, out=None, lse=None, want_lse: bool = False, splits: int = 0,
                           workspace=None, stream=None, window: int = 0, mem_valid=None):
    """relattn_fwd and mem_update(mem, h, mem_len, ext_len) in one call (txl_relattn_fwd_mem_update).

    Arguments as for those two; returns (out, new_mem) or (out, lse, new_mem).
    """
    import torch
    d, out, lse, workspace, ws_bytes = _fwd_args(q, k, v, r_k, u, vb, scale, out, lse, want_lse, splits, workspace,
                                                 window, mem_valid)
    B, L, dm = h.shape
    M_cur = 0 if mem is None else mem.shape[1]
    M_new = _new_len(M_cur, L, mem_len, ext_len)
    if new_mem is None:
        new_mem = torch.empty((B, M_new, dm), dtype=h.dtype, device=h.device)
    for t in (mem, h, new_mem):
        if t is not None and t.numel() and (t.stride(-1) != 1 or t.stride(-2) != dm):
            raise ValueError("rows must be contiguous")
    got = ctypes.c_int(-1)
    _check(lib().txl_relattn_fwd_mem_update(
        ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(r_k), _ptr(u), _ptr(vb), _ptr(out), _ptr(lse),
        _ptr(workspace), ws_bytes, _ptr(mem if M_cur else None), M_cur, _ptr(h), L, _ptr(new_mem), mem_len, ext_len,
        B, dm, _dtype_code(h), mem.stride(0) if M_cur else 0, h.stride(0), new_mem.stride(0), ctypes.byref(got),
        _stream(stream)))
    assert got.value == M_new
    return (out, lse, new_mem) if lse is not None else (out, new_mem)


def _bwd_desc(q, k, v, r_k, out, dout, scale, window, mem_valid) -> RelAttnDesc:
    import torch
    if dout.stride() != out.stride() or dout.shape != out.shape:
        raise ValueError("dout must have the shape and strides of out")
    d = _desc(q, k, r_k, out, v, scale, 0)
    d.window = int(window)
    if mem_valid is not None:
        if mem_valid.dtype != torch.int32 or not mem_valid.is_contiguous() or mem_valid.numel() != q.shape[0]:
            raise ValueError("mem_valid must be a contiguous int32 tensor of B entries")
        d.mem_valid = mem_valid.data_ptr()
    return d


def relattn_bwd_workspace_size(q, k, v, r_k, out, dout, window: int = 0, mem_valid=None) -> int:
    """Workspace bytes txl_relattn_bwd needs for these tensors."""
    d = _bwd_desc(q, k, v, r_k, out, dout, None, window, mem_valid)
    n = ctypes.c_size_t(0)
    _check(lib().txl_relattn_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def relattn_bwd(q, k, v, r_k, u, vb, out, lse, dout, *, scale: float | None = None, window: int = 0,
                mem_valid=None, dq=None, dk=None, dv=None, dr=None, du=None, dvb=None, workspace=None, stream=None):
    """Gradients of relattn_fwd (txl_relattn_bwd): bf16, dh = 64.

    q, k, v, r_k, u, vb, scale, window and mem_valid as given to relattn_fwd;
    out and lse [B, H, L] float32 as it returned them; dout is the upstream
    gradient of out (same shape and strides).  Returns (dq, dk, dv, dr, du,
    dvb): dq, dk, dv like q, k, v (bf16), dr [H, K, dh], du and dvb [H, dh]
    float32.  Output tensors may be passed in (dq, dk, dv with the strides of
    q, k, v; the float32 ones contiguous).
    """
    import torch
    for t in (u, vb, lse):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("u, vb and lse must be contiguous float32")
    d = _bwd_desc(q, k, v, r_k, out, dout, scale, window, mem_valid)
    H, K, dh = r_k.shape
    dev = q.device
    if dq is None:
        dq = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=dev)
    if dk is None:
        dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=dev)
    if dv is None:
        dv = torch.empty_strided(v.shape, v.stride(), dtype=v.dtype, device=dev)
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.stride() != ref.stride() or t.shape != ref.shape:
            raise ValueError(f"{name} must have the shape and strides of {name[1:]}")
    dr = torch.empty((H, K, dh), dtype=torch.float32, device=dev) if dr is None else dr
    du = torch.empty((H, dh), dtype=torch.float32, device=dev) if du is None else du
    dvb = torch.empty((H, dh), dtype=torch.float32, device=dev) if dvb is None else dvb
    for t in (dr, du, dvb):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("dr, du and dvb must be contiguous float32")
    need = ctypes.c_size_t(0)
    _check(lib().txl_relattn_bwd_workspace_size(ctypes.byref(d), ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().txl_relattn_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(r_k), _ptr(u), _ptr(vb), _ptr(out),
                                 _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dr), _ptr(du), _ptr(dvb),
                                 _ptr(workspace), ws_bytes, _stream(stream)))
    return dq, dk, dv, dr, du, dvb


def _new_len(M_cur: int, L: int, mem_len: int, ext_len: int) -> int:
    """Rows of the new memory, as the library computes them (txl_mem_update_len)."""
    n = ctypes.c_int(-1)
    _check(lib().txl_mem_update_len(M_cur, L, mem_len, ext_len, ctypes.byref(n)))
    return n.value


def mem_update(mem, h, mem_len: int, ext_len: int = 0, out=None, stream=None):
    """Tail_M memory update (txl_mem_update): mem [B, M_cur, d] or None, h [B, L, d] -> [B, M_new, d]."""
    import torch
    B, L, d = h.shape
    M_cur = 0 if mem is None else mem.shape[1]
    M_new = _new_len(M_cur, L, mem_len, ext_len)
    if out is None:
        out = torch.empty((B, M_new, d), dtype=h.dtype, device=h.device)
    for t in (mem, h, out):
        if t is not None and t.numel() and (t.stride(-1) != 1 or t.stride(-2) != d):
            raise ValueError("rows must be contiguous")
    got = ctypes.c_int(-1)
    _check(lib().txl_mem_update(_ptr(mem if M_cur else None), M_cur, _ptr(h), L, _ptr(out), mem_len, ext_len, B, d,
                                _dtype_code(h), mem.stride(0) if M_cur else 0, h.stride(0), out.stride(0),
                                ctypes.byref(got), _stream(stream)))
    assert got.value == M_new
    return out


def mem_update_batched(mems, hs, mem_len: int, ext_len: int = 0, outs=None, stream=None):
    """One launch updating every buffer (txl_mem_update_batched); all share shapes."""
    import torch
    n = len(hs)
    B, L, d = hs[0].shape
    M_cur = 0 if mems is None or mems[0] is None else mems[0].shape[1]
    M_new = _new_len(M_cur, L, mem_len, ext_len)
    if outs is None:
        outs = [torch.empty((B, M_new, d), dtype=hs[0].dtype, device=hs[0].device) for _ in range(n)]
    arr = ctypes.c_void_p * n
    mp = arr(*[(m.data_ptr() if M_cur else 0) for m in (mems if M_cur else [None] * n)]) if M_cur else arr()
    hp = arr(*[t.data_ptr() for t in hs])
    op = arr(*[t.data_ptr() for t in outs])
    got = ctypes.c_int(-1)
    _check(lib().txl_mem_update_batched(n, mp, M_cur, hp, L, op, mem_len, ext_len, B, d, _dtype_code(hs[0]),
                                        mems[0].stride(0) if M_cur else 0, hs[0].stride(0),
                                        outs[0].stride(0) if M_new else 0, ctypes.byref(got), _stream(stream)))
    return outs


class Context:
    """A library context (txl_context_create) on the device current at
    creation; txl_layer_fwd needs one.  close() synchronises the device and
    destroys it; the binding's own contexts (context()) are closed at exit."""

    def __init__(self):
        h = ctypes.c_void_p(0)
        _check(lib().txl_context_create(ctypes.byref(h)))
        self._h = h

    @property
    def handle(self):
        return self._h

    def close(self):
        if self._h is not None and self._h.value:
            import torch
            torch.cuda.synchronize()
            lib().txl_context_destroy(self._h)
        self._h = None



_contexts: dict = {}


def _close_contexts():
    for c in _contexts.values():
        try:
            c.close()
        except Exception:
            pass
    _contexts.clear()


atexit.register(_close_contexts)


def context(device=None) -> Context:
    """The binding's context for `device` (default: the current device), created on first use."""
    import torch
    idx = torch.cuda.current_device() if device is None else torch.device(device).index
    if idx not in _contexts:
        with torch.cuda.device(idx):
            _contexts[idx] = Context()
    return _contexts[idx]


def _layer_desc(h_in, w, n_head: int, d_head: int, eps: float) -> LayerDesc:
    B, L, d = h_in.shape
    return LayerDesc(B, L, d, n_head, d_head, w["W1"].shape[0], eps, 0, 0, None)


def layer_workspace_size(h_in, w, n_head: int, d_head: int, M_cur: int, eps: float = 1e-5) -> int:
    """Workspace bytes txl_layer_fwd needs."""
    n = ctypes.c_size_t(0)
    desc = _layer_desc(h_in, w, n_head, d_head, eps)
    _check(lib().txl_layer_workspace_size(ctypes.byref(desc), M_cur, ctypes.byref(n)))
    return n.value


def layer_fwd(h_in, mem, w: dict, u, vb, n_head: int, d_head: int, *, eps: float = 1e-5, out=None, workspace=None,
              stream=None, clamp_len: int = 0, same_length: int = 0, mem_valid=None, ctx: Context | None = None):
    """One post-LN decoder layer (txl_layer_fwd).

    h_in [B, L, d] bf16; mem [B, M_cur, d] bf16 or None; w maps LAYER_KEYS to
    tensors (matrices bf16 in nn.Linear [out, in] layout, vectors float32, b1 /
    b2 may be None); u, vb [H, dh] float32.  clamp_len / same_length as in
    [SRC] MemTransformerLM (0 = off); mem_valid: int32 [B] on the device.
    ctx: a Context on h_in's device (default: the binding's own, context()).
    Returns h_out [B, L, d] bf16.
    """
    import torch
    if ctx is None:
        ctx = context(h_in.device)
    M_cur = 0 if mem is None else mem.shape[1]
    desc = _layer_desc(h_in, w, n_head, d_head, eps)
    desc.clamp_len = int(clamp_len)
    desc.same_length = int(same_length)
    if mem_valid is not None:
        if mem_valid.dtype != torch.int32 or not mem_valid.is_contiguous() or mem_valid.numel() != h_in.shape[0]:
            raise ValueError("mem_valid must be a contiguous int32 tensor of B entries")
        desc.mem_valid = mem_valid.data_ptr()
    if out is None:
        out = torch.empty_like(h_in)
    for t in [h_in, out] + ([mem] if M_cur else []) + [w[k] for k in LAYER_KEYS if w.get(k) is not None]:
        if not t.is_contiguous():
            raise ValueError("layer tensors must be contiguous")
    need = ctypes.c_size_t(0)
    _check(lib().txl_layer_workspace_size(ctypes.byref(desc), M_cur, ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(need.value, dtype=torch.uint8, device=h_in.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    lw = LayerWeights(*[(w[k].data_ptr() if w.get(k) is not None else None) for k in LAYER_KEYS])
    _check(lib().txl_layer_fwd(ctx.handle, ctypes.byref(desc), ctypes.byref(lw), _ptr(h_in), _ptr(mem if M_cur else None), M_cur,
                               _ptr(u), _ptr(vb), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def stack_segment(x, mems, layers: list, u, vb, n_head: int, d_head: int, mem_len: int, *, eps: float = 1e-5,
                  workspace=None, stream=None):
    """One segment through a layer stack, as [SRC] MemTransformerLM._forward
    followed by _update_mems: hids[0] = x, hids[n+1] = txl_layer_fwd(hids[n],
    mems[n]), then every memory is replaced by the Tail of [mems[n]; hids[n]]
    in one txl_mem_update_batched call.  Only sequences the library calls.

    x [B, L, d] bf16; mems: None (first segment) or a list of len(layers) + 1
    tensors [B, M_cur, d] bf16; layers: weight dicts as for layer_fwd.
    Returns (hids, new_mems); hids[-1] is the stack output.
    """
    import torch
    M_cur = 0 if mems is None else mems[0].shape[1]
    if workspace is None:
        need = layer_workspace_size(x, layers[0], n_head, d_head, M_cur, eps)
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    hids = [x]
    for n, w in enumerate(layers):
        hids.append(layer_fwd(hids[n], None if mems is None else mems[n], w, u, vb, n_head, d_head, eps=eps,
                              workspace=workspace, stream=stream))
    new_mems = mem_update_batched(mems, hids, mem_len, stream=stream)
    return hids, new_mems
