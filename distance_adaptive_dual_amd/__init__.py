"""DAR (Distance-Adaptive Representation) attention forward pass on MI355X.

Thin ctypes binding over ``libdar.so`` (C ABI in ``include/dar.h``).  The
functions below only marshal arguments: torch tensors provide device memory
and the current HIP stream; every step of the computation runs in the HIP
kernels of the library.  There is no fallback: if the library is missing or
a call fails, an exception is raised.

Method: "Dual Dimensionality for Local and Global Attention", Eqs. (1)-(4).
In bf16 mode the projections handed from dar_project to dar_attn_prefill are
float16 tensors (see include/dar.h); h, the weights and o are bfloat16.
Weights are column-major (pass a [out, in] tensor, the nn.Linear layout: the
equations' W in R^{in x out} transposed and made contiguous).
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdar.so")

DAR_FP32, DAR_BF16 = 0, 1
STATUS = {0: "DAR_OK", 1: "DAR_ERR_INVALID_ARG", 2: "DAR_ERR_UNSUPPORTED",
          3: "DAR_ERR_WORKSPACE", 4: "DAR_ERR_HIP"}
# Every entry point include/dar.h declares.
EXPORTS = ("dar_abi_version", "dar_status_string", "dar_pack_weight", "dar_fold",
           "dar_project",
           "dar_project_sigmoid",
           "dar_attn_prefill", "dar_attn_prefill_lse", "dar_attn_prefill_backward",
           "dar_decode_append", "dar_cache_from_prefill", "dar_prefill_chunk",
           "dar_attn_decode", "dar_cache_from_prefill_varlen", "dar_decode_append_varlen",
           "dar_attn_decode_varlen", "dar_decode_append_sigmoid",
           "dar_decode_append_varlen_sigmoid", "dar_prefill_chunk_sigmoid",
           "dar_attn_decode_noalloc", "dar_attn_decode_drope", "dar_project_drope",
           "dar_attn_prefill_drope", "dar_cache_from_prefill_drope", "dar_decode_append_drope",
           "dar_project_varlen", "dar_attn_prefill_varlen", "dar_cache_from_prefill_packed")

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.POINTER(ctypes.c_size_t)


class DarError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s returned %s" % (fn, STATUS.get(status, str(status))))
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libdar.so (built by ``distance_adaptive_dual_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libdar.so is not built; run python -m distance_adaptive_dual_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.dar_abi_version.restype = _I
        L.dar_abi_version.argtypes = []
        L.dar_status_string.restype = ctypes.c_char_p
        L.dar_status_string.argtypes = [_I]
        L.dar_fold.restype = _I
        L.dar_fold.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P]
        L.dar_project.restype = _I
        L.dar_project.argtypes = [_P] * 8 + [_I] * 7 + [ctypes.c_float, _I] + [_P] * 7 + [_SZ, _P]
        L.dar_project_sigmoid.restype = _I
        L.dar_project_sigmoid.argtypes = L.dar_project.argtypes
        L.dar_attn_prefill.restype = _I
        L.dar_attn_prefill.argtypes = [_P] * 5 + [_I] * 6 + [_P, _P, _SZ, _P]
        L.dar_pack_weight.restype = _I
        L.dar_pack_weight.argtypes = [_P, _I, _I, _I, _P, _P]
        L.dar_attn_prefill_lse.restype = _I
        L.dar_attn_prefill_lse.argtypes = [_P] * 5 + [_I] * 6 + [_P, _P, _P]
        L.dar_attn_prefill_backward.restype = _I
        L.dar_attn_prefill_backward.argtypes = [_P] * 8 + [_I] * 6 + [_P] * 6 + [_SZ, _P]
        L.dar_decode_append.restype = _I
        L.dar_decode_append.argtypes = [_P] * 5 + [_I] * 8 + [ctypes.c_float, _I] + [_P] * 5 + [
            _SZ, _P]
        L.dar_cache_from_prefill.restype = _I
        L.dar_cache_from_prefill.argtypes = [_P] * 3 + [_I] * 7 + [_I] + [_P] * 4
        L.dar_prefill_chunk.restype = _I
        L.dar_prefill_chunk.argtypes = [_P] * 7 + [_I] * 9 + [ctypes.c_float, _I] + [_P] * 5 + [
            _SZ, _P]
        L.dar_attn_decode.restype = _I
        L.dar_attn_decode.argtypes = [_P] * 6 + [_I] * 7 + [ctypes.c_float, _I, _P, _P, _SZ, _P]
        L.dar_cache_from_prefill_varlen.restype = _I
        L.dar_cache_from_prefill_varlen.argtypes = [_P] * 3 + [_I, _I, _P] + [_I] * 6 + [_P] * 4
        L.dar_decode_append_varlen.restype = _I
        L.dar_decode_append_varlen.argtypes = [_P] * 5 + [_I] * 5 + [_P, _I, _I, ctypes.c_float,
                                                                   _I] + [_P] * 5 + [_SZ, _P]
        L.dar_decode_append_sigmoid.restype = _I
        L.dar_decode_append_sigmoid.argtypes = L.dar_decode_append.argtypes
        L.dar_decode_append_varlen_sigmoid.restype = _I
        L.dar_decode_append_varlen_sigmoid.argtypes = L.dar_decode_append_varlen.argtypes
        L.dar_prefill_chunk_sigmoid.restype = _I
        L.dar_prefill_chunk_sigmoid.argtypes = L.dar_prefill_chunk.argtypes
        L.dar_attn_decode_noalloc.restype = _I
        L.dar_attn_decode_noalloc.argtypes = [_P] * 6 + [_I] * 7 + [ctypes.c_float, _I, _P, _P]
        L.dar_project_drope.restype = _I
        L.dar_project_drope.argtypes = [_P] * 10 + [_I] * 8 + [ctypes.c_float, _I] + [_P] * 9 + [
            _SZ, _P]
        L.dar_attn_prefill_drope.restype = _I
        L.dar_attn_prefill_drope.argtypes = [_P] * 7 + [_I] * 7 + [_P, _P]
        L.dar_cache_from_prefill_drope.restype = _I
        L.dar_cache_from_prefill_drope.argtypes = [_P] * 4 + [_I] * 9 + [_P] * 5
        L.dar_decode_append_drope.restype = _I
        L.dar_decode_append_drope.argtypes = [_P] * 7 + [_I] * 9 + [ctypes.c_float, _I] + [
            _P] * 7 + [_SZ, _P]
        L.dar_attn_decode_drope.restype = _I
        L.dar_attn_decode_drope.argtypes = [_P] * 8 + [_I] * 8 + [_I, _P, _P, _SZ, _P]
        L.dar_project_varlen.restype = _I
        L.dar_project_varlen.argtypes = [_P] * 9 + [_I] * 7 + [ctypes.c_float, _I] + [_P] * 7 + [
            _SZ, _P]
        L.dar_attn_prefill_varlen.restype = _I
        L.dar_attn_prefill_varlen.argtypes = [_P] * 6 + [_I] * 7 + [_P, _P]
        L.dar_cache_from_prefill_packed.restype = _I
        L.dar_cache_from_prefill_packed.argtypes = [_P] * 4 + [_I] * 9 + [_P] * 4
        L.dar_attn_decode_varlen.restype = _I
        L.dar_attn_decode_varlen.argtypes = [_P] * 6 + [_I, _P] + [_I] * 6 + [
            ctypes.c_float, _I, _P, _P, _SZ, _P]
        _lib = L
    return _lib


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    """Library mode of a tensor: bf16 I/O (bfloat16 tensors, or the float16
    intermediates of that mode) or fp32."""
    torch = _torch()
    if t.dtype in (torch.bfloat16, torch.float16):
        return DAR_BF16
    if t.dtype == torch.float32:
        return DAR_FP32
    raise TypeError("DAR tensors must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("DAR tensors must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("DAR tensors must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _on_stream(fn):
    """Run a binding call on the caller's `stream`, if one is given: the
    workspace and outputs it allocates, and the fills of fresh cache buffers,
    then belong to the stream the library launches on, so the caching
    allocator cannot hand their blocks out again while that stream still
    uses them."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def call(*args, **kwargs):
        stream = sig.bind_partial(*args, **kwargs).arguments.get("stream")
        if stream is None:
            return fn(*args, **kwargs)
        with _torch().cuda.stream(stream):
            return fn(*args, **kwargs)
    return call


def _check(fn: str, status: int):
    if status != 0:
        raise DarError(fn, status)


def _call_ws(fn: str, f, args, workspace, like, stream):
    """Calls entry point f with a workspace.  A caller-supplied workspace is
    tried first; when none is given (or it is too small) the size is queried
    and a fresh buffer allocated."""
    if workspace is not None and workspace.numel() > 0:  # an empty tensor's pointer is NULL
        n = ctypes.c_size_t(workspace.numel())
        st = f(*args, _ptr(workspace), ctypes.byref(n), _stream(stream))
        if st != 3:  # DAR_ERR_WORKSPACE
            _check(fn, st)
            return
    n = ctypes.c_size_t(0)
    _check(fn, f(*args, None, ctypes.byref(n), None))
    workspace = _workspace(n.value, like)
    n = ctypes.c_size_t(n.value)
    _check(fn, f(*args, _ptr(workspace), ctypes.byref(n), _stream(stream)))


def torch_uint8():
    return _torch().uint8


def _workspace(nbytes: int, like):
    # never NULL: a NULL workspace asks the library for its size instead
    return _torch().empty(max(nbytes, 256), dtype=torch_uint8(), device=like.device)


@_on_stream
def dar_fold(W_up, W_K, W_V, heads: int, d_k: int, W_upK=None, W_upV=None, stream=None):
    """W_upK = W_up W_K, W_upV = W_up W_V (column-major, [heads*d_k, d_down] tensors)."""
    torch = _torch()
    d_down, d = W_up.shape[1], W_up.shape[0]  # W_up given as [d, d_down] (column-major)
    hd = heads * d_k
    if W_upK is None:
        W_upK = torch.empty((hd, d_down), dtype=W_up.dtype, device=W_up.device)
    if W_upV is None:
        W_upV = torch.empty((hd, d_down), dtype=W_up.dtype, device=W_up.device)
    st = lib().dar_fold(_ptr(W_up), _ptr(W_K), _ptr(W_V), d, d_down, heads, d_k,
                        _dtype_code(W_up), _ptr(W_upK), _ptr(W_upV), _stream(stream))
    _check("dar_fold", st)
    return W_upK, W_upV


def _fake(i: int) -> int:
    """Distinct, aligned, never-dereferenced addresses for size queries (the
    library only compares them when workspace is NULL)."""
    return (1 << 44) + (i << 38)


def project_workspace_bytes(B, N, d, d_down, heads, d_k, pos0=0, folded=True, dtype=DAR_BF16):
    n = ctypes.c_size_t(0)
    f = [_fake(i) for i in range(14)]
    st = lib().dar_project(f[0], f[1], f[2], f[3], f[4], f[5],
                           f[6] if folded else None, f[7] if folded else None,
                           B, N, d, d_down, heads, d_k, pos0, 10000.0, dtype,
                           f[8], f[9], f[10], f[11], f[12], f[13], None, ctypes.byref(n), None)
    _check("dar_project", st)
    return n.value


@_on_stream
def dar_project(h, W_down, W_up, W_Q, W_K, W_V, heads: int, d_k: int, W_upK=None, W_upV=None,
                pos0: int = 0, rope_base: float = 10000.0, out=None, workspace=None,
                stream=None, sigmoid: bool = False):
    """Eqs. (1)-(3) projections.  Returns dict Q, K_loc, V_loc, h_D, K_glob, V_glob.

    h [B, N, d]; weights column-major ([out, in] tensors).  V_loc / V_glob come
    back as [B, heads, d_k, N] (token innermost).  sigmoid=True calls
    dar_project_sigmoid (h^D = sigmoid(h W_down))."""
    torch = _torch()
    B, N, d = h.shape
    d_down = W_down.shape[0]
    dt = _dtype_code(h)
    if out is None:
        kw = dict(dtype=torch.float16 if dt == DAR_BF16 else torch.float32, device=h.device)
        out = dict(Q=torch.empty((B, heads, N, d_k), **kw),
                   K_loc=torch.empty((B, heads, N, d_k), **kw),
                   V_loc=torch.empty((B, heads, d_k, N), **kw),
                   h_D=torch.empty((B, N, d_down), **kw),
                   K_glob=torch.empty((B, heads, N, d_k), **kw),
                   V_glob=torch.empty((B, heads, d_k, N), **kw))
    args = [_ptr(h), _ptr(W_down), _ptr(W_up), _ptr(W_Q), _ptr(W_K), _ptr(W_V),
            _ptr(W_upK), _ptr(W_upV), B, N, d, d_down, heads, d_k, pos0, float(rope_base), dt]
    args += [_ptr(out[k]) for k in ("Q", "K_loc", "V_loc", "h_D", "K_glob", "V_glob")]
    name = "dar_project_sigmoid" if sigmoid else "dar_project"
    _call_ws(name, getattr(lib(), name), args, workspace, h, stream)
    return out


def attn_backward_workspace_bytes(B, N, heads, d_k, dtype=DAR_BF16):
    n = ctypes.c_size_t(0)
    f = [_fake(i) for i in range(12)]
    st = lib().dar_attn_prefill_backward(*f[:7], None, B, N, heads, d_k, 0, dtype, *f[7:], None,
                                         ctypes.byref(n), None)
    _check("dar_attn_prefill_backward", st)
    return n.value


@_on_stream
def dar_attn_prefill_backward(Q, K_loc, V_loc, K_glob, V_glob, o, dO, w: int, lse=None,
                              out=None, workspace=None, stream=None):
    """Gradients of dar_attn_prefill for dL/do = dO.  Returns dict dQ, dK_loc,
    dV_loc, dK_glob, dV_glob (float32, [B, heads, N, d_k]; dV not transposed).
    lse: the forward's normaliser from dar_attn_prefill_lse, or None."""
    torch = _torch()
    B, H, N, d_k = Q.shape
    dt = _dtype_code(Q)
    if out is None:
        out = {k: torch.empty((B, H, N, d_k), dtype=torch.float32, device=Q.device)
               for k in ("dQ", "dK_loc", "dV_loc", "dK_glob", "dV_glob")}
    args = [_ptr(Q), _ptr(K_loc), _ptr(V_loc), _ptr(K_glob), _ptr(V_glob), _ptr(o), _ptr(dO),
            _ptr(lse), B, N, H, d_k, int(w), dt]
    args += [_ptr(out[k]) for k in ("dQ", "dK_loc", "dV_loc", "dK_glob", "dV_glob")]
    _call_ws("dar_attn_prefill_backward", lib().dar_attn_prefill_backward, args, workspace, Q,
             stream)
    return out


@_on_stream
def dar_attn_prefill_lse(Q, K_loc, V_loc, K_glob, V_glob, w: int, o=None, lse=None,
                         stream=None):
    """dar_attn_prefill that also returns lse [B, heads, N] (float32, natural log)."""
    torch = _torch()
    B, H, N, d_k = Q.shape
    dt = _dtype_code(Q)
    if o is None:
        o = torch.empty((B, N, H * d_k), dtype=torch.bfloat16 if dt == DAR_BF16 else torch.float32,
                        device=Q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=Q.device)
    st = lib().dar_attn_prefill_lse(_ptr(Q), _ptr(K_loc), _ptr(V_loc), _ptr(K_glob), _ptr(V_glob),
                                    B, N, H, d_k, int(w), dt, _ptr(o), _ptr(lse), _stream(stream))
    _check("dar_attn_prefill_lse", st)
    return o, lse


@_on_stream
def dar_attn_prefill(Q, K_loc, V_loc, K_glob, V_glob, w: int, o=None, stream=None):
    """Eq. (4) with the Eq. (3) selection.  Returns o [B, N, heads*d_k]."""
    torch = _torch()
    B, H, N, d_k = Q.shape
    dt = _dtype_code(Q)
    if o is None:
        o = torch.empty((B, N, H * d_k), dtype=torch.bfloat16 if dt == DAR_BF16 else torch.float32,
                        device=Q.device)
    st = lib().dar_attn_prefill(_ptr(Q), _ptr(K_loc), _ptr(V_loc), _ptr(K_glob), _ptr(V_glob),
                                B, N, H, d_k, int(w), dt, _ptr(o), None, None, _stream(stream))
    _check("dar_attn_prefill", st)
    return o


@_on_stream
def dar_pack_weight(W, out=None, stream=None):
    """The equations' matrix W in R^{rows x cols}, given row-major as a
    [rows, cols] tensor, in the library's column-major layout: returns a
    [cols, rows] tensor holding the same matrix (a bit-exact transpose run by
    the library)."""
    torch = _torch()
    rows, cols = W.shape
    if out is None:
        out = torch.empty((cols, rows), dtype=W.dtype, device=W.device)
    st = lib().dar_pack_weight(_ptr(W), rows, cols, _dtype_code(W), _ptr(out), _stream(stream))
    _check("dar_pack_weight", st)
    return out


@_on_stream
def dar_decode_append(h, W_down, W_Q, W_K, W_V, heads: int, d_k: int, pos: int, q, K_win, V_win,
                      h_D, rope_base: float = 10000.0, workspace=None, stream=None,
                      sigmoid: bool = False):
    """Project the token at position `pos` of every sequence into the cache:
    q [B, heads, d_k] (RoPE'd), ring slot pos mod w of K_win / V_win, row pos
    of h_D.  h [B, d]; weights column-major.  Returns q."""
    B, d = h.shape
    d_down = W_down.shape[0]
    w = K_win.shape[2] if K_win is not None else 0
    cap = h_D.shape[1]
    args = [_ptr(h), _ptr(W_down), _ptr(W_Q), _ptr(W_K), _ptr(W_V), B, d, d_down, heads, d_k,
            int(pos), int(w), cap, float(rope_base), _dtype_code(h), _ptr(q),
            _ptr(K_win) if w > 0 else None, _ptr(V_win) if w > 0 else None, _ptr(h_D)]
    name = "dar_decode_append_sigmoid" if sigmoid else "dar_decode_append"
    _call_ws(name, getattr(lib(), name), args, workspace, h, stream)
    return q


@_on_stream
def dar_cache_from_prefill(h_D, K_loc, V_loc, w: int, cap: int = None, h_D_cache=None,
                           K_win=None, V_win=None, stream=None):
    """Decode cache of a prefilled prompt from dar_project's outputs (fp16):
    latent rows 0..N-1 and the ring slots of positions max(0, N-w)..N-1, in
    bf16.  Returns (h_D_cache [B, cap, d_down], K_win, V_win [B, heads, w, d_k]);
    K_win / V_win are None when w = 0."""
    torch = _torch()
    B, N, d_down = h_D.shape
    _, H, _, d_k = K_loc.shape
    cap = N if cap is None else cap
    kw = dict(dtype=torch.bfloat16, device=h_D.device)
    if h_D_cache is None:
        h_D_cache = torch.zeros((B, cap, d_down), **kw)
    if w > 0 and K_win is None:
        K_win = torch.zeros((B, H, w, d_k), **kw)
    if w > 0 and V_win is None:
        V_win = torch.zeros((B, H, w, d_k), **kw)
    st = lib().dar_cache_from_prefill(_ptr(h_D), _ptr(K_loc) if w > 0 else None,
                                      _ptr(V_loc) if w > 0 else None, B, N, H, d_k, d_down,
                                      int(w), int(h_D_cache.shape[1]), _dtype_code(h_D),
                                      _ptr(h_D_cache), _ptr(K_win) if w > 0 else None,
                                      _ptr(V_win) if w > 0 else None, _stream(stream))
    _check("dar_cache_from_prefill", st)
    return h_D_cache, K_win, V_win


def _lens(t, B: int):
    """A device int32 vector of B per-sequence lengths or positions."""
    torch = _torch()
    if t.dtype != torch.int32 or t.dim() != 1 or t.numel() != B:
        raise ValueError("per-sequence lengths/positions must be an int32 vector of %d" % B)
    return _ptr(t)


@_on_stream
def dar_cache_from_prefill_varlen(h_D, K_loc, V_loc, lens, w: int, cap: int = None,
                                  h_D_cache=None, K_win=None, V_win=None, stream=None):
    """dar_cache_from_prefill for a padded batch whose sequence b has lens[b]
    tokens (lens: device int32 [B]).  Returns (h_D_cache, K_win, V_win)."""
    torch = _torch()
    B, N, d_down = h_D.shape
    _, H, _, d_k = K_loc.shape
    cap = N if cap is None else cap
    kw = dict(dtype=torch.bfloat16, device=h_D.device)
    if h_D_cache is None:
        h_D_cache = torch.zeros((B, cap, d_down), **kw)
    if w > 0 and K_win is None:
        K_win = torch.zeros((B, H, w, d_k), **kw)
    if w > 0 and V_win is None:
        V_win = torch.zeros((B, H, w, d_k), **kw)
    st = lib().dar_cache_from_prefill_varlen(
        _ptr(h_D), _ptr(K_loc) if w > 0 else None, _ptr(V_loc) if w > 0 else None, B, N,
        _lens(lens, B), H, d_k, d_down, int(w), int(h_D_cache.shape[1]), _dtype_code(h_D),
        _ptr(h_D_cache), _ptr(K_win) if w > 0 else None, _ptr(V_win) if w > 0 else None,
        _stream(stream))
    _check("dar_cache_from_prefill_varlen", st)
    return h_D_cache, K_win, V_win


@_on_stream
def dar_decode_append_varlen(h, W_down, W_Q, W_K, W_V, heads: int, d_k: int, pos, q, K_win,
                             V_win, h_D, rope_base: float = 10000.0, workspace=None,
                             stream=None, sigmoid: bool = False):
    """dar_decode_append with sequence b's token at position pos[b] (device
    int32 [B]).  Returns q."""
    B, d = h.shape
    d_down = W_down.shape[0]
    w = K_win.shape[2] if K_win is not None else 0
    cap = h_D.shape[1]
    args = [_ptr(h), _ptr(W_down), _ptr(W_Q), _ptr(W_K), _ptr(W_V), B, d, d_down, heads, d_k,
            _lens(pos, B), int(w), cap, float(rope_base), _dtype_code(h), _ptr(q),
            _ptr(K_win) if w > 0 else None, _ptr(V_win) if w > 0 else None, _ptr(h_D)]
    name = "dar_decode_append_varlen_sigmoid" if sigmoid else "dar_decode_append_varlen"
    _call_ws(name, getattr(lib(), name), args, workspace, h, stream)
    return q


@_on_stream
def dar_attn_decode_varlen(q, K_win, V_win, h_D, W_upK, W_upV, ctx_lens, max_ctx: int, w: int,
                           rope_base: float = 10000.0, o=None, workspace=None, stream=None):
    """dar_attn_decode with sequence b's query at position ctx_lens[b] - 1
    (device int32 [B], each in [1, max_ctx]).  Returns o [B, heads*d_k]."""
    torch = _torch()
    B, H, d_k = q.shape
    cap, d_down = h_D.shape[1], h_D.shape[2]
    if o is None:
        o = torch.empty((B, H * d_k), dtype=q.dtype, device=q.device)
    args = [_ptr(q), _ptr(K_win) if w > 0 else None, _ptr(V_win) if w > 0 else None, _ptr(h_D),
            _ptr(W_upK), _ptr(W_upV), B, _lens(ctx_lens, B), int(max_ctx), cap, H, d_k, d_down,
            int(w), float(rope_base), _dtype_code(q), _ptr(o)]
    _call_ws("dar_attn_decode_varlen", lib().dar_attn_decode_varlen, args, workspace, q, stream)
    return o


def chunk_workspace_bytes(B, C, d, d_down, heads, d_k, p0, w, cap):
    n = ctypes.c_size_t(0)
    f = [_fake(i) for i in range(12)]
    st = lib().dar_prefill_chunk(*f[:7], B, C, d, d_down, heads, d_k, p0, w, cap, 10000.0,
                                 DAR_BF16, f[7], f[8] if w > 0 else None, f[9] if w > 0 else None,
                                 f[10], None, ctypes.byref(n), None)
    _check("dar_prefill_chunk", st)
    return n.value


@_on_stream
def dar_prefill_chunk(h, W_down, W_Q, W_K, W_V, W_upK, W_upV, heads: int, d_k: int, p0: int,
                      h_D_cache, K_win, V_win, w: int, o=None, rope_base: float = 10000.0,
                      workspace=None, stream=None, sigmoid: bool = False):
    """Prefill the chunk h [B, C, d] at positions p0 .. p0+C-1 over the cache
    (h_D_cache [B, cap, d_down], ring K_win / V_win [B, heads, w, d_k], bf16;
    updated in place).  Returns o [B, C, heads*d_k]."""
    torch = _torch()
    B, C, d = h.shape
    d_down = W_down.shape[0]
    cap = h_D_cache.shape[1]
    if o is None:
        o = torch.empty((B, C, heads * d_k), dtype=torch.bfloat16, device=h.device)
    args = [_ptr(h), _ptr(W_down), _ptr(W_Q), _ptr(W_K), _ptr(W_V), _ptr(W_upK), _ptr(W_upV),
            B, C, d, d_down, heads, d_k, int(p0), int(w), cap, float(rope_base), _dtype_code(h),
            _ptr(h_D_cache), _ptr(K_win) if w > 0 else None, _ptr(V_win) if w > 0 else None,
            _ptr(o)]
    name = "dar_prefill_chunk_sigmoid" if sigmoid else "dar_prefill_chunk"
    _call_ws(name, getattr(lib(), name), args, workspace, h, stream)
    return o


def decode_workspace_bytes(B, ctx_len, cap, heads, d_k, d_down, w, dtype=DAR_BF16):
    n = ctypes.c_size_t(0)
    f = [_fake(i) for i in range(7)]
    st = lib().dar_attn_decode(f[0], f[1], f[2], f[3], f[4], f[5], B, ctx_len, cap, heads, d_k,
                               d_down, w, 10000.0, dtype, f[6], None, ctypes.byref(n), None)
    _check("dar_attn_decode", st)
    return n.value


@_on_stream
def dar_attn_decode(q, K_win, V_win, h_D, W_upK, W_upV, ctx_len: int, w: int,
                    rope_base: float = 10000.0, o=None, workspace=None, stream=None):
    """One query per sequence at position ctx_len-1 over the mixed cache.  Returns o [B, heads*d_k]."""
    torch = _torch()
    B, H, d_k = q.shape
    cap, d_down = h_D.shape[1], h_D.shape[2]
    if o is None:
        o = torch.empty((B, H * d_k), dtype=q.dtype, device=q.device)
    args = [_ptr(q), _ptr(K_win) if w > 0 else None, _ptr(V_win) if w > 0 else None, _ptr(h_D),
            _ptr(W_upK), _ptr(W_upV), B, int(ctx_len), cap, H, d_k, d_down, int(w),
            float(rope_base), _dtype_code(q), _ptr(o)]
    _call_ws("dar_attn_decode", lib().dar_attn_decode, args, workspace, q, stream)
    return o


@_on_stream
def dar_attn_decode_noalloc(q, K_win, V_win, h_D, W_upK, W_upV, ctx_len: int, w: int, o,
                            rope_base: float = 10000.0, stream=None):
    """dar_attn_decode without a workspace: the library's static per-GPU
    scratch array serves as one (calls on one GPU must not overlap).  The
    output o [B, heads*d_k] must be given: nothing is allocated.  Returns o."""
    B, H, d_k = q.shape
    cap, d_down = h_D.shape[1], h_D.shape[2]
    st = lib().dar_attn_decode_noalloc(
        _ptr(q), _ptr(K_win) if w > 0 else None, _ptr(V_win) if w > 0 else None, _ptr(h_D),
        _ptr(W_upK), _ptr(W_upV), B, int(ctx_len), cap, H, d_k, d_down, int(w),
        float(rope_base), _dtype_code(q), _ptr(o), _stream(stream))
    _check("dar_attn_decode_noalloc", st)
    return o


def decode_drope_workspace_bytes(B, ctx_len, cap, heads, d_k, d_R, d_down, w):
    n = ctypes.c_size_t(0)
    f = [_fake(i) for i in range(9)]
    st = lib().dar_attn_decode_drope(*f[:8], B, ctx_len, cap, heads, d_k, d_R, d_down, w,
                                     DAR_BF16, f[8], None, ctypes.byref(n), None)
    _check("dar_attn_decode_drope", st)
    return n.value


@_on_stream
def dar_attn_decode_drope(qC, qR, K_win, V_win, KR, h_D, W_upK, W_upV, ctx_len: int, w: int,
                          o=None, workspace=None, stream=None):
    """Decode step of the decoupled-RoPE variant at position ctx_len-1.
    qC [B, heads, d_k], qR [B, heads, d_R] (rotated); K_win / V_win
    [B, heads, w, d_k] (content keys, values); KR [B, cap, d_R] (rotary keys
    of every position); h_D [B, cap, d_down]; W_upK / W_upV from dar_fold.
    Returns o [B, heads*d_k]."""
    torch = _torch()
    B, H, d_k = qC.shape
    d_R = qR.shape[2]
    cap, d_down = h_D.shape[1], h_D.shape[2]
    if o is None:
        o = torch.empty((B, H * d_k), dtype=qC.dtype, device=qC.device)
    args = [_ptr(qC), _ptr(qR), _ptr(K_win) if w > 0 else None, _ptr(V_win) if w > 0 else None,
            _ptr(KR), _ptr(h_D), _ptr(W_upK), _ptr(W_upV), B, int(ctx_len), cap, H, d_k, d_R,
            d_down, int(w), _dtype_code(qC), _ptr(o)]
    _call_ws("dar_attn_decode_drope", lib().dar_attn_decode_drope, args, workspace, qC, stream)
    return o


@_on_stream
def dar_project_drope(h, W_down, W_up, W_Q, W_K, W_V, W_QR, W_KR, heads: int, d_k: int,
                      W_upK=None, W_upV=None, pos0: int = 0, rope_base: float = 10000.0,
                      out=None, workspace=None, stream=None):
    """Projections of the decoupled-RoPE variant.  Returns dict QC, QR, K_loc,
    V_loc, h_D, K_glob, V_glob, KR (fp16).  Weights column-major ([out, in]):
    W_QR [heads*d_R, d], W_KR [d_R, d]."""
    torch = _torch()
    B, N, d = h.shape
    d_down = W_down.shape[0]
    d_R = W_KR.shape[0]
    if out is None:
        kw = dict(dtype=torch.float16, device=h.device)
        out = dict(QC=torch.empty((B, heads, N, d_k), **kw),
                   QR=torch.empty((B, heads, N, d_R), **kw),
                   K_loc=torch.empty((B, heads, N, d_k), **kw),
                   V_loc=torch.empty((B, heads, d_k, N), **kw),
                   h_D=torch.empty((B, N, d_down), **kw),
                   K_glob=torch.empty((B, heads, N, d_k), **kw),
                   V_glob=torch.empty((B, heads, d_k, N), **kw),
                   KR=torch.empty((B, N, d_R), **kw))
    args = [_ptr(h), _ptr(W_down), _ptr(W_up), _ptr(W_Q), _ptr(W_K), _ptr(W_V), _ptr(W_QR),
            _ptr(W_KR), _ptr(W_upK), _ptr(W_upV), B, N, d, d_down, heads, d_k, d_R, int(pos0),
            float(rope_base), _dtype_code(h)]
    args += [_ptr(out[k]) for k in ("QC", "QR", "K_loc", "V_loc", "h_D", "K_glob", "V_glob", "KR")]
    _call_ws("dar_project_drope", lib().dar_project_drope, args, workspace, h, stream)
    return out


@_on_stream
def dar_attn_prefill_drope(P, w: int, o=None, stream=None):
    """Attention of the variant from dar_project_drope's outputs P.  Returns
    o [B, N, heads*d_k] (bf16)."""
    torch = _torch()
    B, H, N, d_k = P["QC"].shape
    d_R = P["KR"].shape[2]
    if o is None:
        o = torch.empty((B, N, H * d_k), dtype=torch.bfloat16, device=P["QC"].device)
    st = lib().dar_attn_prefill_drope(_ptr(P["QC"]), _ptr(P["QR"]), _ptr(P["K_loc"]),
                                      _ptr(P["V_loc"]), _ptr(P["K_glob"]), _ptr(P["V_glob"]),
                                      _ptr(P["KR"]), B, N, H, d_k, d_R, int(w),
                                      _dtype_code(P["QC"]), _ptr(o), _stream(stream))
    _check("dar_attn_prefill_drope", st)
    return o


@_on_stream
def dar_cache_from_prefill_drope(P, w: int, cap: int = None, stream=None):
    """The variant's decode cache from dar_project_drope's outputs P: returns
    (h_D_cache [B, cap, d_down], K_win, V_win [B, heads, w, d_k] or None,
    KR_cache [B, cap, d_R]), bf16."""
    torch = _torch()
    B, N, d_down = P["h_D"].shape
    _, H, _, d_k = P["K_loc"].shape
    d_R = P["KR"].shape[2]
    cap = N if cap is None else cap
    kw = dict(dtype=torch.bfloat16, device=P["h_D"].device)
    L = torch.zeros((B, cap, d_down), **kw)
    KRc = torch.zeros((B, cap, d_R), **kw)
    Kw = torch.zeros((B, H, w, d_k), **kw) if w > 0 else None
    Vw = torch.zeros((B, H, w, d_k), **kw) if w > 0 else None
    st = lib().dar_cache_from_prefill_drope(
        _ptr(P["h_D"]), _ptr(P["K_loc"]) if w > 0 else None, _ptr(P["V_loc"]) if w > 0 else None,
        _ptr(P["KR"]), B, N, H, d_k, d_down, d_R, int(w), cap, DAR_BF16, _ptr(L),
        _ptr(Kw) if w > 0 else None, _ptr(Vw) if w > 0 else None, _ptr(KRc), _stream(stream))
    _check("dar_cache_from_prefill_drope", st)
    return L, Kw, Vw, KRc


@_on_stream
def dar_decode_append_drope(h, W_down, W_Q, W_K, W_V, W_QR, W_KR, heads: int, d_k: int,
                            pos: int, qC, qR, K_win, V_win, h_D, KR, rope_base: float = 10000.0,
                            workspace=None, stream=None):
    """The variant's token at position `pos` of every sequence into its cache.
    h [B, d]; weights column-major.  Returns (qC, qR)."""
    B, d = h.shape
    d_down = W_down.shape[0]
    d_R = W_KR.shape[0]
    w = K_win.shape[2] if K_win is not None else 0
    cap = h_D.shape[1]
    args = [_ptr(h), _ptr(W_down), _ptr(W_Q), _ptr(W_K), _ptr(W_V), _ptr(W_QR), _ptr(W_KR), B, d,
            d_down, heads, d_k, d_R, int(pos), int(w), cap, float(rope_base), _dtype_code(h),
            _ptr(qC), _ptr(qR), _ptr(K_win) if w > 0 else None, _ptr(V_win) if w > 0 else None,
            _ptr(h_D), _ptr(KR)]
    _call_ws("dar_decode_append_drope", lib().dar_decode_append_drope, args, workspace, h, stream)
    return qC, qR


@_on_stream
def dar_project_varlen(h, W_down, W_up, W_Q, W_K, W_V, heads: int, d_k: int, cu_seqlens,
                       max_len: int, W_upK=None, W_upV=None, rope_base: float = 10000.0, out=None,
                       workspace=None, stream=None):
    """Projections of a ragged batch without padding: h [T, d] packs the
    prompts, cu_seqlens (int32 device tensor, B + 1 entries) their starts.
    Returns dict Q, K_loc, V_loc, K_glob, V_glob (flat fp16 tensors of
    T*heads*d_k elements, one block per prompt; see varlen_block) and h_D
    [T, d_down]."""
    torch = _torch()
    T, d = h.shape
    d_down = W_down.shape[0]
    B = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if out is None:
        kw = dict(dtype=torch.float16, device=h.device)
        n = T * heads * d_k
        out = {k: torch.empty(n, **kw) for k in ("Q", "K_loc", "V_loc", "K_glob", "V_glob")}
        out["h_D"] = torch.empty((T, d_down), **kw)
    args = [_ptr(h), _ptr(W_down), _ptr(W_up), _ptr(W_Q), _ptr(W_K), _ptr(W_V), _ptr(W_upK),
            _ptr(W_upV), _ptr(cu_seqlens), B, T, int(max_len), d, d_down, heads, d_k,
            float(rope_base), _dtype_code(h)]
    args += [_ptr(out[k]) for k in ("Q", "K_loc", "V_loc", "h_D", "K_glob", "V_glob")]
    _call_ws("dar_project_varlen", lib().dar_project_varlen, args, workspace, h, stream)
    return out


def varlen_block(x, starts, b: int, heads: int, d_k: int, transposed: bool = False):
    """Prompt b's block of a packed head-major array from dar_project_varlen:
    a view [heads, len_b, d_k] ([heads, d_k, len_b] for V).  starts: the
    prompts' start rows as host integers (cu_seqlens on the host)."""
    lo, hi = int(starts[b]), int(starts[b + 1])
    blk = x[lo * heads * d_k:hi * heads * d_k]
    return blk.view(heads, d_k, hi - lo) if transposed else blk.view(heads, hi - lo, d_k)


@_on_stream
def dar_attn_prefill_varlen(P, cu_seqlens, max_len: int, heads: int, d_k: int, w: int, o=None,
                            stream=None):
    """Attention of a ragged batch from dar_project_varlen's outputs P.
    Returns o [T, heads*d_k] (bf16)."""
    torch = _torch()
    T = P["h_D"].shape[0]
    B = cu_seqlens.numel() - 1
    if o is None:
        o = torch.empty((T, heads * d_k), dtype=torch.bfloat16, device=P["Q"].device)
    st = lib().dar_attn_prefill_varlen(_ptr(P["Q"]), _ptr(P["K_loc"]), _ptr(P["V_loc"]),
                                       _ptr(P["K_glob"]), _ptr(P["V_glob"]), _ptr(cu_seqlens), B,
                                       T, int(max_len), heads, d_k, int(w),
                                       _dtype_code(P["Q"]), _ptr(o), _stream(stream))
    _check("dar_attn_prefill_varlen", st)
    return o


@_on_stream
def dar_cache_from_prefill_packed(P, cu_seqlens, max_len: int, heads: int, d_k: int, w: int,
                                  cap: int = None, h_D_cache=None, K_win=None, V_win=None,
                                  stream=None):
    """The decode cache of a ragged batch from dar_project_varlen's outputs P:
    prompt b's latent rows and its last min(w, len_b) ring slots.  Returns
    (h_D_cache [B, cap, d_down], K_win, V_win [B, heads, w, d_k]) (bf16)."""
    torch = _torch()
    T, d_down = P["h_D"].shape
    B = cu_seqlens.numel() - 1
    cap = int(max_len) if cap is None else cap
    kw = dict(dtype=torch.bfloat16, device=P["h_D"].device)
    if h_D_cache is None:
        h_D_cache = torch.zeros((B, cap, d_down), **kw)
    if w > 0 and K_win is None:
        K_win = torch.zeros((B, heads, w, d_k), **kw)
    if w > 0 and V_win is None:
        V_win = torch.zeros((B, heads, w, d_k), **kw)
    st = lib().dar_cache_from_prefill_packed(
        _ptr(P["h_D"]), _ptr(P["K_loc"]) if w > 0 else None,
        _ptr(P["V_loc"]) if w > 0 else None, _ptr(cu_seqlens), B, T, int(max_len), heads, d_k,
        d_down, int(w), int(h_D_cache.shape[1]), _dtype_code(P["h_D"]), _ptr(h_D_cache),
        _ptr(K_win) if w > 0 else None, _ptr(V_win) if w > 0 else None, _stream(stream))
    _check("dar_cache_from_prefill_packed", st)
    return h_D_cache, K_win, V_win
