"""fp64 CPU oracle for DAR attention (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It is independent of the HIP path:
it shares no code with ``distance_adaptive_dual_amd`` and never imports it.

The arithmetic lives in ``dar_oracle.c`` (plain loops from the DAR paper,
"Dual Dimensionality for Local and Global Attention", Eqs. 1-4); this module
only marshals numpy float64 arrays to it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dar_oracle.c")
_LIB = os.path.join(_HERE, "libdar_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.dar_oracle_threads.restype = ctypes.c_int
        lib.dar_oracle_project.restype = ctypes.c_int
        lib.dar_oracle_project.argtypes = [_D] * 6 + [ctypes.c_int] * 6 + [
            ctypes.c_long, ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int] + [_D] * 7
        lib.dar_oracle_project_act.restype = ctypes.c_int
        lib.dar_oracle_project_act.argtypes = [_D] * 6 + [ctypes.c_int] * 6 + [
            ctypes.c_long, ctypes.c_double] + [ctypes.c_int] * 4 + [_D] * 7
        lib.dar_oracle_attend.restype = ctypes.c_int
        lib.dar_oracle_attend.argtypes = [_D] * 5 + [ctypes.c_int] * 4 + [ctypes.c_long] + [_D] * 2
        lib.dar_oracle_attend_rows.restype = ctypes.c_int
        lib.dar_oracle_attend_rows.argtypes = [_D] * 5 + [ctypes.c_int] * 4 + [
            ctypes.c_long, ctypes.c_int, _I, _I, _I, _D, _D]
        lib.dar_oracle_attend_lse.restype = ctypes.c_int
        lib.dar_oracle_attend_lse.argtypes = [_D] * 3 + [ctypes.c_int] * 4 + [ctypes.c_long, _D]
        lib.dar_oracle_attend_backward.restype = ctypes.c_int
        lib.dar_oracle_attend_backward.argtypes = [_D] * 6 + [ctypes.c_int] * 4 + [
            ctypes.c_long] + [_D] * 5
        lib.dar_oracle_decode.restype = ctypes.c_int
        lib.dar_oracle_decode.argtypes = [_D] * 7 + [ctypes.c_int, ctypes.c_long, ctypes.c_long] + [
            ctypes.c_int] * 4 + [ctypes.c_long, ctypes.c_double, ctypes.c_int, ctypes.c_int, _D]
        lib.dar_oracle_project_drope.restype = ctypes.c_int
        lib.dar_oracle_project_drope.argtypes = [_D] * 8 + [ctypes.c_int] * 7 + [
            ctypes.c_long, ctypes.c_double] + [ctypes.c_int] * 3 + [_D] * 9
        lib.dar_oracle_attend_drope.restype = ctypes.c_int
        lib.dar_oracle_attend_drope.argtypes = [_D] * 7 + [ctypes.c_int] * 5 + [
            ctypes.c_long, _D, _D]
        lib.dar_oracle_decode_drope.restype = ctypes.c_int
        lib.dar_oracle_decode_drope.argtypes = [_D] * 9 + [ctypes.c_int, ctypes.c_long,
                                                           ctypes.c_long] + [ctypes.c_int] * 5 + [
            ctypes.c_long, ctypes.c_int, ctypes.c_int, _D]
        _lib = lib
    return _lib


def _p(a):
    return a.ctypes.data_as(_D)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def threads() -> int:
    return _load().dar_oracle_threads()


def project(h, W_down, W_up, W_Q, W_K, W_V, H, d_k, pos0=0, base=10000.0, n_tok=None,
            heads=None, act="linear"):
    """Eqs. 1-3 projections.  Returns dict hD, hp, Q, KL, VL, KG, VG (float64).

    h [B,N,d]; Q/KL/VL/KG/VG [B,H,N,d_k]; only tokens < n_tok and heads in the
    ``heads`` range (lo, hi) are computed (the rest stay zero).  act="sigmoid":
    the variant with a sigmoid after the down-projection of Eq. 1.
    """
    if act not in ("linear", "sigmoid"):
        raise ValueError("act must be 'linear' or 'sigmoid'")
    h, W_down, W_up, W_Q, W_K, W_V = map(_f64, (h, W_down, W_up, W_Q, W_K, W_V))
    B, N, d = h.shape
    d_down = W_down.shape[1]
    assert W_down.shape == (d, d_down) and W_up.shape == (d_down, d)
    assert W_Q.shape == W_K.shape == W_V.shape == (d, H * d_k)
    n_tok = N if n_tok is None else int(n_tok)
    lo, hi = (0, H) if heads is None else heads
    out = dict(hD=np.zeros((B, N, d_down)), hp=np.zeros((B, N, d)))
    for k in ("Q", "KL", "VL", "KG", "VG"):
        out[k] = np.zeros((B, H, N, d_k))
    rc = _load().dar_oracle_project_act(
        _p(h), _p(W_down), _p(W_up), _p(W_Q), _p(W_K), _p(W_V), B, N, d, d_down, H, d_k,
        int(pos0), float(base), n_tok, lo, hi, 1 if act == "sigmoid" else 0, _p(out["hD"]),
        _p(out["hp"]), _p(out["Q"]), _p(out["KL"]), _p(out["VL"]), _p(out["KG"]),
        _p(out["VG"]))
    if rc != 0:
        raise ValueError("dar_oracle_project rejected its arguments")
    return out


def attend(P, w):
    """Eq. 3 selection + Eq. 4 for every row.  Returns (o [B,N,H*d_k], rowsum [B,H,N])."""
    Q, KL, VL, KG, VG = (_f64(P[k]) for k in ("Q", "KL", "VL", "KG", "VG"))
    B, H, N, d_k = Q.shape
    o = np.zeros((B, N, H * d_k))
    rs = np.zeros((B, H, N))
    rc = _load().dar_oracle_attend(_p(Q), _p(KL), _p(VL), _p(KG), _p(VG), B, N, H, d_k,
                                   int(w), _p(o), _p(rs))
    if rc != 0:
        raise ValueError("dar_oracle_attend rejected its arguments")
    return o, rs


def attend_rows(P, w, rows):
    """Selected rows [(b, head, i), ...].  Returns (o_rows [n, d_k], rowsum [n])."""
    Q, KL, VL, KG, VG = (_f64(P[k]) for k in ("Q", "KL", "VL", "KG", "VG"))
    B, H, N, d_k = Q.shape
    rows = np.asarray(rows, dtype=np.int32).reshape(-1, 3)
    rb, rh, ri = (np.ascontiguousarray(rows[:, c]) for c in range(3))
    o = np.zeros((len(rows), d_k))
    rs = np.zeros(len(rows))
    I = lambda a: a.ctypes.data_as(_I)  # noqa: E731
    rc = _load().dar_oracle_attend_rows(_p(Q), _p(KL), _p(VL), _p(KG), _p(VG), B, N, H, d_k,
                                        int(w), len(rows), I(rb), I(rh), I(ri), _p(o), _p(rs))
    if rc != 0:
        raise ValueError("dar_oracle_attend_rows rejected its arguments")
    return o, rs


def attend_lse(P, w):
    """Row normalisers of Eq. 4: lse [B,H,N] = log sum_{j<=i} exp(q_i.k_j/sqrt(d_k))."""
    Q, KL, KG = (_f64(P[k]) for k in ("Q", "KL", "KG"))
    B, H, N, d_k = Q.shape
    lse = np.zeros((B, H, N))
    rc = _load().dar_oracle_attend_lse(_p(Q), _p(KL), _p(KG), B, N, H, d_k, int(w), _p(lse))
    if rc != 0:
        raise ValueError("dar_oracle_attend_lse rejected its arguments")
    return lse


def attend_backward(P, w, dO):
    """Gradients of the Eq. 3-4 attention for dL/do = dO [B,N,H*d_k].  Returns
    dict dQ, dKL, dVL, dKG, dVG, each [B,H,N,d_k] (float64)."""
    Q, KL, VL, KG, VG = (_f64(P[k]) for k in ("Q", "KL", "VL", "KG", "VG"))
    dO = _f64(dO)
    B, H, N, d_k = Q.shape
    assert dO.shape == (B, N, H * d_k)
    g = {k: np.zeros((B, H, N, d_k)) for k in ("dQ", "dKL", "dVL", "dKG", "dVG")}
    rc = _load().dar_oracle_attend_backward(_p(Q), _p(KL), _p(VL), _p(KG), _p(VG), _p(dO), B, N,
                                            H, d_k, int(w), _p(g["dQ"]), _p(g["dKL"]),
                                            _p(g["dVL"]), _p(g["dKG"]), _p(g["dVG"]))
    if rc != 0:
        raise ValueError("dar_oracle_attend_backward rejected its arguments")
    return g


def prefill(inp, H, d_k, w, pos0=0, base=10000.0, act="linear"):
    """Whole forward pass: projections then attention.  Returns (o, rowsum, projections)."""
    P = project(inp["h"], inp["W_down"], inp["W_up"], inp["W_Q"], inp["W_K"], inp["W_V"],
                H, d_k, pos0=pos0, base=base, act=act)
    o, rs = attend(P, w)
    return o, rs, P


def decode(q, K_win, V_win, hD, W_up, W_K, W_V, ctx, w, base=10000.0, heads=None):
    """Mixed-cache decode at position ctx-1.  q [B,H,d_k]; K_win/V_win [B,H,w,d_k];
    hD [B,cap,d_down].  Returns o [B, H*d_k] (heads outside ``heads`` are zero)."""
    q, hD, W_up, W_K, W_V = map(_f64, (q, hD, W_up, W_K, W_V))
    B, H, d_k = q.shape
    cap, d_down = hD.shape[1], hD.shape[2]
    d = W_up.shape[1]
    if w > 0:
        K_win, V_win = _f64(K_win), _f64(V_win)
        assert K_win.shape == V_win.shape == (B, H, w, d_k)
    else:
        K_win = V_win = np.zeros(1)
    lo, hi = (0, H) if heads is None else heads
    o = np.zeros((B, H * d_k))
    rc = _load().dar_oracle_decode(_p(q), _p(K_win), _p(V_win), _p(hD), _p(W_up), _p(W_K),
                                   _p(W_V), B, int(ctx), cap, H, d_k, d_down, d, int(w),
                                   float(base), lo, hi, _p(o))
    if rc != 0:
        raise ValueError("dar_oracle_decode rejected its arguments (rc=%d)" % rc)
    return o


# ---------------------------------------------------------------- decoupled RoPE
def project_drope(h, W_down, W_up, W_Q, W_K, W_V, W_QR, W_KR, H, d_k, d_R, pos0=0,
                  base=10000.0, n_tok=None, heads=None):
    """Projections of the decoupled-RoPE variant.  Returns dict hD, hp, QC, QR,
    KL, VL, KG, VG, KR (float64): content parts and values [B,H,N,d_k], rotary
    queries QR [B,H,N,d_R], rotary keys KR [B,N,d_R] (one per token)."""
    h, W_down, W_up, W_Q, W_K, W_V = map(_f64, (h, W_down, W_up, W_Q, W_K, W_V))
    B, N, d = h.shape
    d_down = W_down.shape[1]
    W_QR = _f64(W_QR) if d_R else np.zeros((d, 0))
    W_KR = _f64(W_KR) if d_R else np.zeros((d, 0))
    assert W_QR.shape == (d, H * d_R) and W_KR.shape == (d, d_R)
    n_tok = N if n_tok is None else int(n_tok)
    lo, hi = (0, H) if heads is None else heads
    out = dict(hD=np.zeros((B, N, d_down)), hp=np.zeros((B, N, d)),
               QR=np.zeros((B, H, N, d_R)), KR=np.zeros((B, N, d_R)))
    for k in ("QC", "KL", "VL", "KG", "VG"):
        out[k] = np.zeros((B, H, N, d_k))
    z = np.zeros(1)
    rc = _load().dar_oracle_project_drope(
        _p(h), _p(W_down), _p(W_up), _p(W_Q), _p(W_K), _p(W_V),
        _p(W_QR) if d_R else _p(z), _p(W_KR) if d_R else _p(z), B, N, d, d_down, H, d_k, d_R,
        int(pos0), float(base), n_tok, lo, hi, _p(out["hD"]), _p(out["hp"]), _p(out["QC"]),
        _p(out["QR"]) if d_R else _p(z), _p(out["KL"]), _p(out["VL"]), _p(out["KG"]),
        _p(out["VG"]), _p(out["KR"]) if d_R else _p(z))
    if rc != 0:
        raise ValueError("dar_oracle_project_drope rejected its arguments")
    return out


def attend_drope(P, w):
    """Attention of the decoupled-RoPE variant for every row.  P holds QC, QR,
    KL, VL, KG, VG, KR.  Returns (o [B,N,H*d_k], rowsum [B,H,N])."""
    QC, KL, VL, KG, VG = (_f64(P[k]) for k in ("QC", "KL", "VL", "KG", "VG"))
    B, H, N, d_k = QC.shape
    QR, KR = _f64(P["QR"]), _f64(P["KR"])
    d_R = QR.shape[-1]
    assert QR.shape == (B, H, N, d_R) and KR.shape == (B, N, d_R)
    o = np.zeros((B, N, H * d_k))
    rs = np.zeros((B, H, N))
    z = np.zeros(1)
    rc = _load().dar_oracle_attend_drope(_p(QC), _p(QR) if d_R else _p(z), _p(KL), _p(VL),
                                         _p(KG), _p(VG), _p(KR) if d_R else _p(z), B, N, H, d_k,
                                         d_R, int(w), _p(o), _p(rs))
    if rc != 0:
        raise ValueError("dar_oracle_attend_drope rejected its arguments")
    return o, rs


def prefill_drope(inp, H, d_k, d_R, w, pos0=0, base=10000.0):
    """Whole forward pass of the variant.  Returns (o, rowsum, projections)."""
    P = project_drope(inp["h"], inp["W_down"], inp["W_up"], inp["W_Q"], inp["W_K"], inp["W_V"],
                      inp.get("W_QR"), inp.get("W_KR"), H, d_k, d_R, pos0=pos0, base=base)
    o, rs = attend_drope(P, w)
    return o, rs, P


def decode_drope(qC, qR, K_win, V_win, KR, hD, W_up, W_K, W_V, ctx, w, heads=None):
    """Decode step of the variant at position ctx-1 over its cache.  qC [B,H,d_k],
    qR [B,H,d_R]; K_win/V_win [B,H,w,d_k] (content keys, values); KR [B,cap,d_R]
    (rotary keys of every position); hD [B,cap,d_down].  Returns o [B, H*d_k]."""
    qC, hD, W_up, W_K, W_V = map(_f64, (qC, hD, W_up, W_K, W_V))
    B, H, d_k = qC.shape
    qR, KR = _f64(qR), _f64(KR)
    d_R = qR.shape[-1]
    cap, d_down = hD.shape[1], hD.shape[2]
    d = W_up.shape[1]
    assert KR.shape == (B, cap, d_R)
    if w > 0:
        K_win, V_win = _f64(K_win), _f64(V_win)
        assert K_win.shape == V_win.shape == (B, H, w, d_k)
    else:
        K_win = V_win = np.zeros(1)
    lo, hi = (0, H) if heads is None else heads
    o = np.zeros((B, H * d_k))
    z = np.zeros(1)
    rc = _load().dar_oracle_decode_drope(_p(qC), _p(qR) if d_R else _p(z), _p(K_win),
                                         _p(V_win), _p(KR) if d_R else _p(z), _p(hD), _p(W_up),
                                         _p(W_K), _p(W_V), B, int(ctx), cap, H, d_k, d_R, d_down,
                                         d, int(w), lo, hi, _p(o))
    if rc != 0:
        raise ValueError("dar_oracle_decode_drope rejected its arguments (rc=%d)" % rc)
    return o
