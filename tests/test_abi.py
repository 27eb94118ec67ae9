"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/dar.h declares, and rejects bad arguments before
any device work.  Only size queries and rejected calls are made here, with
fake, never-dereferenced addresses."""
import ctypes
import os
import re

import pytest

import distance_adaptive_dual_amd as dar

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dar.h")
OK, INVALID, UNSUP, WS = 0, 1, 2, 3


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:dar_status|int|const char\*)\s+(dar_\w+)\s*\(", text,
                                 re.M)))


def test_exports_match_header():
    names = declared()
    assert set(names) == set(dar.EXPORTS)
    L = dar.lib()
    for n in names:
        assert hasattr(L, n), n


def _param_counts(text):
    """Number of parameters of every dar_* declaration in a header."""
    out = {}
    for m in re.finditer(r"^\s*(?:dar_status|int|const char\*)\s+(dar_\w+)\s*\(([^)]*)\)\s*;",
                         text, re.M):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_argtypes_match_header():
    """Every entry point the binding types has as many arguments as the
    header declares (a miscount would shift every later argument)."""
    counts = _param_counts(open(HEADER).read())
    assert set(counts) == set(declared())
    L = dar.lib()
    for n, c in counts.items():
        at = getattr(L, n).argtypes
        assert at is not None, n
        assert len(at) == c, "%s: binding %d, header %d" % (n, len(at), c)


def test_version_and_status_strings():
    L = dar.lib()
    assert L.dar_abi_version() == 2
    for code, name in dar.STATUS.items():
        assert L.dar_status_string(code).decode() == name


F = dar._fake


PROJECT_ENTRIES = ("dar_project", "dar_project_sigmoid")  # same arguments and checks


def project(entry="dar_project", **kw):
    a = dict(h=F(0), W_down=F(1), W_up=F(2), W_Q=F(3), W_K=F(4), W_V=F(5), W_upK=F(6),
             W_upV=F(7), B=2, N=128, d=256, d_down=64, heads=4, d_k=64, pos0=0, base=10000.0,
             dtype=1, Q=F(8), K_loc=F(9), V_loc=F(10), h_D=F(11), K_glob=F(12), V_glob=F(13),
             ws=None, wsb=0)
    a.update(kw)
    n = ctypes.c_size_t(a["wsb"])
    st = getattr(dar.lib(), entry)(a["h"], a["W_down"], a["W_up"], a["W_Q"], a["W_K"], a["W_V"],
                               a["W_upK"], a["W_upV"], a["B"], a["N"], a["d"], a["d_down"],
                               a["heads"], a["d_k"], a["pos0"], a["base"], a["dtype"], a["Q"],
                               a["K_loc"], a["V_loc"], a["h_D"], a["K_glob"], a["V_glob"],
                               a["ws"], ctypes.byref(n), None)
    return st, n.value


@pytest.mark.parametrize("entry", PROJECT_ENTRIES)
def test_project_size_query(entry):
    st, n = project(entry)
    assert st == OK and n > 0
    st2, n2 = project(entry, W_upK=None, W_upV=None)  # fold into the workspace
    assert st2 == OK and n2 > n
    st3, n3 = project(entry, N=4096)                  # longer RoPE table
    assert st3 == OK and n3 > n
    assert (n, n2, n3) == (project()[1], project(W_upK=None, W_upV=None)[1], project(N=4096)[1])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), INVALID), (dict(N=0), INVALID), (dict(d_k=63), INVALID), (dict(pos0=-1), INVALID),
    (dict(h=None), INVALID), (dict(Q=F(8) + 2), INVALID), (dict(dtype=7), INVALID),
    (dict(base=0.5), INVALID),
    (dict(K_glob=F(0)), INVALID),              # output aliases an input
    (dict(V_glob=F(8)), INVALID),              # two outputs alias
    (dict(W_upK=None, W_upV=None, W_up=None), INVALID),
    (dict(d_k=96), UNSUP), (dict(d=200), UNSUP), (dict(d_down=48), UNSUP),
])
@pytest.mark.parametrize("entry", PROJECT_ENTRIES)
def test_project_rejects(entry, kw, code):
    assert project(entry, **kw)[0] == code


@pytest.mark.parametrize("entry", PROJECT_ENTRIES)
def test_project_small_workspace(entry):
    st, n = project(entry)
    assert project(entry, ws=F(20), wsb=n - 1)[0] == WS
    assert project(entry, ws=F(20) + 16, wsb=n)[0] == INVALID  # workspace must be 256-B aligned


def attn(**kw):
    a = dict(Q=F(0), K_loc=F(1), V_loc=F(2), K_glob=F(3), V_glob=F(4), B=1, N=64, heads=2,
             d_k=64, w=8, dtype=1, o=F(5))
    a.update(kw)
    n = ctypes.c_size_t(12345)
    # workspace NULL with a size pointer: the size query, which validates and
    # launches nothing even for a valid problem
    st = dar.lib().dar_attn_prefill(a["Q"], a["K_loc"], a["V_loc"], a["K_glob"], a["V_glob"],
                                    a["B"], a["N"], a["heads"], a["d_k"], a["w"], a["dtype"],
                                    a["o"], None, ctypes.byref(n), None)
    assert st != OK or n.value == 0
    return st


def test_prefill_size_query():
    assert attn() == OK
    assert attn(dtype=0) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(w=-1), INVALID), (dict(N=0), INVALID), (dict(o=F(0)), INVALID), (dict(Q=None), INVALID),
    (dict(d_k=32), UNSUP),
])
def test_prefill_rejects(kw, code):
    assert attn(**kw) == code


def attn_bwd(**kw):
    a = dict(Q=F(0), K_loc=F(1), V_loc=F(2), K_glob=F(3), V_glob=F(4), o=F(5), dO=F(6),
             lse=None, B=1, N=64, heads=2, d_k=64, w=8, dtype=1, dQ=F(7), dK_loc=F(8),
             dV_loc=F(9), dK_glob=F(10), dV_glob=F(11), ws=None, wsb=0)
    a.update(kw)
    n = ctypes.c_size_t(a["wsb"])
    st = dar.lib().dar_attn_prefill_backward(
        a["Q"], a["K_loc"], a["V_loc"], a["K_glob"], a["V_glob"], a["o"], a["dO"], a["lse"],
        a["B"], a["N"],
        a["heads"], a["d_k"], a["w"], a["dtype"], a["dQ"], a["dK_loc"], a["dV_loc"], a["dK_glob"],
        a["dV_glob"], a["ws"], ctypes.byref(n), None)
    return st, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(lse=None), INVALID), (dict(lse=F(6) + 4), INVALID),  # null or misaligned
    (dict(lse=F(5)), INVALID),                                 # lse overlaps o
    (dict(lse=F(0)), INVALID),                                 # lse overlaps Q
    (dict(N=0), INVALID), (dict(d_k=32), UNSUP),
])
def test_prefill_lse_rejects(kw, code):
    a = dict(Q=F(0), K_loc=F(1), V_loc=F(2), K_glob=F(3), V_glob=F(4), B=1, N=64, heads=2,
             d_k=64, w=8, dtype=1, o=F(5), lse=F(6))
    a.update(kw)
    st = dar.lib().dar_attn_prefill_lse(a["Q"], a["K_loc"], a["V_loc"], a["K_glob"], a["V_glob"],
                                        a["B"], a["N"], a["heads"], a["d_k"], a["w"], a["dtype"],
                                        a["o"], a["lse"], None)
    assert st == code


def test_backward_size_query():
    st, n = attn_bwd()
    assert st == OK and n == 2 * 512  # lse and D: 4 bytes per (b, head, query), 256-B rounded
    assert attn_bwd(N=1000, heads=4, B=3)[1] == 2 * ((4 * 3 * 4 * 1000 + 255) // 256 * 256)


@pytest.mark.parametrize("kw,code", [
    (dict(w=-1), INVALID), (dict(N=0), INVALID), (dict(dO=None), INVALID),
    (dict(dQ=F(0)), INVALID),          # gradient aliases an input
    (dict(dV_glob=F(7)), INVALID),     # two gradients alias
    (dict(o=F(5) + 8), INVALID),       # misaligned
    (dict(lse=F(12) + 2), INVALID),    # misaligned lse
    (dict(lse=F(7)), INVALID),         # lse overlaps a gradient
    (dict(dtype=3), INVALID), (dict(d_k=96), UNSUP),
])
def test_backward_rejects(kw, code):
    assert attn_bwd(**kw)[0] == code


def test_backward_workspace_checks():
    _, n = attn_bwd()
    assert attn_bwd(ws=F(20), wsb=n - 1)[0] == WS
    assert attn_bwd(ws=F(20) + 16, wsb=n)[0] == INVALID
    assert attn_bwd(ws=F(7), wsb=n)[0] == INVALID  # workspace overlaps a gradient


def decode(**kw):
    a = dict(q=F(0), K_win=F(1), V_win=F(2), h_D=F(3), W_upK=F(4), W_upV=F(5), B=2, ctx=1000,
             cap=1000, heads=4, d_k=128, d_down=256, w=128, base=10000.0, dtype=1, o=F(6),
             ws=None, wsb=0)
    a.update(kw)
    n = ctypes.c_size_t(a["wsb"])
    st = dar.lib().dar_attn_decode(a["q"], a["K_win"], a["V_win"], a["h_D"], a["W_upK"],
                                   a["W_upV"], a["B"], a["ctx"], a["cap"], a["heads"], a["d_k"],
                                   a["d_down"], a["w"], a["base"], a["dtype"], a["o"], a["ws"],
                                   ctypes.byref(n), None)
    return st, n.value


def test_decode_size_query_and_rejects():
    st, n = decode()
    assert st == OK and n > 0
    assert decode(cap=800)[0] == INVALID        # cache shorter than the latent range
    assert decode(cap=873)[0] == OK             # exactly p - w + 1 rows
    assert decode(w=-1)[0] == INVALID
    assert decode(dtype=0)[0] == UNSUP          # fp32 decode is not provided
    assert decode(d_down=96)[0] == UNSUP
    assert decode(d_down=512)[0] == OK          # two latent slices per frequency block
    assert decode(d_down=1024)[0] == UNSUP
    assert decode(w=0, K_win=None, V_win=None)[0] == OK
    assert decode(ws=F(20), wsb=n - 1)[0] == WS


def decode_noalloc(**kw):
    a = dict(q=F(0), K_win=F(1), V_win=F(2), h_D=F(3), W_upK=F(4), W_upV=F(5), B=2, ctx=1000,
             cap=1000, heads=4, d_k=128, d_down=256, w=128, base=10000.0, dtype=1, o=F(6))
    a.update(kw)
    return dar.lib().dar_attn_decode_noalloc(a["q"], a["K_win"], a["V_win"], a["h_D"],
                                             a["W_upK"], a["W_upV"], a["B"], a["ctx"], a["cap"],
                                             a["heads"], a["d_k"], a["d_down"], a["w"], a["base"],
                                             a["dtype"], a["o"], None)


def test_decode_noalloc_rejects_before_touching_the_device():
    """The allocation-free decode validates like dar_attn_decode, and a problem
    whose workspace would exceed its 32 MiB static scratch returns
    DAR_ERR_WORKSPACE; none of these reaches the device (fake addresses)."""
    assert decode_noalloc(cap=800) == INVALID
    assert decode_noalloc(w=-1) == INVALID
    assert decode_noalloc(o=F(3)) == INVALID     # output aliases the latent cache
    assert decode_noalloc(dtype=0) == UNSUP
    assert decode_noalloc(d_down=96) == UNSUP
    # 5M positions: the RoPE tables alone need ~40 MB
    st, n = decode(ctx=5_000_000, cap=5_000_000)
    assert st == OK and n > (32 << 20)
    assert decode_noalloc(ctx=5_000_000, cap=5_000_000) == WS
    st, n = decode(ctx=1_000_000, cap=1_000_000)
    assert st == OK and n <= (32 << 20)          # a million positions fit


def test_fold_rejects():
    L = dar.lib()
    assert L.dar_fold(F(0), F(1), F(2), 256, 64, 4, 64, 1, F(3), F(0), None) == INVALID
    assert L.dar_fold(F(0), F(1), F(2), 256, 64, 4, 48, 1, F(3), F(4), None) == UNSUP
    assert L.dar_fold(None, F(1), F(2), 256, 64, 4, 64, 1, F(3), F(4), None) == INVALID


def append(**kw):
    a = dict(h=F(0), W_down=F(1), W_Q=F(2), W_K=F(3), W_V=F(4), B=2, d=256, d_down=64,
             heads=4, d_k=64, pos=100, w=16, cap=200, base=10000.0, dtype=1, q=F(5),
             K_win=F(6), V_win=F(7), h_D=F(8), ws=None, wsb=0)
    a.update(kw)
    n = ctypes.c_size_t(a["wsb"])
    st = dar.lib().dar_decode_append(a["h"], a["W_down"], a["W_Q"], a["W_K"], a["W_V"], a["B"],
                                     a["d"], a["d_down"], a["heads"], a["d_k"], a["pos"], a["w"],
                                     a["cap"], a["base"], a["dtype"], a["q"], a["K_win"],
                                     a["V_win"], a["h_D"], a["ws"], ctypes.byref(n), None)
    return st, n.value


def test_append_size_query_and_rejects():
    st, n = append()
    assert st == OK and n > 0
    assert append(pos=200)[0] == INVALID        # position beyond the latent cache
    assert append(pos=-1)[0] == INVALID
    assert append(w=-1)[0] == INVALID
    assert append(q=F(0))[0] == INVALID         # output aliases an input
    assert append(dtype=0)[0] == UNSUP
    assert append(d_k=96)[0] == UNSUP
    assert append(w=0, K_win=None, V_win=None)[0] == OK
    assert append(ws=F(20), wsb=n - 1)[0] == WS


CALIB_HEADER = os.path.join(ROOT, "include", "dar_calib.h")


def test_calib_library_exports_and_rejects():
    """libdar_calib.so (the benchmark's calibration kernels) exports what
    include/dar_calib.h declares and rejects bad arguments before launching."""
    text = open(CALIB_HEADER).read()
    names = set(re.findall(r"^\s*(?:int|double)\s+(dar_\w+)\s*\(", text, re.M))
    assert names == {"dar_calib_mfma_flops", "dar_calib_mfma", "dar_calib_copy", "dar_calib_read",
                     "dar_calib_read_lds"}
    L = ctypes.CDLL(os.path.join(ROOT, "distance_adaptive_dual_amd", "libdar_calib.so"))
    for n in names:
        assert hasattr(L, n), n
    L.dar_calib_mfma_flops.restype = ctypes.c_double
    L.dar_calib_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    assert L.dar_calib_mfma_flops(2, 3, 0) == 2 * 4 * 3 * 4 * 32768
    assert L.dar_calib_mfma_flops(2, 3, 1) == 2 * 4 * 3 * 4 * 16384
    L.dar_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p]
    L.dar_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p]
    assert L.dar_calib_mfma(F(0), 0, 10, 0, None) != 0       # no workgroups
    assert L.dar_calib_mfma(None, 4, 10, 0, None) != 0       # no sink
    assert L.dar_calib_mfma(F(0), 4, 10, 2, None) != 0       # unknown shape
    assert L.dar_calib_copy(F(0), F(1), 100, None) != 0      # not a multiple of 16
    assert L.dar_calib_copy(F(0) + 8, F(1), 64, None) != 0   # misaligned source
    L.dar_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                 ctypes.c_void_p]
    assert L.dar_calib_read(F(0), 100, F(1), None) != 0      # not a multiple of 16
    assert L.dar_calib_read(F(0), 64, None, None) != 0       # no sink
    L.dar_calib_read_lds.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert L.dar_calib_read_lds(F(0), 16000, None) != 0      # not a multiple of 16 KB
    assert L.dar_calib_read_lds(F(0) + 8, 16384, None) != 0  # misaligned source
    assert L.dar_calib_read_lds(None, 16384, None) != 0      # no source


def cache(**kw):
    a = dict(h_D=F(0), K_loc=F(1), V_loc=F(2), B=2, N=100, heads=4, d_k=64, d_down=64, w=16,
             cap=128, dtype=1, h_D_cache=F(3), K_win=F(4), V_win=F(5))
    a.update(kw)
    return dar.lib().dar_cache_from_prefill(a["h_D"], a["K_loc"], a["V_loc"], a["B"], a["N"],
                                            a["heads"], a["d_k"], a["d_down"], a["w"], a["cap"],
                                            a["dtype"], a["h_D_cache"], a["K_win"], a["V_win"],
                                            None)


@pytest.mark.parametrize("kw,code", [
    (dict(cap=99), INVALID),                    # the cache must hold the N prompt rows
    (dict(N=0), INVALID), (dict(w=-1), INVALID), (dict(B=0), INVALID),
    (dict(h_D_cache=F(0)), INVALID),            # output aliases an input
    (dict(K_win=F(3)), INVALID),                # two outputs alias
    (dict(V_win=None), INVALID),                # w > 0 needs the ring
    (dict(h_D=F(0) + 8), INVALID),              # misaligned
    (dict(dtype=0), UNSUP), (dict(d_k=96), UNSUP), (dict(d_down=60), UNSUP),
])
def test_cache_from_prefill_rejects(kw, code):
    assert cache(**kw) == code


def chunk(**kw):
    a = dict(B=2, C=100, d=256, d_down=64, heads=4, d_k=64, p0=300, w=64, cap=512, base=10000.0,
             dtype=1, ring=True, o=F(10), ws=None, wsb=0)
    a.update(kw)
    n = ctypes.c_size_t(a["wsb"])
    f = [F(i) for i in range(10)]
    st = dar.lib().dar_prefill_chunk(*f[:7], a["B"], a["C"], a["d"], a["d_down"], a["heads"],
                                     a["d_k"], a["p0"], a["w"], a["cap"], a["base"], a["dtype"],
                                     f[7], f[8] if a["ring"] else None,
                                     f[9] if a["ring"] else None, a["o"], a["ws"],
                                     ctypes.byref(n), None)
    return st, n.value


def test_chunk_size_query_and_rejects():
    st, n = chunk()
    assert st == OK and n > 0
    assert chunk(p0=400)[0] == OK and chunk(p0=400)[1] > n   # longer prefix, more to rebuild
    assert chunk(w=0, ring=False)[0] == OK                   # no window: no ring needed
    assert chunk(p0=450)[0] == INVALID                       # p0 + C beyond the cache
    assert chunk(p0=-1)[0] == INVALID
    assert chunk(C=0)[0] == INVALID
    assert chunk(ring=False)[0] == INVALID                   # w > 0 needs the ring
    assert chunk(o=F(0))[0] == INVALID                       # output aliases an input
    assert chunk(o=F(7))[0] == INVALID                       # output aliases the cache
    assert chunk(dtype=0)[0] == UNSUP
    assert chunk(d_k=96)[0] == UNSUP
    assert chunk(ws=F(20), wsb=n - 1)[0] == WS


# Ragged-batch entry points: the per-sequence arrays are device int32 [B].
def decode_varlen(**kw):
    a = dict(lens=F(7), max_ctx=1000, cap=1000, w=128, d_down=256, ws=None, wsb=0)
    a.update(kw)
    n = ctypes.c_size_t(a["wsb"])
    st = dar.lib().dar_attn_decode_varlen(F(0), F(1), F(2), F(3), F(4), F(5), 2, a["lens"],
                                          a["max_ctx"], a["cap"], 4, 128, a["d_down"], a["w"],
                                          10000.0, 1, F(6), a["ws"], ctypes.byref(n), None)
    return st, n.value


def test_decode_varlen_size_query_and_rejects():
    st, n = decode_varlen()
    assert st == OK and n == decode()[1]        # sized by the longest context
    assert decode_varlen(lens=None)[0] == INVALID
    assert decode_varlen(lens=F(7) + 2)[0] == INVALID   # misaligned lengths
    assert decode_varlen(lens=F(6))[0] == INVALID        # lengths alias the output
    assert decode_varlen(cap=800)[0] == INVALID
    assert decode_varlen(d_down=96)[0] == UNSUP
    assert decode_varlen(ws=F(20), wsb=n - 1)[0] == WS


def append_varlen(**kw):
    a = dict(pos=F(9), cap=200, w=16, ws=None, wsb=0)
    a.update(kw)
    n = ctypes.c_size_t(a["wsb"])
    st = dar.lib().dar_decode_append_varlen(F(0), F(1), F(2), F(3), F(4), 2, 256, 64, 4, 64,
                                            a["pos"], a["w"], a["cap"], 10000.0, 1, F(5), F(6),
                                            F(7), F(8), a["ws"], ctypes.byref(n), None)
    return st, n.value


def test_append_varlen_size_query_and_rejects():
    st, n = append_varlen()
    assert st == OK and n == append(pos=199)[1]  # tables up to the last cache row
    assert append_varlen(pos=None)[0] == INVALID
    assert append_varlen(pos=F(9) + 1)[0] == INVALID
    assert append_varlen(pos=F(5))[0] == INVALID         # positions alias the q output
    assert append_varlen(ws=F(20), wsb=n - 1)[0] == WS


def cache_varlen(**kw):
    a = dict(lens=F(6), N=100, cap=128)
    a.update(kw)
    return dar.lib().dar_cache_from_prefill_varlen(F(0), F(1), F(2), 2, a["N"], a["lens"], 4, 64,
                                                   64, 16, a["cap"], 1, F(3), F(4), F(5), None)


def test_cache_varlen_rejects():
    # (valid arguments would launch; the CPU suite checks rejections only)
    assert cache_varlen(lens=None) == INVALID
    assert cache_varlen(lens=F(6) + 2) == INVALID
    assert cache_varlen(lens=F(3)) == INVALID           # lengths alias the cache
    assert cache_varlen(cap=99) == INVALID


# ------------------------------------------------------------------ decoupled-RoPE variant
def project_drope(**kw):
    a = dict(h=F(0), W_down=F(1), W_up=F(2), W_Q=F(3), W_K=F(4), W_V=F(5), W_QR=F(6),
             W_KR=F(7), W_upK=None, W_upV=None, B=2, N=128, d=256, d_down=64, heads=4, d_k=64,
             d_R=64, pos0=0, base=10000.0, dtype=1, QC=F(10), QR=F(11), K_loc=F(12),
             V_loc=F(13), h_D=F(14), K_glob=F(15), V_glob=F(16), KR=F(17), ws=None, wsb=0)
    a.update(kw)
    n = ctypes.c_size_t(a["wsb"])
    keys = ("h", "W_down", "W_up", "W_Q", "W_K", "W_V", "W_QR", "W_KR", "W_upK", "W_upV", "B",
            "N", "d", "d_down", "heads", "d_k", "d_R", "pos0", "base", "dtype", "QC", "QR",
            "K_loc", "V_loc", "h_D", "K_glob", "V_glob", "KR", "ws")
    st = dar.lib().dar_project_drope(*[a[k] for k in keys], ctypes.byref(n), None)
    return st, n.value


def test_project_drope_size_query_and_rejects():
    st, n = project_drope()
    assert st == OK and n > 0                     # RoPE tables and the fold
    st2, n2 = project_drope(W_upK=F(8), W_upV=F(9))
    assert st2 == OK and n2 < n                   # folded weights given: tables only
    assert project_drope(W_upK=F(8))[0] == INVALID  # one folded weight without the other
    assert project_drope(d_R=63)[0] == INVALID
    assert project_drope(d_R=32)[0] == UNSUP      # rotary width 64 only
    assert project_drope(d_k=96)[0] == UNSUP
    assert project_drope(dtype=0)[0] == UNSUP
    assert project_drope(KR=F(0))[0] == INVALID   # output aliases h
    assert project_drope(ws=F(30), wsb=n - 1)[0] == WS


def prefill_drope(**kw):
    a = dict(QC=F(0), QR=F(1), K_loc=F(2), V_loc=F(3), K_glob=F(4), V_glob=F(5), KR=F(6), B=2,
             N=128, heads=4, d_k=128, d_R=64, w=32, dtype=1, o=F(7))
    a.update(kw)
    keys = ("QC", "QR", "K_loc", "V_loc", "K_glob", "V_glob", "KR", "B", "N", "heads", "d_k",
            "d_R", "w", "dtype", "o")
    return dar.lib().dar_attn_prefill_drope(*[a[k] for k in keys], None)


def test_prefill_drope_rejects():
    assert prefill_drope(w=-1) == INVALID
    assert prefill_drope(N=0) == INVALID
    assert prefill_drope(o=F(6)) == INVALID      # output aliases the rotary keys
    assert prefill_drope(QR=F(1) + 8) == INVALID  # misaligned
    assert prefill_drope(dtype=0) == UNSUP
    assert prefill_drope(d_R=128) == UNSUP
    assert prefill_drope(d_k=256) == UNSUP


def append_drope(**kw):
    a = dict(h=F(0), W_down=F(1), W_Q=F(2), W_K=F(3), W_V=F(4), W_QR=F(5), W_KR=F(6), B=2,
             d=256, d_down=64, heads=4, d_k=64, d_R=64, pos=100, w=16, cap=200, base=10000.0,
             dtype=1, qC=F(7), qR=F(8), K_win=F(9), V_win=F(10), h_D=F(11), KR=F(12), ws=None,
             wsb=0)
    a.update(kw)
    n = ctypes.c_size_t(a["wsb"])
    keys = ("h", "W_down", "W_Q", "W_K", "W_V", "W_QR", "W_KR", "B", "d", "d_down", "heads",
            "d_k", "d_R", "pos", "w", "cap", "base", "dtype", "qC", "qR", "K_win", "V_win", "h_D",
            "KR", "ws")
    st = dar.lib().dar_decode_append_drope(*[a[k] for k in keys], ctypes.byref(n), None)
    return st, n.value


def test_append_drope_size_query_and_rejects():
    st, n = append_drope()
    assert st == OK and n > 0
    assert append_drope(pos=200)[0] == INVALID    # position past the cache
    assert append_drope(w=0, K_win=None, V_win=None)[0] == OK
    assert append_drope(KR=F(11))[0] == INVALID   # rotary keys alias the latent cache
    assert append_drope(d_R=32)[0] == UNSUP
    assert append_drope(dtype=0)[0] == UNSUP
    assert append_drope(ws=F(30), wsb=n - 1)[0] == WS


def cache_drope(**kw):
    a = dict(h_D=F(0), K_loc=F(1), V_loc=F(2), KR=F(3), B=2, N=100, heads=4, d_k=64, d_down=64,
             d_R=64, w=16, cap=128, dtype=1, L=F(4), K_win=F(5), V_win=F(6), KRc=F(7))
    a.update(kw)
    keys = ("h_D", "K_loc", "V_loc", "KR", "B", "N", "heads", "d_k", "d_down", "d_R", "w", "cap",
            "dtype", "L", "K_win", "V_win", "KRc")
    return dar.lib().dar_cache_from_prefill_drope(*[a[k] for k in keys], None)


def test_cache_from_prefill_drope_rejects():
    assert cache_drope(cap=99) == INVALID         # cache shorter than the prompt
    assert cache_drope(KRc=F(3)) == INVALID       # output aliases the input rotary keys
    assert cache_drope(KRc=F(4)) == INVALID       # rotary cache aliases the latent cache
    assert cache_drope(dtype=0) == UNSUP
    assert cache_drope(d_R=32) == UNSUP


def test_pack_weight_rejects():
    L = dar.lib()
    assert L.dar_pack_weight(F(0), 0, 64, 1, F(1), None) == INVALID
    assert L.dar_pack_weight(F(0), 64, 64, 1, F(0) + 4096, None) == INVALID  # overlap
    assert L.dar_pack_weight(F(0) + 8, 64, 64, 1, F(1), None) == INVALID    # misaligned
    assert L.dar_pack_weight(None, 64, 64, 1, F(1), None) == INVALID
    assert L.dar_pack_weight(F(0), 64, 64, 7, F(1), None) == INVALID       # unknown dtype
    assert L.dar_pack_weight(F(0), 64 * 65536, 1, 1, F(1), None) == UNSUP


def project_varlen(**kw):
    a = dict(h=F(0), W_down=F(1), W_up=F(2), W_Q=F(3), W_K=F(4), W_V=F(5), W_upK=F(6), W_upV=F(7),
             cu=F(8), B=3, T=500, max_len=300, d=256, d_down=64, heads=4, d_k=64, base=10000.0,
             dtype=1, Q=F(10), K_loc=F(11), V_loc=F(12), h_D=F(13), K_glob=F(14), V_glob=F(15),
             ws=None, wsb=0)
    a.update(kw)
    n = ctypes.c_size_t(a["wsb"])
    keys = ("h", "W_down", "W_up", "W_Q", "W_K", "W_V", "W_upK", "W_upV", "cu", "B", "T",
            "max_len", "d", "d_down", "heads", "d_k", "base", "dtype", "Q", "K_loc", "V_loc",
            "h_D", "K_glob", "V_glob", "ws")
    st = dar.lib().dar_project_varlen(*[a[k] for k in keys], ctypes.byref(n), None)
    return st, n.value


def test_project_varlen_size_query_and_rejects():
    st, n = project_varlen()
    assert st == OK and n > 0
    assert project_varlen(max_len=501)[0] == INVALID   # longer than the packed batch
    assert project_varlen(max_len=0)[0] == INVALID
    assert project_varlen(cu=None)[0] == INVALID
    assert project_varlen(cu=F(8) + 2)[0] == INVALID   # int32 alignment
    assert project_varlen(cu=F(10))[0] == INVALID      # lengths alias an output
    assert project_varlen(dtype=0)[0] == UNSUP
    assert project_varlen(d_k=96)[0] == UNSUP
    assert project_varlen(ws=F(30), wsb=n - 1)[0] == WS


def attn_varlen(**kw):
    a = dict(Q=F(0), K_loc=F(1), V_loc=F(2), K_glob=F(3), V_glob=F(4), cu=F(5), B=3, T=500,
             max_len=300, heads=4, d_k=64, w=16, dtype=1, o=F(6))
    a.update(kw)
    keys = ("Q", "K_loc", "V_loc", "K_glob", "V_glob", "cu", "B", "T", "max_len", "heads", "d_k",
            "w", "dtype", "o")
    return dar.lib().dar_attn_prefill_varlen(*[a[k] for k in keys], None)


def test_attn_prefill_varlen_rejects():
    assert attn_varlen(w=-1) == INVALID
    assert attn_varlen(max_len=501) == INVALID
    assert attn_varlen(o=F(5)) == INVALID       # output aliases the lengths
    assert attn_varlen(o=F(0)) == INVALID       # output aliases Q
    assert attn_varlen(cu=None) == INVALID
    assert attn_varlen(dtype=0) == UNSUP
    assert attn_varlen(d_k=32) == UNSUP


def cache_packed(**kw):
    a = dict(h_D=F(0), K_loc=F(1), V_loc=F(2), cu=F(3), B=3, T=500, max_len=300, heads=4, d_k=64,
             d_down=64, w=16, cap=320, dtype=1, cache=F(4), K_win=F(5), V_win=F(6))
    a.update(kw)
    keys = ("h_D", "K_loc", "V_loc", "cu", "B", "T", "max_len", "heads", "d_k", "d_down", "w",
            "cap", "dtype", "cache", "K_win", "V_win")
    return dar.lib().dar_cache_from_prefill_packed(*[a[k] for k in keys], None)


def test_cache_from_prefill_packed_rejects():
    assert cache_packed(cap=299) == INVALID        # a prompt of max_len rows would not fit
    assert cache_packed(max_len=501) == INVALID
    assert cache_packed(cu=None) == INVALID
    assert cache_packed(cu=F(3) + 2) == INVALID    # int32 alignment
    assert cache_packed(K_win=F(1)) == INVALID     # ring aliases K_loc
    assert cache_packed(cache=F(3)) == INVALID     # cache aliases the starts
    assert cache_packed(h_D=F(0) + 8) == INVALID   # 16-byte alignment
    assert cache_packed(dtype=0) == UNSUP
    assert cache_packed(d_down=12) == UNSUP
    assert cache_packed(d_k=96) == UNSUP
