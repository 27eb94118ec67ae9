"""GPU parity of dar_attn_prefill_backward against the fp64 oracle's
backward (oracle.attend_backward), through the C ABI.

Inputs are seeded on the host (Q, K, V in fp16 for the bf16 mode, fp32 for
the fp32 mode; dO in bf16 / fp32) and given to both sides.  The forward
output o that the backward reads comes from dar_attn_prefill on the GPU; the
oracle forms its own o in fp64, so the bf16 rounding of o (2^-9 relative)
enters the GPU's D_i = dO_i . o_i only.  Bounds: with |dO| ~ 1 that moves
D_i by about sqrt(d_k) |o| 2^-9 < 1e-2 and each gradient by that times a
softmax-weighted mean of |k| / sqrt(d_k) or |q| / sqrt(d_k); the rest is fp32
rounding.  The test takes max-abs <= 2e-2 (the bf16 bound of the forward)
plus 2e-3 of the array's largest reference magnitude in bf16 mode (the value
gradients sum p dO over up to N queries), and 1e-4 (plus 1e-5 of it) in
fp32 mode.
"""
import numpy as np
import pytest
import torch

import dar_inputs as di
import distance_adaptive_dual_amd as dar
import oracle
from gpu_helpers import dev, host, log

pytestmark = pytest.mark.gpu

NAMES = (("dQ", "dQ"), ("dK_loc", "dKL"), ("dV_loc", "dVL"), ("dK_glob", "dKG"),
         ("dV_glob", "dVG"))


def _inputs(B, H, N, d_k, seed, mode):
    t = "f16" if mode == "bf16" else "f32"
    sh = (B, H, N, d_k)
    P = {k: di.gaussian(seed + i, sh, 1.0, t) for i, k in enumerate(("Q", "KL", "VL", "KG", "VG"))}
    dO = di.gaussian(seed + 9, (B, N, H * d_k), 1.0, "bf16" if mode == "bf16" else "f32")
    return P, dO


def _gpu(P, dO, w, mode, use_lse=False):
    """Forward then backward on the GPU; with use_lse the backward takes the
    forward's normaliser (dar_attn_prefill_lse) instead of recomputing it."""
    t = "f16" if mode == "bf16" else "f32"
    Q, KL, KG = (dev(P[k], t) for k in ("Q", "KL", "KG"))
    VL = dev(P["VL"].transpose(0, 1, 3, 2), t)
    VG = dev(P["VG"].transpose(0, 1, 3, 2), t)
    lse = None
    if use_lse:
        o, lse = dar.dar_attn_prefill_lse(Q, KL, VL, KG, VG, w)
    else:
        o = dar.dar_attn_prefill(Q, KL, VL, KG, VG, w)
    g = dar.dar_attn_prefill_backward(Q, KL, VL, KG, VG, o, dev(dO, "bf16" if mode == "bf16"
                                                                else "f32"), w, lse=lse)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in g.items()}


def _check(got, ref, mode, tag):
    for gname, rname in NAMES:
        r = ref[rname]
        scale = float(np.abs(r).max())
        tol = (2e-2 + 2e-3 * scale) if mode == "bf16" else (1e-4 + 1e-5 * scale)
        err = float(np.abs(got[gname] - r).max())
        log("  %s %s max err %.3g (max |ref| %.3g)" % (tag, gname, err, scale))
        assert err <= tol, (gname, err, tol)


@pytest.mark.parametrize("B,H,N,d_k,w", [
    (2, 2, 300, 64, 77),     # ragged N, boundary tiles
    (1, 2, 257, 128, 129),   # d_k 128, a tail of one key
    (2, 2, 200, 64, 0),      # w = 0: every pair global
    (1, 2, 190, 128, 1),     # w = 1: only the diagonal is local
    (1, 2, 333, 64, 1000),   # w >= N: every pair local
    (1, 2, 1, 64, 5),        # a single token
    (1, 3, 7, 128, 3),       # shorter than one tile
    (1, 1, 2048, 64, 128),   # one (batch, head) of the Pythia-70M layer
])
def test_backward_bf16(B, H, N, d_k, w):
    P, dO = _inputs(B, H, N, d_k, 300 + N + w, "bf16")
    log("backward bf16 B%d H%d N%d dk%d w%d" % (B, H, N, d_k, w))
    got = _gpu(P, dO, w, "bf16")
    ref = oracle.attend_backward(P, w, dO)
    _check(got, ref, "bf16", "bf16")


def _sweep_cases(n=12, seed=4242):
    """Seeded shapes around the staging boundaries of the MFMA kernels: N not a
    multiple of the 32- or 64-row blocks or of the 128-key/query tiles,
    windows 0, 1, random and >= N, both head widths, with and without lse."""
    g = np.random.Generator(np.random.PCG64(seed))
    out = []
    for k in range(n):
        N = int(g.integers(2, 600))
        d_k = (64, 128)[k % 2]
        w = (0, 1, int(g.integers(2, N + 10)), N + 100)[(k // 2) % 4]
        out.append((int(g.integers(1, 3)), int(g.integers(1, 4)), N, d_k, w, bool(k % 3 == 0)))
    return out


@pytest.mark.parametrize("B,H,N,d_k,w,use_lse", _sweep_cases())
def test_backward_bf16_seeded_sweep(B, H, N, d_k, w, use_lse):
    P, dO = _inputs(B, H, N, d_k, 7100 + N + w, "bf16")
    log("backward sweep B%d H%d N%d dk%d w%d lse=%s" % (B, H, N, d_k, w, use_lse))
    got = _gpu(P, dO, w, "bf16", use_lse=use_lse)
    ref = oracle.attend_backward(P, w, dO)
    _check(got, ref, "bf16", "sweep")


@pytest.mark.parametrize("N,d_k,w", [(200, 64, 50), (150, 128, 40)])
def test_backward_fp32(N, d_k, w):
    P, dO = _inputs(1, 2, N, d_k, 900 + N, "f32")
    log("backward fp32 N%d dk%d w%d" % (N, d_k, w))
    got = _gpu(P, dO, w, "f32")
    ref = oracle.attend_backward(P, w, dO)
    _check(got, ref, "f32", "fp32")


def test_backward_pythia70m_sampled_heads():
    """The whole Pythia-70M-shaped launch (B8 N2048 8 heads of 64, w128);
    two (batch, head) slices checked against the oracle, every slice against
    the softmax invariances (key gradients of both sources sum to zero; value
    gradients sum to the sum of dO)."""
    B, H, N, d_k, w = 8, 8, 2048, 64, 128
    P, dO = _inputs(B, H, N, d_k, 4242, "bf16")
    got = _gpu(P, dO, w, "bf16")
    ks = (got["dK_loc"] + got["dK_glob"]).sum(axis=2)
    vs = (got["dV_loc"] + got["dV_glob"]).sum(axis=2)
    want = dO.reshape(B, N, H, d_k).sum(axis=1)
    log("  invariants: |sum dK| %.3g, |sum dV - sum dO| %.3g" % (np.abs(ks).max(),
                                                                 np.abs(vs - want).max()))
    assert np.abs(ks).max() < 5e-2
    assert np.abs(vs - want).max() < 5e-2
    for b, h in ((0, 0), (7, 5)):
        Ps = {k: P[k][b:b + 1, h:h + 1] for k in P}
        dOs = dO[b:b + 1, :, h * d_k:(h + 1) * d_k]
        ref = oracle.attend_backward(Ps, w, dOs)
        sub = {k: v[b:b + 1, h:h + 1] for k, v in got.items()}
        _check(sub, ref, "bf16", "b%d h%d" % (b, h))


@pytest.mark.parametrize("mode,N,d_k,w", [("bf16", 300, 64, 77), ("bf16", 257, 128, 129),
                                          ("bf16", 200, 64, 0), ("f32", 150, 64, 1000)])
def test_forward_lse_and_backward_from_it(mode, N, d_k, w):
    """dar_attn_prefill_lse: o identical to dar_attn_prefill's, lse against the
    oracle's row normalisers (the bf16 mode sums p rounded to fp16: |error| of
    lse <= log(1 + 2^-11) plus fp32 score rounding, bound 2e-3; fp32 mode 1e-5);
    then the backward fed that lse against the oracle."""
    B, H = 1, 2
    P, dO = _inputs(B, H, N, d_k, 700 + N + w, mode)
    t = "f16" if mode == "bf16" else "f32"
    Q, KL, KG = (dev(P[k], t) for k in ("Q", "KL", "KG"))
    VL = dev(P["VL"].transpose(0, 1, 3, 2), t)
    VG = dev(P["VG"].transpose(0, 1, 3, 2), t)
    o1 = dar.dar_attn_prefill(Q, KL, VL, KG, VG, w)
    o2, lse = dar.dar_attn_prefill_lse(Q, KL, VL, KG, VG, w)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    ref = oracle.attend_lse(P, w)
    err = float(np.abs(host(lse) - ref).max())
    log("lse %s N%d dk%d w%d max err %.3g" % (mode, N, d_k, w, err))
    assert err <= (2e-3 if mode == "bf16" else 1e-5)
    got = _gpu(P, dO, w, mode, use_lse=True)
    _check(got, oracle.attend_backward(P, w, dO), mode, "from lse")


def test_backward_1b_shape_sampled():
    """The 1B-shaped launch (B4 N8192, 16 heads of 128, w512) with the forward's
    lse.  dq_i depends only on keys j <= i, so the first 1024 rows of a sampled
    (batch, head) slice equal the oracle's backward of that slice cut to 1024
    tokens; every slice is checked against the softmax invariances."""
    B, H, N, d_k, w = 4, 16, 8192, 128, 512
    P, dO = _inputs(B, H, N, d_k, 5151, "bf16")
    got = _gpu(P, dO, w, "bf16", use_lse=True)
    ks = (got["dK_loc"] + got["dK_glob"]).sum(axis=2)
    vs = (got["dV_loc"] + got["dV_glob"]).sum(axis=2)
    want = dO.reshape(B, N, H, d_k).sum(axis=1)
    log("  1b invariants: |sum dK| %.3g, |sum dV - sum dO| %.3g" % (np.abs(ks).max(),
                                                                    np.abs(vs - want).max()))
    assert np.abs(ks).max() < 1e-1
    assert np.abs(vs - want).max() < 1e-1
    n = 1024
    for b, h in ((0, 0), (3, 11)):
        Ps = {k: P[k][b:b + 1, h:h + 1, :n] for k in P}
        dOs = dO[b:b + 1, :n, h * d_k:(h + 1) * d_k]
        ref = oracle.attend_backward(Ps, w, dOs)
        err = float(np.abs(got["dQ"][b, h, :n] - ref["dQ"][0, 0]).max())
        scale = float(np.abs(ref["dQ"]).max())
        log("  1b b%d h%d dQ rows < %d max err %.3g (max |ref| %.3g)" % (b, h, n, err, scale))
        assert err <= 2e-2 + 2e-3 * scale
