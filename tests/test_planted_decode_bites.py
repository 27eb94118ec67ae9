"""The planted long-context decode inputs (tests/planted.py) make the GPU
decode test at B16, context 32768 able to see the mistakes it exists for.

Against the oracle's output for one planted (batch, head) pair, each of the
following wrong decodes moves o by more than 4x the 2e-2 tolerance: the
window part dropped, every global key rotated one position too far, the
first, second or last 2016-token chunk of latents dropped.  The wrong decodes
are plain numpy (fp64) re-computations of Eqs. 2-4 with one step broken; the
unbroken one matches the oracle to 1e-12, so the comparison is between
like and like."""
import numpy as np
import pytest

import dar_inputs as di
import oracle
import planted

TOL = 2e-2


@pytest.fixture(scope="module")
def case():
    B, ctx, d, H, d_k, dd, w = 16, 32768, 2048, 16, 128, 256, 512
    inp = di.decode_inputs(B, ctx, d, H, d_k, dd, w, seed0=5000)
    b, a = 4, 7
    P = planted.plant(inp, ctx, w, d_k, [(b, a)], *planted_positions(ctx, w))
    return P, b, a, ctx, w, d_k


def planted_positions(ctx, w, n_chunks=16):
    p = ctx - 1
    ch = (ctx - w) // n_chunks
    glob = [0, ch - 1, ch, 7 * ch + 5, 15 * ch - 1, 15 * ch, p - w]
    win = [p - w + 1, p - 200, p]
    return glob, win


def _numpy_decode(P, b, a, ctx, w, d_k, shift=0.0, drop=None):
    p = ctx - 1
    hD = P["h_D"][b, :p - w + 1]
    Wk = P["W_up"] @ P["W_K"][:, a * d_k:(a + 1) * d_k]
    Wv = P["W_up"] @ P["W_V"][:, a * d_k:(a + 1) * d_k]
    h = d_k // 2
    th = 10000.0 ** (-2.0 * np.arange(h) / d_k)
    pos = np.arange(p - w + 1)[:, None] + shift
    c, s = np.cos(pos * th), np.sin(pos * th)
    k0 = hD @ Wk
    KG = np.concatenate([k0[:, :h] * c - k0[:, h:] * s, k0[:, :h] * s + k0[:, h:] * c], 1)
    wp = np.arange(p - w + 1, p + 1)
    K = np.concatenate([KG, P["K_win"][b, a, wp % w]])
    V = np.concatenate([hD @ Wv, P["V_win"][b, a, wp % w]])
    keep = np.ones(len(K), bool)
    if drop is not None:
        keep[drop[0]:drop[1]] = False
    sc = K[keep] @ P["q"][b, a] / np.sqrt(d_k)
    e = np.exp(sc - sc.max())
    return (e / e.sum()) @ V[keep]


def test_planted_decode_mistakes_exceed_tolerance(case):
    P, b, a, ctx, w, d_k = case
    ref = oracle.decode(P["q"][b:b + 1], P["K_win"][b:b + 1], P["V_win"][b:b + 1],
                        P["h_D"][b:b + 1], P["W_up"], P["W_K"], P["W_V"], ctx, w,
                        heads=(a, a + 1))[0, a * d_k:(a + 1) * d_k]
    assert np.abs(ref).max() > 0.5  # o is of order 1, not ~0.01
    assert np.abs(_numpy_decode(P, b, a, ctx, w, d_k) - ref).max() < 1e-12
    p = ctx - 1
    ch = (ctx - w) // 16
    wrong = {"window dropped": dict(drop=(p - w + 1, p + 1)),
             "global RoPE one position off": dict(shift=1.0),
             "chunk 0 dropped": dict(drop=(0, ch)),
             "chunk 1 dropped": dict(drop=(ch, 2 * ch)),
             "last chunk dropped": dict(drop=(15 * ch, 16 * ch))}
    for name, kw in wrong.items():
        moved = np.abs(_numpy_decode(P, b, a, ctx, w, d_k, **kw) - ref).max()
        assert moved > 4 * TOL, (name, moved)
