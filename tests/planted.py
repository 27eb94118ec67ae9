"""Decode inputs whose output depends visibly on every part of the cache.

With the Gaussian cache of the long-context workload a query spreads its
softmax over thousands of keys and |o| stays near 0.01, so a lost window, a
global key rotated at the wrong position or a dropped chunk moves o by less
than the 2e-2 tolerance.  Here a few latent rows and window slots of chosen
(batch, head) pairs are replaced so that their keys point along that head's
query (scores of about 9-11 against a background of N(0, 1)): those keys then
carry most of the softmax weight and their values, of order 1, dominate o.

A global key is k_j = RoPE_j(h^D_j W_up W_K[:, S_a]) (Eqs. 2-3, the oracle's
reading of RoPE: rotate-half pairs, theta_t = base^(-2t/d_k)), so the planted
latent is the least-norm h^D_j with h^D_j W_up W_K[:, S_a] = c RoPE_{-j}(q),
rounded to bf16.  Window slots get k = c q and a value of norm ~ 2.  This
module only builds inputs; expected values come from the oracle.
"""
from __future__ import annotations

import numpy as np

import dar_inputs as di


def _rot(x, pos, base=10000.0):
    d_k = x.shape[-1]
    h = d_k // 2
    th = base ** (-2.0 * np.arange(h) / d_k)
    c, s = np.cos(pos * th), np.sin(pos * th)
    a, b = x[:h], x[h:]
    return np.concatenate([a * c - b * s, a * s + b * c])


def plant(inp, ctx, w, d_k, pairs, glob_pos, win_pos, seed=1):
    """Copy of decode inputs `inp` with planted keys for each (b, head) in
    `pairs`: latent rows at positions `glob_pos` (each <= ctx-1-w) and window
    slots of positions `win_pos` (each > ctx-1-w).  Returns the new dict."""
    out = {k: np.array(v, copy=True) for k, v in inp.items()}
    g = np.random.Generator(np.random.PCG64(seed))
    p = ctx - 1
    for b, a in pairs:
        q = inp["q"][b, a]
        WM = inp["W_up"] @ inp["W_K"][:, a * d_k:(a + 1) * d_k]   # [d_down, d_k]
        pinv = np.linalg.pinv(WM)                                    # [d_k, d_down]
        qq = float(q @ q)
        for n, j in enumerate(glob_pos):
            assert 0 <= j <= p - w
            score = 9.0 + 2.0 * n / max(1, len(glob_pos) - 1)
            c = score * np.sqrt(d_k) / qq
            out["h_D"][b, j] = di.round_bf16(c * _rot(q, -float(j)) @ pinv)
        for n, j in enumerate(win_pos):
            assert p - w < j <= p
            score = 9.5 + n
            c = score * np.sqrt(d_k) / qq
            out["K_win"][b, a, j % w] = di.round_bf16(c * q)
            out["V_win"][b, a, j % w] = di.round_bf16(2.0 * g.standard_normal(d_k))
    return out
