"""Pins of the fp64 oracle against facts the DAR paper and mathematics fix.

Paper: "Dual Dimensionality for Local and Global Attention" (Eqs. 1-4).
Each pin is chosen so that a plausible slip in the oracle (a dropped term,
the wrong branch of Eq. 3, a sign or index error in RoPE, a transposed
weight) fails at least one of them.  None of them re-types the oracle's
loops: they use an independent brute force (complex-number RoPE, per-query
key lists), a library attention routine, closed forms or hand values.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import dar_inputs as di
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dar_hand_cases.json")


def _inputs(B, N, d, H, d_k, d_down, seed, dtype="f32"):
    return di.prefill_inputs(B, N, d, H, d_k, d_down, dtype=dtype, seed0=seed)


def _sdpa(Q, K, V):
    """Causal softmax attention from torch (fp64, CPU): o [B, N, H*d_k]."""
    o = F.scaled_dot_product_attention(torch.from_numpy(Q), torch.from_numpy(K),
                                       torch.from_numpy(V), is_causal=True).numpy()
    B, H, N, d_k = o.shape
    return o.transpose(0, 2, 1, 3).reshape(B, N, H * d_k)


# ---------------------------------------------------------------- brute force
def _brute(inp, H, d_k, w, pos0=0, base=10000.0):
    """Independent plain-Python reading of Eqs. 1-4 for tiny inputs.

    RoPE is written with complex numbers (pair t, t+d_k/2 as re/im, turned by
    e^{i p theta_t}); for every query i the key list K_i is rebuilt from the
    hidden states, as Eq. 4 writes it."""
    h = inp["h"].tolist()
    Wd, Wu, WQ, WK, WV = (inp[k].tolist() for k in ("W_down", "W_up", "W_Q", "W_K", "W_V"))
    B, N, d = len(h), len(h[0]), len(h[0][0])
    dd = len(Wd[0])

    def row_times(x, W, cols):
        return [sum(x[k] * W[k][c] for k in range(len(x))) for c in cols]

    def rot(x, p):
        half = d_k // 2
        out = [0.0] * d_k
        for t in range(half):
            z = complex(x[t], x[t + half]) * cmath.exp(1j * p * base ** (-2.0 * t / d_k))
            out[t], out[t + half] = z.real, z.imag
        return out

    o = np.zeros((B, N, H * d_k))
    for b in range(B):
        hp = []
        for j in range(N):
            hD = row_times(h[b][j], Wd, range(dd))
            hp.append(row_times(hD, Wu, range(d)))
        for a in range(H):
            cols = range(a * d_k, (a + 1) * d_k)
            for i in range(N):
                q = rot(row_times(h[b][i], WQ, cols), pos0 + i)
                Ki, Vi = [], []
                for j in range(i + 1):
                    src = h[b][j] if i - j < w else hp[j]
                    Ki.append(rot(row_times(src, WK, cols), pos0 + j))
                    Vi.append(row_times(src, WV, cols))
                s = [sum(qq * kk for qq, kk in zip(q, k)) / math.sqrt(d_k) for k in Ki]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                Z = sum(e)
                for t in range(d_k):
                    o[b, i, a * d_k + t] = sum(e[j] * Vi[j][t] for j in range(i + 1)) / Z
    return o


@pytest.mark.parametrize("N,d,H,d_k,d_down,w,pos0", [
    (1, 4, 1, 2, 2, 0, 0),
    (5, 4, 2, 2, 1, 0, 0),
    (5, 6, 1, 4, 3, 1, 3),
    (8, 4, 2, 2, 2, 3, 0),
    (8, 6, 1, 6, 2, 4, 7),
    (7, 4, 1, 4, 4, 100, 0),
    (8, 8, 2, 4, 3, 2, 11),
])
def test_oracle_matches_bruteforce(N, d, H, d_k, d_down, w, pos0):
    inp = _inputs(2, N, d, H, d_k, d_down, seed=10 * N + w)
    o, _, _ = oracle.prefill(inp, H, d_k, w, pos0=pos0)
    ref = _brute(inp, H, d_k, w, pos0=pos0)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- golden
def test_golden_hand_cases():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        arr = {k: np.array(c[k], dtype=np.float64) for k in
               ("W_down", "W_up", "W_Q", "W_K", "W_V")}
        arr["h"] = np.array(c["h"], dtype=np.float64)[None]
        if "expected_o" in c and isinstance(c["expected_o"], dict):
            for w, exp in c["expected_o"].items():
                o, _, _ = oracle.prefill(arr, c["H"], c["d_k"], int(w))
                np.testing.assert_allclose(o[0], np.array(exp), atol=1e-14, err_msg=c["name"])
        if "expected_Q" in c:
            P = oracle.project(arr["h"], arr["W_down"], arr["W_up"], arr["W_Q"], arr["W_K"],
                               arr["W_V"], c["H"], c["d_k"])
            np.testing.assert_allclose(P["Q"][0, 0], np.array(c["expected_Q"]), atol=1e-15)
            np.testing.assert_allclose(P["KL"][0, 0], np.array(c["expected_Q"]), atol=1e-15)
        if "expected_o" in c and isinstance(c["expected_o"], list):
            o, _, _ = oracle.prefill(arr, c["H"], c["d_k"], c["w"])
            np.testing.assert_allclose(o[0], np.array(c["expected_o"]), atol=1e-14,
                                       err_msg=c["name"])


# ---------------------------------------------------------------- special cases
@pytest.mark.parametrize("w_factor", [1, 3])
def test_window_covering_sequence_is_vanilla(w_factor):
    """w >= N: every pair takes the full-state branch -> causal RoPE attention."""
    B, N, d, H, d_k, dd = 2, 37, 32, 2, 8, 8
    inp = _inputs(B, N, d, H, d_k, dd, seed=77)
    o, _, P = oracle.prefill(inp, H, d_k, w=N * w_factor)
    np.testing.assert_allclose(o, _sdpa(P["Q"], P["KL"], P["VL"]), atol=1e-12)


@pytest.mark.parametrize("w", [0, 1, 7, 33])
def test_identity_bottleneck_is_vanilla(w):
    """d_down = d with W_down = W_up = I: h' = h, so both branches agree for any w."""
    B, N, d, H, d_k = 1, 29, 16, 2, 8
    inp = _inputs(B, N, d, H, d_k, d, seed=78)
    inp["W_down"] = np.eye(d)
    inp["W_up"] = np.eye(d)
    o, _, P = oracle.prefill(inp, H, d_k, w=w)
    np.testing.assert_allclose(o, _sdpa(P["Q"], P["KL"], P["VL"]), atol=1e-12)


def test_zero_window_is_uniform_reduction():
    """w = 0: every pair, j = i included, goes through the bottleneck (the paper's
    uniform-reduction baseline)."""
    B, N, d, H, d_k, dd = 2, 31, 32, 2, 8, 4
    inp = _inputs(B, N, d, H, d_k, dd, seed=79)
    o, _, P = oracle.prefill(inp, H, d_k, w=0)
    np.testing.assert_allclose(o, _sdpa(P["Q"], P["KG"], P["VG"]), atol=1e-12)
    # and the global keys really are built from (h W_down) W_up
    hp = inp["h"] @ inp["W_down"] @ inp["W_up"]
    np.testing.assert_allclose(P["hp"], hp, atol=1e-12)


def test_rows_inside_window_are_vanilla():
    """Rows i < w see only local pairs, so they equal vanilla rows."""
    B, N, d, H, d_k, dd, w = 1, 40, 16, 2, 8, 4, 13
    inp = _inputs(B, N, d, H, d_k, dd, seed=80)
    o, _, P = oracle.prefill(inp, H, d_k, w=w)
    ref = _sdpa(P["Q"], P["KL"], P["VL"])
    np.testing.assert_allclose(o[:, :w], ref[:, :w], atol=1e-12)
    assert np.abs(o[:, w:] - ref[:, w:]).max() > 1e-3  # later rows do use the bottleneck


def test_rowsum_is_one():
    B, N, d, H, d_k, dd = 2, 50, 32, 4, 8, 8
    inp = _inputs(B, N, d, H, d_k, dd, seed=81)
    _, rs, _ = oracle.prefill(inp, H, d_k, w=9)
    np.testing.assert_allclose(rs, 1.0, atol=1e-12)


@pytest.mark.parametrize("w", [0, 1, 5, 64])
def test_zero_query_gives_mean_of_selected_values(w):
    """W_Q = 0: all scores are 0, so o_i = (1/(i+1)) * sum_{j<=i} v_j with v_j
    from h_j (i - j < w) or from (h_j W_down) W_up otherwise (Eq. 3)."""
    B, N, d, H, d_k, dd = 2, 21, 16, 2, 4, 4
    inp = _inputs(B, N, d, H, d_k, dd, seed=82)
    inp["W_Q"] = np.zeros_like(inp["W_Q"])
    o, _, _ = oracle.prefill(inp, H, d_k, w=w)
    vl = inp["h"] @ inp["W_V"]
    vg = (inp["h"] @ inp["W_down"] @ inp["W_up"]) @ inp["W_V"]
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    causal = j <= i
    loc = causal & (i - j < w)
    glob = causal & ~(i - j < w)
    ref = (np.einsum("ij,bjc->bic", loc.astype(float), vl) +
           np.einsum("ij,bjc->bic", glob.astype(float), vg)) / (i + 1)
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_rope_dk2_is_rotation_by_position():
    """d_k = 2: one frequency (theta_0 = 1), so q_p is h_p W_Q turned by p radians."""
    B, N, d = 1, 9, 6
    inp = _inputs(B, N, d, 1, 2, 3, seed=83)
    P = oracle.project(inp["h"], inp["W_down"], inp["W_up"], inp["W_Q"], inp["W_K"],
                       inp["W_V"], 1, 2, pos0=4)
    x = inp["h"][0] @ inp["W_Q"]
    p = 4 + np.arange(N)
    ref = np.stack([x[:, 0] * np.cos(p) - x[:, 1] * np.sin(p),
                    x[:, 0] * np.sin(p) + x[:, 1] * np.cos(p)], axis=1)
    np.testing.assert_allclose(P["Q"][0, 0], ref, atol=1e-12)


def test_rope_norm_and_frequencies():
    """Each pair (t, t+d_k/2) keeps its length; at p = 1 pair t turns by base^(-2t/d_k)."""
    d, d_k = 16, 8
    inp = _inputs(1, 2, d, 1, d_k, 4, seed=84)
    P = oracle.project(inp["h"], inp["W_down"], inp["W_up"], inp["W_Q"], inp["W_K"],
                       inp["W_V"], 1, d_k, base=10000.0)
    x = inp["h"][0, 1] @ inp["W_Q"]
    y = P["Q"][0, 0, 1]
    half = d_k // 2
    for t in range(half):
        zx = complex(x[t], x[t + half])
        zy = complex(y[t], y[t + half])
        assert abs(abs(zx) - abs(zy)) < 1e-12
        ang = cmath.phase(zy / zx)
        assert abs(ang - 10000.0 ** (-2.0 * t / d_k)) < 1e-12


def test_position_shift_invariance():
    """q and k both rotated: o depends on i - j only, so shifting every position by
    a constant leaves o unchanged."""
    B, N, d, H, d_k, dd = 1, 33, 32, 2, 16, 8
    inp = _inputs(B, N, d, H, d_k, dd, seed=85)
    o0, _, _ = oracle.prefill(inp, H, d_k, w=6, pos0=0)
    o1, _, _ = oracle.prefill(inp, H, d_k, w=6, pos0=1234)
    np.testing.assert_allclose(o0, o1, atol=1e-11)


def test_value_linearity():
    B, N, d, H, d_k, dd = 1, 25, 16, 2, 8, 4
    inp = _inputs(B, N, d, H, d_k, dd, seed=86)
    o0, _, _ = oracle.prefill(inp, H, d_k, w=5)
    inp2 = dict(inp)
    inp2["W_V"] = inp["W_V"] * -2.5
    o1, _, _ = oracle.prefill(inp2, H, d_k, w=5)
    np.testing.assert_allclose(o1, -2.5 * o0, atol=1e-12)


def test_head_split_is_column_slices():
    """Head a of an H-head layer equals a 1-head layer built from columns S_a."""
    B, N, d, H, d_k, dd = 1, 17, 16, 3, 4, 4
    inp = _inputs(B, N, d, H, d_k, dd, seed=87)
    o, _, _ = oracle.prefill(inp, H, d_k, w=3)
    for a in range(H):
        sl = slice(a * d_k, (a + 1) * d_k)
        one = dict(inp, W_Q=inp["W_Q"][:, sl], W_K=inp["W_K"][:, sl], W_V=inp["W_V"][:, sl])
        o1, _, _ = oracle.prefill(one, 1, d_k, w=3)
        np.testing.assert_allclose(o[..., sl], o1, atol=1e-13)


def test_rows_subset_matches_all_rows():
    B, N, d, H, d_k, dd = 2, 30, 16, 2, 8, 4
    inp = _inputs(B, N, d, H, d_k, dd, seed=88)
    o, rs, P = oracle.prefill(inp, H, d_k, w=4)
    rows = [(0, 0, 0), (1, 1, 29), (0, 1, 17), (1, 0, 4)]
    orow, rsr = oracle.attend_rows(P, 4, rows)
    for r, (b, a, i) in enumerate(rows):
        np.testing.assert_array_equal(orow[r], o[b, i, a * d_k:(a + 1) * d_k])


# ---------------------------------------------------------------- decode oracle
def _cache_from_prefill(P, w, ctx):
    """Mixed cache for the query at p = ctx - 1 from oracle projections:
    ring slot (j mod w) holds position j for the w most recent positions."""
    B, H, N, d_k = P["Q"].shape
    p = ctx - 1
    K_win = np.zeros((B, H, max(w, 1), d_k))
    V_win = np.zeros((B, H, max(w, 1), d_k))
    for j in range(max(0, p - w + 1), p + 1):
        K_win[:, :, j % w] = P["KL"][:, :, j]
        V_win[:, :, j % w] = P["VL"][:, :, j]
    return P["Q"][:, :, p], K_win[:, :, :w], V_win[:, :, :w], P["hD"]


@pytest.mark.parametrize("ctx,w", [(40, 8), (40, 1), (40, 0), (40, 39), (40, 40), (40, 64),
                                   (23, 5)])
def test_decode_oracle_equals_prefill_row(ctx, w):
    B, d, H, d_k, dd = 2, 32, 2, 8, 8
    inp = _inputs(B, ctx, d, H, d_k, dd, seed=89)
    o, _, P = oracle.prefill(inp, H, d_k, w=w)
    q, Kw, Vw, hD = _cache_from_prefill(P, w, ctx)
    od = oracle.decode(q, Kw, Vw, hD, inp["W_up"], inp["W_K"], inp["W_V"], ctx, w)
    np.testing.assert_allclose(od, o[:, ctx - 1], atol=1e-12)
