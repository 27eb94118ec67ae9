"""Pins of the fp64 oracle's decoupled-RoPE variant (dar_oracle_*_drope).

The DAR paper names MLA's decoupled rotary embedding for efficient
implementations (the paragraph after the inference remark) without writing it
out; the oracle's reading is MLA's construction: per head a content part
(Eq. 3 without rotation) and a rotary part of width d_R, the rotary key
computed once per token from the full hidden state and shared by every head
and both paths, scores over both parts scaled by 1/sqrt(d_k + d_R).  None of
these pins re-types the oracle's loops: they use torch's scaled-dot-product
attention, the identity bottleneck, closed forms (uniform weights; a single
rotary frequency whose score is cos(i - j)), a plain-Python brute force with
complex-number rotation, shift invariance, and the cache form against the
prefill form.
"""
import cmath
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import dar_inputs as di
import oracle


def _inputs(B, N, d, H, d_k, dd, d_R, seed):
    return di.drope_prefill_inputs(B, N, d, H, d_k, dd, d_R, dtype="f32", seed0=seed)


def _sdpa(q, k, v):
    return F.scaled_dot_product_attention(torch.tensor(q), torch.tensor(k), torch.tensor(v),
                                          is_causal=True).numpy()


def _cat_keys(P, src, H):
    KR = np.repeat(P["KR"][:, None], H, axis=1)  # one rotary key per token, every head
    return np.concatenate([P[src], KR], axis=-1)


def _heads_to_o(x):  # [B, H, N, d_k] -> [B, N, H d_k]
    B, H, N, d_k = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B, N, H * d_k)


@pytest.mark.parametrize("d_R", [0, 8, 16])
def test_all_local_and_all_global_are_sdpa(d_R):
    """w >= N: every pair local, plain causal attention with keys [kC; kR] and
    scale 1/sqrt(d_k + d_R) (torch's default for that query width).  w = 0:
    the same over the global content keys and values."""
    B, N, d, H, d_k, dd = 2, 37, 48, 3, 16, 12
    inp = _inputs(B, N, d, H, d_k, dd, d_R, seed=11 + d_R)
    o_loc, rs, P = oracle.prefill_drope(inp, H, d_k, d_R, w=N)
    q = np.concatenate([P["QC"], P["QR"]], axis=-1)
    assert np.abs(o_loc - _heads_to_o(_sdpa(q, _cat_keys(P, "KL", H), P["VL"]))).max() < 1e-12
    assert np.abs(rs - 1).max() < 1e-12
    o_glb, _, _ = oracle.prefill_drope(inp, H, d_k, d_R, w=0)
    assert np.abs(o_glb - _heads_to_o(_sdpa(q, _cat_keys(P, "KG", H), P["VG"]))).max() < 1e-12


def test_identity_bottleneck_is_all_local_for_any_window():
    """d_down = d, W_down = W_up = I: both paths carry the same content keys and
    values, so every window gives the w >= N result."""
    B, N, d, H, d_k, d_R = 1, 30, 32, 2, 16, 8
    inp = _inputs(B, N, d, H, d_k, d, d_R, seed=5)
    inp["W_down"] = np.eye(d)
    inp["W_up"] = np.eye(d)
    ref, _, _ = oracle.prefill_drope(inp, H, d_k, d_R, w=N)
    for w in (0, 1, 7, 29):
        o, _, _ = oracle.prefill_drope(inp, H, d_k, d_R, w=w)
        assert np.abs(o - ref).max() < 1e-12, w


@pytest.mark.parametrize("w", [0, 1, 4, 9])
def test_zero_query_averages_the_selected_values(w):
    """W_Q = W_QR = 0: every score is 0, so o_i is the mean over j <= i of the
    value Eq. 3 selects (local if i - j < w, else global)."""
    B, N, d, H, d_k, dd, d_R = 1, 14, 24, 2, 8, 6, 4
    inp = _inputs(B, N, d, H, d_k, dd, d_R, seed=21 + w)
    inp["W_Q"] = np.zeros_like(inp["W_Q"])
    inp["W_QR"] = np.zeros_like(inp["W_QR"])
    o, _, P = oracle.prefill_drope(inp, H, d_k, d_R, w)
    for i in range(N):
        sel = [P["VL"][:, :, j] if i - j < w else P["VG"][:, :, j] for j in range(i + 1)]
        want = np.mean(sel, axis=0)  # [B, H, d_k]
        assert np.abs(o[:, i] - want.reshape(B, H * d_k)).max() < 1e-12


def test_single_rotary_frequency_scores_cos_of_distance():
    """d_R = 2 has one frequency theta_0 = 1: with no content query and rotary
    projections giving (1, 0) before rotation, q_i . k_j = cos(i) cos(j) +
    sin(i) sin(j) = cos(i - j), so o_i = sum_j softmax_j(cos(i-j)/sqrt(d_k+2)) v_j."""
    B, N, d, H, d_k, dd, d_R = 1, 12, 4, 1, 4, 4, 2
    inp = _inputs(B, N, d, H, d_k, dd, d_R, seed=31)
    inp["h"] = np.zeros((B, N, d))
    inp["h"][..., 0] = 1.0                      # every token's hidden state is e_0
    inp["W_Q"] = np.zeros_like(inp["W_Q"])
    inp["W_QR"] = np.zeros((d, d_R))
    inp["W_QR"][0, 0] = 1.0                     # h W_QR = (1, 0)
    inp["W_KR"] = np.zeros((d, d_R))
    inp["W_KR"][0, 0] = 1.0
    w = 3
    o, _, P = oracle.prefill_drope(inp, H, d_k, d_R, w)
    for i in range(N):
        s = np.array([math.cos(i - j) for j in range(i + 1)]) / math.sqrt(d_k + d_R)
        p = np.exp(s - s.max())
        p /= p.sum()
        v = np.array([P["VL"][0, 0, j] if i - j < w else P["VG"][0, 0, j] for j in range(i + 1)])
        assert np.abs(o[0, i] - p @ v).max() < 1e-12


def _brute(inp, H, d_k, d_R, w, base=10000.0):
    """Plain-Python floats; rotation as multiplication of the complex numbers
    x_t + i x_{t + d_R/2} by exp(i p theta_t)."""
    h, Wd, Wu = inp["h"][0].tolist(), inp["W_down"].tolist(), inp["W_up"].tolist()
    WQ, WK, WV = inp["W_Q"].tolist(), inp["W_K"].tolist(), inp["W_V"].tolist()
    WQR, WKR = inp["W_QR"].tolist(), inp["W_KR"].tolist()
    N, d, dd, half = len(h), len(h[0]), len(Wd[0]), d_R // 2

    def mv(x, W, c0, n):
        return [sum(x[k] * W[k][c0 + c] for k in range(len(x))) for c in range(n)]

    def rot(x, p):
        out = [0.0] * d_R
        for t in range(half):
            z = complex(x[t], x[t + half]) * cmath.exp(1j * p * base ** (-2.0 * t / d_R))
            out[t], out[t + half] = z.real, z.imag
        return out

    o = [[0.0] * (H * d_k) for _ in range(N)]
    hp = [mv(mv(h[n], Wd, 0, dd), Wu, 0, d) for n in range(N)]
    kr = [rot(mv(h[n], WKR, 0, d_R), n) for n in range(N)]
    for a in range(H):
        qc = [mv(h[n], WQ, a * d_k, d_k) for n in range(N)]
        qr = [rot(mv(h[n], WQR, a * d_R, d_R), n) for n in range(N)]
        kl = [mv(h[n], WK, a * d_k, d_k) for n in range(N)]
        vl = [mv(h[n], WV, a * d_k, d_k) for n in range(N)]
        kg = [mv(hp[n], WK, a * d_k, d_k) for n in range(N)]
        vg = [mv(hp[n], WV, a * d_k, d_k) for n in range(N)]
        for i in range(N):
            s, vs = [], []
            for j in range(i + 1):
                kc, v = (kl[j], vl[j]) if i - j < w else (kg[j], vg[j])
                s.append((sum(x * y for x, y in zip(qc[i], kc)) +
                          sum(x * y for x, y in zip(qr[i], kr[j]))) / math.sqrt(d_k + d_R))
                vs.append(v)
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for t in range(d_k):
                o[i][a * d_k + t] = sum(e[j] * vs[j][t] for j in range(i + 1)) / z
    return np.array(o)


@pytest.mark.parametrize("N,w", [(1, 1), (5, 0), (8, 3), (7, 7)])
def test_brute_force_small(N, w):
    H, d, d_k, dd, d_R = 2, 6, 4, 3, 4
    inp = _inputs(1, N, d, H, d_k, dd, d_R, seed=40 + N + w)
    o, _, _ = oracle.prefill_drope(inp, H, d_k, d_R, w)
    assert np.abs(o[0] - _brute(inp, H, d_k, d_R, w)).max() < 1e-12


def test_position_shift_leaves_output_unchanged():
    """Only relative positions enter the rotary scores."""
    B, N, d, H, d_k, dd, d_R = 1, 25, 32, 2, 8, 8, 8
    inp = _inputs(B, N, d, H, d_k, dd, d_R, seed=61)
    a, _, _ = oracle.prefill_drope(inp, H, d_k, d_R, 6)
    b, _, _ = oracle.prefill_drope(inp, H, d_k, d_R, 6, pos0=1000)
    assert np.abs(a - b).max() < 1e-11


@pytest.mark.parametrize("w", [0, 1, 10, 60])
def test_decode_cache_form_equals_prefill_row(w):
    """The cache form (content keys of old positions rebuilt from h^D through
    W_up, rotary keys read from their own cache, the window ring) gives row p
    of the prefill form."""
    B, N, d, H, d_k, dd, d_R = 2, 40, 32, 2, 8, 8, 4
    inp = _inputs(B, N, d, H, d_k, dd, d_R, seed=70 + w)
    o, _, P = oracle.prefill_drope(inp, H, d_k, d_R, w)
    p = N - 1
    K_win = np.zeros((B, H, max(w, 1), d_k))
    V_win = np.zeros((B, H, max(w, 1), d_k))
    for j in range(max(0, p - w + 1), p + 1):
        K_win[:, :, j % w] = P["KL"][:, :, j]
        V_win[:, :, j % w] = P["VL"][:, :, j]
    got = oracle.decode_drope(P["QC"][:, :, p], P["QR"][:, :, p], K_win[:, :, :w],
                              V_win[:, :, :w], P["KR"], P["hD"], inp["W_up"], inp["W_K"],
                              inp["W_V"], N, w)
    assert np.abs(got - o[:, p]).max() < 1e-12
