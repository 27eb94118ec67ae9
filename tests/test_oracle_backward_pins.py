"""Pins of the fp64 oracle's attention backward (gradients of Eqs. 3-4).

Paper: "Dual Dimensionality for Local and Global Attention": Eq. (3) picks,
per (query i, key j) pair, the full-state key/value when i - j < w and the
bottleneck one otherwise; Eq. (4) is softmax attention; the training remark
after Eq. (4) says the bottleneck weights learn only from pairs that use the
global path.  The gradient of a pair therefore flows to the source it used.
None of these pins re-types the oracle's loops: they use central finite
differences of the (separately pinned) forward oracle, torch's autograd of
its own attention routine, exact invariances of softmax, and a closed form.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def _rand(B, H, N, d_k, seed):
    r = np.random.default_rng(seed)
    P = {k: r.standard_normal((B, H, N, d_k)) for k in ("Q", "KL", "VL", "KG", "VG")}
    dO = r.standard_normal((B, N, H * d_k))
    return P, dO


def _loss(P, w, dO):
    o, _ = oracle.attend(P, w)
    return float(np.sum(o * dO))


@pytest.mark.parametrize("w", [0, 1, 3, 50])
def test_backward_matches_finite_differences(w):
    B, H, N, d_k = 1, 2, 7, 4
    P, dO = _rand(B, H, N, d_k, seed=100 + w)
    g = oracle.attend_backward(P, w, dO)
    eps = 1e-5
    for name, gname in (("Q", "dQ"), ("KL", "dKL"), ("VL", "dVL"), ("KG", "dKG"), ("VG", "dVG")):
        num = np.zeros_like(P[name])
        for idx in np.ndindex(P[name].shape):
            save = P[name][idx]
            P[name][idx] = save + eps
            lp = _loss(P, w, dO)
            P[name][idx] = save - eps
            lm = _loss(P, w, dO)
            P[name][idx] = save
            num[idx] = (lp - lm) / (2 * eps)
        assert np.abs(num - g[gname]).max() < 1e-7, (name, np.abs(num - g[gname]).max())


def _sdpa_grads(Q, K, V, dO):
    """torch's causal attention and its autograd, fp64 on the CPU."""
    t = [torch.tensor(x, requires_grad=True) for x in (Q, K, V)]
    o = F.scaled_dot_product_attention(*t, is_causal=True)
    B, H, N, d_k = Q.shape
    g = torch.tensor(dO.reshape(B, N, H, d_k).transpose(0, 2, 1, 3))
    o.backward(g)
    return [x.grad.numpy() for x in t]


def test_window_covering_sequence_is_vanilla_backward():
    """w >= N: every pair is local; the gradients equal those of plain causal
    attention over (Q, KL, VL) and the global source receives nothing."""
    P, dO = _rand(2, 3, 33, 8, seed=7)
    g = oracle.attend_backward(P, 33, dO)
    dq, dk, dv = _sdpa_grads(P["Q"], P["KL"], P["VL"], dO)
    assert np.abs(g["dQ"] - dq).max() < 1e-10
    assert np.abs(g["dKL"] - dk).max() < 1e-10
    assert np.abs(g["dVL"] - dv).max() < 1e-10
    assert not g["dKG"].any() and not g["dVG"].any()


def test_zero_window_is_global_backward():
    """w = 0: every pair (the diagonal too) is global."""
    P, dO = _rand(1, 2, 29, 8, seed=8)
    g = oracle.attend_backward(P, 0, dO)
    dq, dk, dv = _sdpa_grads(P["Q"], P["KG"], P["VG"], dO)
    assert np.abs(g["dQ"] - dq).max() < 1e-10
    assert np.abs(g["dKG"] - dk).max() < 1e-10
    assert np.abs(g["dVG"] - dv).max() < 1e-10
    assert not g["dKL"].any() and not g["dVL"].any()


@pytest.mark.parametrize("w", [1, 5, 17])
def test_softmax_invariances(w):
    """Shifting every key (both sources) by one vector leaves each softmax
    unchanged, so the key gradients sum to zero; the softmax weights of each
    row sum to one, so the value gradients sum to the sum of dO."""
    B, H, N, d_k = 2, 2, 40, 8
    P, dO = _rand(B, H, N, d_k, seed=w)
    g = oracle.attend_backward(P, w, dO)
    ksum = (g["dKL"] + g["dKG"]).sum(axis=2)
    assert np.abs(ksum).max() < 1e-10
    vsum = (g["dVL"] + g["dVG"]).sum(axis=2)
    want = dO.reshape(B, N, H, d_k).sum(axis=1)
    assert np.abs(vsum - want).max() < 1e-10


@pytest.mark.parametrize("w", [0, 4, 9])
def test_uniform_attention_value_gradient_closed_form(w):
    """Q = 0 makes every row's softmax uniform over j <= i, so
    dv_j = sum over i >= j with the pair on that source of dO_i / (i + 1)."""
    B, H, N, d_k = 1, 2, 12, 4
    P, dO = _rand(B, H, N, d_k, seed=3 + w)
    P["Q"][:] = 0.0
    g = oracle.attend_backward(P, w, dO)
    G = dO.reshape(B, N, H, d_k).transpose(0, 2, 1, 3)
    wl = np.zeros_like(G)
    wg = np.zeros_like(G)
    for j in range(N):
        for i in range(j, N):
            if i - j < w:
                wl[:, :, j] += G[:, :, i] / (i + 1)
            else:
                wg[:, :, j] += G[:, :, i] / (i + 1)
    assert np.abs(g["dVL"] - wl).max() < 1e-12
    assert np.abs(g["dVG"] - wg).max() < 1e-12


def test_lse_uniform_and_vanilla():
    """Q = 0: every score is 0, so lse_i = log(i + 1).  w >= N: the causal
    log-sum-exp of plain attention, from torch."""
    B, H, N, d_k = 1, 2, 40, 8
    P, _ = _rand(B, H, N, d_k, seed=11)
    Z = dict(P)
    Z["Q"] = np.zeros_like(P["Q"])
    lse = oracle.attend_lse(Z, 7)
    assert np.abs(lse - np.log(np.arange(1, N + 1))[None, None]).max() < 1e-13
    s = torch.tensor(P["Q"]) @ torch.tensor(P["KL"]).transpose(-1, -2) / np.sqrt(d_k)
    s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    want = torch.logsumexp(s, dim=-1).numpy()
    assert np.abs(oracle.attend_lse(P, N) - want).max() < 1e-12


@pytest.mark.parametrize("w", [0, 1, 5, 39])
def test_lse_window_edge_closed_form(w):
    """Eq. 3's edge i - j < w in the normaliser.  q = e_0, local keys 0 (score
    0), global keys with q.k = c sqrt(d_k) (score c): row i has min(i+1, w)
    local pairs and max(0, i+1-w) global ones, so
    lse_i = log(min(i+1, w) + max(0, i+1-w) e^c).  Taking i - j <= w instead
    moves one pair per row from e^c to 1 and fails this."""
    B, H, N, d_k, c = 1, 2, 40, 8, 1.5
    Q = np.zeros((B, H, N, d_k))
    Q[..., 0] = 1.0
    KG = np.zeros((B, H, N, d_k))
    KG[..., 0] = c * np.sqrt(d_k)
    P = dict(Q=Q, KL=np.zeros((B, H, N, d_k)), KG=KG)
    i = np.arange(N)
    want = np.log(np.minimum(i + 1, w) + np.maximum(0, i + 1 - w) * np.exp(c))
    got = oracle.attend_lse(P, w)
    assert np.abs(got - want[None, None]).max() < 1e-13
