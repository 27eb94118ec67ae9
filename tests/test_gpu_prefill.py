"""GPU parity of the prefill path (dar_fold, dar_project, dar_attn_prefill)
against the fp64 oracle, through the C ABI.

Tolerances: max-abs 2e-2 for bf16 I/O with fp32 accumulation and 1e-4 for
the fp32 mode, on the attention output o (before W_O).  Intermediates (fp16
in bf16 mode) are checked with the same absolute bound plus 1% of the
reference magnitude: the global keys and values go through the bf16 folded
weights, which round at 2^-9 relative."""
import numpy as np
import pytest
import torch

import dar_inputs as di
import distance_adaptive_dual_amd as dar
import oracle
from gpu_helpers import TOL, dev, dev_w, host, log, max_err, prefill_case, weights_dev

pytestmark = pytest.mark.gpu


def run_prefill(inp, H, d_k, w, dtype, fold=True, pos0=0):
    W = weights_dev(inp, dtype)
    h = dev(inp["h"], dtype)
    Wk = Wv = None
    if fold:
        Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    out = dar.dar_project(h, W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"], H, d_k,
                          W_upK=Wk, W_upV=Wv, pos0=pos0)
    o = dar.dar_attn_prefill(out["Q"], out["K_loc"], out["V_loc"], out["K_glob"], out["V_glob"],
                             w)
    torch.cuda.synchronize()
    return o, out


def check_projections(out, P, dtype):
    tol = TOL[dtype]
    pairs = [("Q", P["Q"]), ("K_loc", P["KL"]), ("V_loc", P["VL"].transpose(0, 1, 3, 2)),
             ("h_D", P["hD"]), ("K_glob", P["KG"]), ("V_glob", P["VG"].transpose(0, 1, 3, 2))]
    for name, ref in pairs:
        got = host(out[name])
        err = np.abs(got - ref)
        # rounding of a stored 16-bit operand scales with the operand, not with
        # the (possibly cancelling) result: add a term in the row's rms
        axis = 2 if name in ("V_loc", "V_glob") else -1
        rms = np.sqrt(np.mean(ref ** 2, axis=axis, keepdims=True))
        bound = (tol + 1e-2 * np.abs(ref) + 1e-2 * rms if dtype == "bf16"
                 else tol * (1 + np.abs(ref)))
        assert np.all(err <= bound), "%s: max err %.3g" % (name, err.max())


# ------------------------------------------------------------------ end to end
@pytest.mark.parametrize("fold", [True, False])
def test_fp32_layer_512(fold):
    """fp32 layer: B1, N512, d512, 8 heads of 64, w128, d_down128 (1e-4)."""
    B, N, d, H, d_k, w, dd = 1, 512, 512, 8, 64, 128, 128
    inp = prefill_case(B, N, d, H, d_k, dd, "f32", seed=1000)
    log("fp32 layer fold=%s" % fold)
    o, out = run_prefill(inp, H, d_k, w, "f32", fold=fold)
    ref, rs, P = oracle.prefill(inp, H, d_k, w)
    check_projections(out, P, "f32")
    err = max_err(host(o), ref)
    log("  max err %.3g" % err)
    assert err <= TOL["f32"]


@pytest.mark.parametrize("B,N,d,H,d_k,dd,w", [
    (2, 300, 256, 4, 64, 64, 77),      # ragged N (not a multiple of any tile)
    (1, 257, 128, 2, 128, 32, 129),    # d_k 128, tail of one key
    (2, 200, 256, 4, 64, 128, 0),      # w = 0: every pair global
    (1, 190, 128, 2, 64, 64, 1),       # w = 1: only the diagonal is local
    (1, 333, 256, 2, 128, 128, 1000),  # w >= N: every pair local
    (2, 512, 256, 4, 64, 96, 128),     # d_down not a power of two
    (1, 1, 128, 2, 64, 32, 5),         # a single token
    (1, 7, 128, 2, 128, 64, 3),        # shorter than one tile
])
def test_bf16_small(B, N, d, H, d_k, dd, w):
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=31 * N + w)
    log("bf16 B%d N%d d%d H%d dk%d dd%d w%d" % (B, N, d, H, d_k, dd, w))
    o, out = run_prefill(inp, H, d_k, w, "bf16")
    ref, _, P = oracle.prefill(inp, H, d_k, w)
    check_projections(out, P, "bf16")
    err = max_err(host(o), ref)
    log("  max err %.3g" % err)
    assert err <= TOL["bf16"]


def test_fp32_ragged_and_pos0():
    """fp32, ragged N, d_k 128, nonzero start position."""
    B, N, d, H, d_k, dd, w = 2, 150, 128, 2, 128, 64, 40
    inp = prefill_case(B, N, d, H, d_k, dd, "f32", seed=77)
    o, out = run_prefill(inp, H, d_k, w, "f32", pos0=1000)
    ref, _, P = oracle.prefill(inp, H, d_k, w, pos0=1000)
    check_projections(out, P, "f32")
    assert max_err(host(o), ref) <= TOL["f32"]


@pytest.mark.parametrize("pos0,d_k", [(32768 - 40, 64), (2 ** 24 - 96, 128), (1234567, 64)])
def test_bf16_rope_large_positions(pos0, d_k):
    """bf16 projections at large positions: the rotation matches the fp64 one
    to within the fp16 rounding of the output (relative to the magnitude of
    each rotated pair)."""
    B, N, d, H, dd, w = 1, 96, 128, 2, 32, 16
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=pos0 % 1000 + 5)
    log("bf16 rope pos0 %d d_k %d" % (pos0, d_k))
    o, out = run_prefill(inp, H, d_k, w, "bf16", pos0=pos0)
    ref, _, P = oracle.prefill(inp, H, d_k, w, pos0=pos0)
    half = d_k // 2
    for name, r in (("Q", P["Q"]), ("K_loc", P["KL"])):
        mag = np.sqrt(r[..., :half] ** 2 + r[..., half:] ** 2)
        mag = np.concatenate([mag, mag], axis=-1)
        err = np.abs(host(out[name]) - r)
        worst = float((err / (mag + 1e-6)).max())
        log("  %s worst err / pair magnitude %.3g" % (name, worst))
        assert np.all(err <= 2.0 ** -10 * mag + 1e-5), name
    assert max_err(host(o), ref) <= TOL["bf16"]


def test_peaked_softmax_and_hot_rows():
    """W_Q x4 (sharp softmax) and rows of h scaled x8 (scores in the tens).

    With a near one-hot softmax, 16-bit storage of q and k moves scores by up
    to |q||k| 2^-11 and the output by O(|v|) between near-tied keys, so the
    end-to-end output is not comparable at 2e-2.  The projections are checked
    end to end, and the attention stage is checked on the oracle's own
    projections rounded to fp16 (the kernel's input format), which isolates
    the max subtraction and the online softmax."""
    B, N, d, H, d_k, dd, w = 2, 384, 256, 4, 64, 64, 100
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=91, q_scale=4.0, hot_rows=20)
    _, out = run_prefill(inp, H, d_k, w, "bf16")
    _, _, P = oracle.prefill(inp, H, d_k, w)
    check_projections(out, P, "bf16")
    R = {k: di.round_f16(P[k]) for k in ("Q", "KL", "VL", "KG", "VG")}
    got = _attn_gpu(R, w)
    ref, _ = oracle.attend(R, w)
    # values of hot rows reach |v| ~ 30, where one bf16 output ulp is 0.25:
    # the bound adds the output's own rounding (2^-9 relative) to 2e-2
    err = np.abs(got - ref) - 2.0 ** -8 * np.abs(ref)
    log("  peaked (attention stage) max err beyond output rounding %.3g" % err.max())
    assert err.max() <= TOL["bf16"]


@pytest.mark.parametrize("dd", [256, 128, 64])
def test_pythia70m_layer(dd):
    """B8, N2048, d512, 8 heads of 64, w128: every output against the oracle."""
    B, N, d, H, d_k, w = 8, 2048, 512, 8, 64, 128
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=2000 + dd)
    log("pythia70m dd=%d" % dd)
    o, out = run_prefill(inp, H, d_k, w, "bf16")
    ref, rs, P = oracle.prefill(inp, H, d_k, w)
    check_projections(out, P, "bf16")
    err = max_err(host(o), ref)
    log("  max err %.3g" % err)
    assert err <= TOL["bf16"]


def test_pythia410m_layer():
    """B8, N2048, d1024, 16 heads of 64, w128, d_down 256."""
    B, N, d, H, d_k, w, dd = 8, 2048, 1024, 16, 64, 128, 256
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=3000)
    o, _ = run_prefill(inp, H, d_k, w, "bf16")
    ref, _, _ = oracle.prefill(inp, H, d_k, w)
    err = max_err(host(o), ref)
    log("  410m max err %.3g" % err)
    assert err <= TOL["bf16"]


def test_1b_layer_sampled():
    """B4, N8192, d2048, 16 heads of 128, w512, d_down 512: the full-size launch,
    checked on sampled rows of two (batch, head) pairs (oracle on one batch and
    one head at a time)."""
    B, N, d, H, d_k, w, dd = 4, 8192, 2048, 16, 128, 512, 512
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=4000)
    o, _ = run_prefill(inp, H, d_k, w, "bf16")
    o = host(o)
    rng = np.random.Generator(np.random.PCG64(4007))
    for b, hh in [(0, 3), (3, 14)]:
        one = dict(inp, h=inp["h"][b:b + 1])
        P = oracle.project(one["h"], one["W_down"], one["W_up"], one["W_Q"], one["W_K"],
                           one["W_V"], H, d_k, heads=(hh, hh + 1))
        rows_i = np.concatenate([[0, 1, 511, 512, 513, 8191],
                                 rng.integers(0, N, size=26)])
        rows = [(0, hh, int(i)) for i in rows_i]
        ref, _ = oracle.attend_rows(P, w, rows)
        got = np.stack([o[b, i, hh * d_k:(hh + 1) * d_k] for (_, _, i) in rows])
        err = max_err(got, ref)
        log("  1b b%d h%d max err %.3g" % (b, hh, err))
        assert err <= TOL["bf16"]


# ------------------------------------------------------------------ fold
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fold_is_matrix_product(dtype):
    """W_upK = W_up W_K and W_upV = W_up W_V (Eqs. 2-3), stored column-major."""
    d, dd, H, d_k = 256, 64, 4, 64
    inp = prefill_case(1, 4, d, H, d_k, dd, dtype, seed=5)
    W = weights_dev(inp, dtype)
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    torch.cuda.synchronize()
    for got, Wx in ((Wk, inp["W_K"]), (Wv, inp["W_V"])):
        ref = (inp["W_up"] @ Wx).T  # column-major storage = transpose, row-major
        err = np.abs(host(got) - ref)
        bound = (1e-5 if dtype == "f32" else 0) + 2.0 ** -8 * np.abs(ref) + 1e-6
        assert np.all(err <= bound), err.max()


# ------------------------------------------------------------------ attention only
def _attn_inputs(B, H, N, d_k, seed, dtype="f16", std=1.0):
    sh = (B, H, N, d_k)
    return {k: di.gaussian(seed + i, sh, std, dtype)
            for i, k in enumerate(("Q", "KL", "VL", "KG", "VG"))}


def _attn_gpu(P, w, dtype="f16"):
    """bf16 mode of dar_attn_prefill: fp16 Q/K/V in, bf16 o out."""
    Q, KL, KG = (dev(P[k], dtype) for k in ("Q", "KL", "KG"))
    VL = dev(P["VL"].transpose(0, 1, 3, 2), dtype)
    VG = dev(P["VG"].transpose(0, 1, 3, 2), dtype)
    o = dar.dar_attn_prefill(Q, KL, VL, KG, VG, w)
    torch.cuda.synchronize()
    return host(o)


@pytest.mark.parametrize("N,d_k,w", [(1000, 64, 0), (1000, 64, 63), (1000, 64, 64),
                                     (1000, 64, 65), (777, 128, 127), (777, 128, 128),
                                     (777, 128, 129), (640, 128, 256), (129, 64, 16),
                                     (64, 128, 4), (2048, 64, 128)])
def test_attention_seeded(N, d_k, w):
    """dar_attn_prefill on seeded fp16 Q/K/V against the oracle's Eq. 3-4 loops."""
    B, H = 2, 2
    P = _attn_inputs(B, H, N, d_k, seed=100 + N + w)
    got = _attn_gpu(P, w)
    ref, _ = oracle.attend(P, w)
    err = max_err(got, ref)
    log("attn N%d dk%d w%d max err %.3g" % (N, d_k, w, err))
    assert err <= TOL["bf16"]


def _sweep_cases(n=12, seed=5151):
    """Seeded shapes around the 64-key tiles and 128-query tiles (and the
    zero rows the K staging reads past N): random N, windows 0, 1, random and
    >= N, both head widths, 1-2 batches and 1-3 heads."""
    g = np.random.Generator(np.random.PCG64(seed))
    out = []
    for k in range(n):
        N = int(g.integers(1, 900))
        w = (0, 1, int(g.integers(2, N + 10)), N + 50)[(k // 2) % 4]
        out.append((int(g.integers(1, 3)), int(g.integers(1, 4)), N, (64, 128)[k % 2], w))
    return out


@pytest.mark.parametrize("B,H,N,d_k,w", _sweep_cases())
def test_attention_seeded_sweep(B, H, N, d_k, w):
    P = _attn_inputs(B, H, N, d_k, seed=6100 + N + w)
    got = _attn_gpu(P, w)
    ref, _ = oracle.attend(P, w)
    err = max_err(got, ref)
    log("attn sweep B%d H%d N%d dk%d w%d max err %.3g" % (B, H, N, d_k, w, err))
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("N,d_k,w", [(700, 64, 100), (700, 128, 100), (300, 64, 0),
                                     (300, 128, 1), (2048, 128, 512), (513, 64, 700)])
def test_selection_counts_exact(N, d_k, w):
    """Closed form of Eq. 3's selection.  Q = 0 makes the softmax uniform over
    j <= i.  Value dims [0, d_k/2) carry an indicator of j mod (d_k/2) on the
    local source, dims [d_k/2, d_k) the same on the global source, so
    (i+1) * o_i[c] counts the pairs of each residue that took each path; the
    counts are small integers, far from bf16 rounding."""
    B, H = 1, 2
    R = d_k // 2
    Q = np.zeros((B, H, N, d_k))
    KL = di.gaussian(7, (B, H, N, d_k), 1.0, "bf16")
    KG = di.gaussian(8, (B, H, N, d_k), 1.0, "bf16")
    VL = np.zeros((B, H, N, d_k))
    VG = np.zeros((B, H, N, d_k))
    j = np.arange(N)
    VL[:, :, j, j % R] = 1.0
    VG[:, :, j, R + j % R] = 1.0
    got = _attn_gpu(dict(Q=Q, KL=KL, VL=VL, KG=KG, VG=VG), w)
    i = np.arange(N)[:, None]
    jj = np.arange(N)[None, :]
    causal = jj <= i
    loc = causal & (i - jj < w)
    glob = causal & ~(i - jj < w)
    onehot = np.zeros((N, R))
    onehot[np.arange(N), np.arange(N) % R] = 1.0
    cnt = np.concatenate([loc.astype(float) @ onehot, glob.astype(float) @ onehot], axis=1)
    scaled = got[0].reshape(N, H, d_k) * (np.arange(N)[:, None, None] + 1)
    for hh in range(H):
        assert np.max(np.abs(scaled[:, hh, :] - cnt)) < 0.25


@pytest.mark.parametrize("N,d_k,w", [(600, 64, 100), (600, 128, 257), (300, 64, 1)])
def test_key_source_selection(N, d_k, w):
    """Keys follow the same rule as values: q = e_0, local keys -1024 e_0 (their
    softmax weight underflows to 0 wherever a global pair exists), global keys
    0.  Rows i >= w then average the global values of j <= i - w only; rows
    i < w average their local values."""
    B, H = 1, 1
    R = d_k // 2
    Q = np.zeros((B, H, N, d_k))
    Q[..., 0] = 1.0
    KL = np.zeros((B, H, N, d_k))
    KL[..., 0] = -1024.0
    KG = np.zeros((B, H, N, d_k))
    VL = np.zeros((B, H, N, d_k))
    VG = np.zeros((B, H, N, d_k))
    j = np.arange(N)
    VL[:, :, j, j % R] = 1.0
    VG[:, :, j, R + j % R] = 1.0
    got = _attn_gpu(dict(Q=Q, KL=KL, VL=VL, KG=KG, VG=VG), w)[0]
    for i in range(N):
        exp = np.zeros(d_k)
        if i >= w:
            js = np.arange(0, i - w + 1)
            np.add.at(exp, R + js % R, 1.0 / len(js))
        else:
            js = np.arange(0, i + 1)
            np.add.at(exp, js % R, 1.0 / len(js))
        assert np.max(np.abs(got[i] - exp) * (i + 1)) < 0.25, i


def test_deterministic():
    B, N, d, H, d_k, dd, w = 2, 700, 256, 4, 128, 64, 128
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=55)
    o1, _ = run_prefill(inp, H, d_k, w, "bf16")
    o2, _ = run_prefill(inp, H, d_k, w, "bf16")
    assert torch.equal(o1, o2)
