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


def bf16_half_spacing(x):
    """Half the distance between adjacent bf16 values around |x| (8
    significant bits): the largest error of rounding x to bf16, between
    2^-9 |x| (top of a binade) and 2^-8 |x| (bottom)."""
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 8)


def storage_error_bound(inp, P, w, d_k, nsig=7.0):
    """Per-element bound on |o_gpu - o_ref| of the bf16 path, to first order in
    the roundings of what the kernels store in 16 bits.  Each stored element
    is rounded independently, by at most u |x| (u = 2^-11 for the fp16
    Q, K, V and h^D, 2^-8 for the bf16 folded weights W_up W_K, W_up W_V), so
    its error has variance (u x)^2 / 3.  Then, with p_ij the softmax weights:
      - a pair's score s_ij = q_i.k_j / sqrt(d_k) moves by ds_ij, a sum of
        many such terms (q and k storage; for global keys also h^D storage and
        the folded weight, whose rotation by RoPE is bounded through the
        rotation-invariant pair sums q_t^2 + q_{t+d_k/2}^2);
      - to first order o_i moves by sum_j p_ij ds_ij (v_j - o_i), at most
        Ds_i J_i with Ds_i = nsig max_j sd(ds_ij), J_i = sum_j p_ij |v_j - o_i|;
        P rounded to fp16 adds 2^-11 J_i;
      - value storage adds sum_j p_ij dv_j, whose variance is summed the same
        way (the folded-weight part is common to every j: sum_j p_ij h^D_j
        multiplies it);
      - fp32 arithmetic: 1e-4 max |o|.
    The bf16 rounding of o itself is added by the caller.  Returns
    (bound, o_ref) with o_ref the fp64 output rebuilt from P."""
    u, ub = 2.0 ** -11, 2.0 ** -8
    h = d_k // 2
    B, H, N, _ = P["Q"].shape
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    causal = j <= i
    local = causal & (i - j < w)
    glob = causal & ~(i - j < w)
    Wk_all = inp["W_up"] @ inp["W_K"]
    Wv_all = inp["W_up"] @ inp["W_V"]
    bound = np.zeros((B, N, H * d_k))
    o_all = np.zeros((B, N, H * d_k))
    for b in range(B):
        hD = P["hD"][b]
        hD2 = hD ** 2
        for a in range(H):
            Q, KL, KG = P["Q"][b, a], P["KL"][b, a], P["KG"][b, a]
            VL, VG = P["VL"][b, a], P["VG"][b, a]
            Wk = Wk_all[:, a * d_k:(a + 1) * d_k]
            Wv = Wv_all[:, a * d_k:(a + 1) * d_k]
            s = np.where(local, Q @ KL.T, Q @ KG.T) / np.sqrt(d_k)
            s = np.where(causal, s, -np.inf)
            pr = np.exp(s - s.max(1, keepdims=True))
            pr /= pr.sum(1, keepdims=True)
            o = np.where(local[:, :, None], VL[None], VG[None])
            o = np.einsum("ij,ijc->ic", pr, o)
            o_all[b, :, a * d_k:(a + 1) * d_k] = o
            # score variances
            qq = Q[:, :h] ** 2 + Q[:, h:] ** 2                       # [N, h]
            var_loc = (2 * u * u / 3) * (Q ** 2 @ (KL ** 2).T) / d_k
            Wmax = np.maximum(Wk[:, :h] ** 2, Wk[:, h:] ** 2)         # [dd, h]
            wn = np.sqrt(Wk[:, :h] ** 2 + Wk[:, h:] ** 2)             # [dd, h]
            fold = (qq @ Wmax.T) @ hD2.T                              # [N_i, N_j]
            hdr = ((np.sqrt(qq) @ wn.T) ** 2) @ hD2.T
            var_glb = ((2 * u * u / 3) * (Q ** 2 @ (KG ** 2).T)
                       + (ub * ub / 3) * fold + (u * u / 3) * hdr) / d_k
            sd = np.sqrt(np.where(local, var_loc, np.where(glob, var_glb, 0.0)))
            Ds = nsig * sd.max(1)
            V = np.where(local[:, :, None], VL[None], VG[None])       # [i, j, c]
            J = np.einsum("ij,ijc->ic", pr, np.abs(V - o[:, None, :]))
            pg = np.where(glob, pr, 0.0)
            var_v = ((u * u / 3) * ((pr ** 2) [:, :, None] * V ** 2).sum(1)
                     + (ub * ub / 3) * ((pg @ hD) ** 2 @ Wv ** 2)
                     + (u * u / 3) * ((pg ** 2) @ (hD2 @ Wv ** 2)))
            bound[b, :, a * d_k:(a + 1) * d_k] = ((Ds + u)[:, None] * J + nsig * np.sqrt(var_v)
                                                  + 1e-4 * np.abs(o).max())
    return bound, o_all


def test_peaked_softmax_and_hot_rows():
    """W_Q x4 (sharp softmax) and rows of h scaled x8 (scores in the tens).

    End to end, a near one-hot softmax turns the 16-bit storage of q and k into
    output changes of O(|v|) between near-tied keys, so the whole layer is
    checked against a per-element bound derived from those roundings
    (storage_error_bound) plus the bf16 rounding of o.  The attention stage
    alone is checked on the oracle's projections rounded to fp16 (the
    kernel's input format) at 2e-2 plus the bf16 rounding of o."""
    B, N, d, H, d_k, dd, w = 2, 384, 256, 4, 64, 64, 100
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=91, q_scale=4.0, hot_rows=20)
    o, out = run_prefill(inp, H, d_k, w, "bf16")
    ref_e2e, _, P = oracle.prefill(inp, H, d_k, w)
    check_projections(out, P, "bf16")
    got_e2e = host(o)
    bound, o64 = storage_error_bound(inp, P, w, d_k)
    assert np.abs(o64 - ref_e2e).max() < 1e-9  # the bound's own softmax is the oracle's
    bound += bf16_half_spacing(ref_e2e)
    excess = np.abs(got_e2e - ref_e2e) - bound
    log("  peaked end to end: max err %.3g, max bound %.3g, max excess %.3g"
        % (np.abs(got_e2e - ref_e2e).max(), bound.max(), excess.max()))
    assert excess.max() <= 0.0
    R = {k: di.round_f16(P[k]) for k in ("Q", "KL", "VL", "KG", "VG")}
    got = _attn_gpu(R, w)
    ref, _ = oracle.attend(R, w)
    # hot rows reach |o| ~ 30, where the bf16 rounding of o alone is up to 0.06
    err = np.abs(got - ref) - bf16_half_spacing(ref)
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


def test_1b_layer_slices():
    """B4, N8192, d2048, 16 heads of 128, w512, d_down 512: the full-size launch.
    Four (batch, head) slices, one in each batch and spread over the heads,
    are checked in full: every output row of the slice, the slice's Q, K_loc,
    V_loc, K_glob, V_glob and the batch's h^D (the oracle runs on one batch
    and one head at a time)."""
    B, N, d, H, d_k, w, dd = 4, 8192, 2048, 16, 128, 512, 512
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=4000)
    o, out = run_prefill(inp, H, d_k, w, "bf16")
    for b, hh in [(0, 0), (1, 5), (2, 10), (3, 15)]:
        one = dict(inp, h=inp["h"][b:b + 1])
        P = oracle.project(one["h"], one["W_down"], one["W_up"], one["W_Q"], one["W_K"],
                           one["W_V"], H, d_k, heads=(hh, hh + 1))
        S = {k: np.ascontiguousarray(P[k][:, hh:hh + 1]) for k in ("Q", "KL", "VL", "KG", "VG")}
        sl = {k: out[k][b:b + 1, hh:hh + 1] for k in ("Q", "K_loc", "V_loc", "K_glob", "V_glob")}
        sl["h_D"] = out["h_D"][b:b + 1]
        check_projections(sl, dict(S, hD=P["hD"]), "bf16")
        ref, _ = oracle.attend(S, w)
        got = host(o[b:b + 1, :, hh * d_k:(hh + 1) * d_k])
        err = max_err(got, ref)
        log("  1b b%d h%d every row: max err %.3g (max |o| %.3g)" % (b, hh, err,
                                                                    np.abs(ref).max()))
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


@pytest.mark.parametrize("N,w", [(64, 4), (128, 0), (320, 1), (320, 63), (512, 64), (512, 65),
                                 (448, 1000), (1216, 257), (1216, 1216)])
def test_attention_ring_tiles(N, w):
    """d_k 128 whole prefills whose N is a multiple of 64 run the ring kernel
    (eight waves, 256 queries per workgroup, key tiles by direct loads into a
    four-stage LDS ring): one key tile, partial 256-query tiles (N = 320, 448,
    1216, so the pairs of query tiles include a short last one), windows on
    both sides of the 64-key tile edge, w = 0 and w >= N.  o against the
    oracle at 2e-2, and the log-sum-exp variant's lse against the oracle's row
    normalisers at 2e-3 (its o bit-identical to dar_attn_prefill's)."""
    B, H, d_k = 2, 3, 128
    P = _attn_inputs(B, H, N, d_k, seed=8800 + N + w)
    got = _attn_gpu(P, w)
    ref, _ = oracle.attend(P, w)
    err = max_err(got, ref)
    Q, KL, KG = (dev(P[k], "f16") for k in ("Q", "KL", "KG"))
    VL = dev(P["VL"].transpose(0, 1, 3, 2), "f16")
    VG = dev(P["VG"].transpose(0, 1, 3, 2), "f16")
    o2, lse = dar.dar_attn_prefill_lse(Q, KL, VL, KG, VG, w)
    torch.cuda.synchronize()
    lse_err = np.abs(host(lse) - oracle.attend_lse(P, w)).max()
    log("ring N%d w%d: max err %.3g, lse err %.3g" % (N, w, err, lse_err))
    assert err <= TOL["bf16"]
    assert np.array_equal(host(o2), got)
    assert lse_err <= 2e-3


@pytest.mark.parametrize("N,d_k,w", [(700, 64, 100), (700, 128, 100), (300, 64, 0),
                                     (300, 128, 1), (2048, 128, 512), (513, 64, 700),
                                     (1216, 128, 100), (320, 128, 0), (1216, 64, 100),
                                     (320, 64, 0)])
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


@pytest.mark.parametrize("N,d_k,w", [(600, 64, 100), (600, 128, 257), (300, 64, 1),
                                     (1216, 128, 257), (320, 128, 1), (1216, 64, 257),
                                     (320, 64, 1)])
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


# ------------------------------------------------------------------ fp16 range
def test_fp16_intermediates_near_range_edge():
    """In bf16 mode the projections are stored as fp16 (largest finite 65504).
    h scaled so that the largest projection reaches ~6e4: every intermediate
    still matches the oracle to its fp16 rounding and o is finite.  The
    attention stage alone, fed values of magnitude up to ~6e4, matches the
    oracle at the usual bound scaled by the value scale (the softmax is
    invariant to it) plus the bf16 rounding of o."""
    B, N, d, H, d_k, dd, w = 1, 200, 256, 2, 64, 64, 50
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=6553)
    _, _, P0 = oracle.prefill(inp, H, d_k, w)
    peak = max(np.abs(P0[k]).max() for k in ("Q", "KL", "VL", "hD", "KG", "VG"))
    scale = 2.0 ** np.floor(np.log2(6.0e4 / peak))  # a power of two keeps h exact in bf16
    big = dict(inp, h=inp["h"] * scale)
    o, out = run_prefill(big, H, d_k, w, "bf16")
    _, _, P = oracle.prefill(big, H, d_k, w)
    peak_big = max(np.abs(P[k]).max() for k in ("Q", "KL", "VL", "hD", "KG", "VG"))
    log("  fp16 edge: largest intermediate %.4g" % peak_big)
    assert 3.0e4 <= peak_big < 65504
    for name, ref in (("Q", P["Q"]), ("K_loc", P["KL"]), ("V_loc", P["VL"].transpose(0, 1, 3, 2)),
                      ("h_D", P["hD"]), ("K_glob", P["KG"]),
                      ("V_glob", P["VG"].transpose(0, 1, 3, 2))):
        got = host(out[name])
        assert np.all(np.isfinite(got)), name
        rms = np.sqrt(np.mean(ref ** 2, axis=2 if name.startswith("V_") else -1, keepdims=True))
        assert np.all(np.abs(got - ref) <= 1e-2 * (np.abs(ref) + rms) + 1e-3), name
    assert torch.isfinite(o.float()).all()
    # attention stage, values up to ~6e4
    vs = 2.0 ** 13
    A = _attn_inputs(1, 2, 300, 64, seed=6554)
    for k in ("VL", "VG"):
        A[k] = di.round_f16(np.clip(A[k] * vs, -6.0e4, 6.0e4))
    got = _attn_gpu(A, 70)
    ref, _ = oracle.attend(A, 70)
    err = np.abs(got - ref) - bf16_half_spacing(ref)
    log("  fp16 edge attention: max |v| %.4g, max err beyond rounding / scale %.3g"
        % (max(np.abs(A["VL"]).max(), np.abs(A["VG"]).max()), err.max() / vs))
    assert err.max() <= TOL["bf16"] * vs


def test_fp16_intermediates_beyond_range_become_inf():
    """The stated behaviour past the fp16 range: a projection of magnitude
    >= 65520 rounds to +-inf in the intermediate (round to nearest even), and
    no status reports it (the values exist only on the device)."""
    B, N, d, H, d_k, dd, w = 1, 64, 128, 2, 64, 32, 16
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=6555)
    big = dict(inp, h=inp["h"].copy())
    big["h"][0, 10] *= 2.0 ** 18  # token 10's projections move far past 65504
    _, out = run_prefill(big, H, d_k, w, "bf16")
    _, _, P = oracle.prefill(big, H, d_k, w)
    V = host(out["V_loc"])[0, :, :, 10]  # [heads, d_k]
    ref = P["VL"][0, :, 10]
    over = np.abs(ref) >= 65520
    assert over.any()
    assert np.all(np.isinf(V[over]) & (np.sign(V[over]) == np.sign(ref[over])))
    assert np.all(np.isfinite(V[~over]))
