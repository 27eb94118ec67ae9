"""GPU parity of the decoupled-RoPE variant's prefill path, through the C ABI,
against the fp64 oracle (dar_oracle_project_drope / dar_oracle_attend_drope):
the projections (dar_project_drope), the fused attention
(dar_attn_prefill_drope), the cache built from a prompt
(dar_cache_from_prefill_drope) and the token append (dar_decode_append_drope)
feeding the variant's decode.  bf16 I/O, max-abs 2e-2."""
import numpy as np
import pytest
import torch

import dar_inputs as di
import distance_adaptive_dual_amd as dar
import oracle
from gpu_helpers import TOL, dev, dev_w, host, log, max_err

pytestmark = pytest.mark.gpu

D_R = 64
WNAMES = ("W_down", "W_up", "W_Q", "W_K", "W_V", "W_QR", "W_KR")


def wdev(inp):
    return {k: dev_w(inp[k], "bf16") for k in WNAMES}


def project(inp, H, d_k, fold=True, pos0=0, h=None):
    W = wdev(inp)
    Wk = Wv = None
    if fold:
        Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    h = dev(inp["h"], "bf16") if h is None else h
    out = dar.dar_project_drope(h, W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"],
                                W["W_QR"], W["W_KR"], H, d_k, W_upK=Wk, W_upV=Wv, pos0=pos0)
    return out, W, Wk, Wv


def check_projections(out, P):
    """Every stored projection against the oracle's: max-abs 2e-2 plus the
    rounding of the 16-bit operands, which scales with the row's magnitude."""
    pairs = [("QC", P["QC"]), ("QR", P["QR"]), ("K_loc", P["KL"]),
             ("V_loc", P["VL"].transpose(0, 1, 3, 2)), ("h_D", P["hD"]), ("K_glob", P["KG"]),
             ("V_glob", P["VG"].transpose(0, 1, 3, 2)), ("KR", P["KR"])]
    for name, ref in pairs:
        got = host(out[name])
        axis = 2 if name in ("V_loc", "V_glob") else -1
        rms = np.sqrt(np.mean(ref ** 2, axis=axis, keepdims=True))
        bound = TOL["bf16"] + 1e-2 * np.abs(ref) + 1e-2 * rms
        err = np.abs(got - ref)
        assert np.all(err <= bound), "%s: max err %.3g" % (name, err.max())


# ------------------------------------------------------------------ end to end
@pytest.mark.parametrize("B,N,d,H,d_k,dd,w,fold,pos0", [
    (2, 256, 256, 4, 64, 128, 64, True, 0),
    (1, 333, 256, 2, 128, 64, 100, True, 0),     # ragged N, d_k 128
    (2, 200, 512, 8, 64, 256, 0, False, 0),      # w = 0, W_up applied unfolded
    (1, 150, 256, 4, 128, 128, 1, True, 17),     # w = 1, positions from 17
    (2, 97, 256, 2, 64, 64, 500, True, 0),       # w >= N: every pair local
    (1, 7, 128, 2, 64, 32, 3, True, 0),          # fewer tokens than one tile
    (1, 520, 512, 16, 128, 256, 128, True, 0),   # 16 heads, several key tiles
])
def test_drope_prefill(B, N, d, H, d_k, dd, w, fold, pos0):
    log("drope prefill B%d N%d d%d H%d dk%d dd%d w%d fold%d pos0 %d"
        % (B, N, d, H, d_k, dd, w, fold, pos0))
    inp = di.drope_prefill_inputs(B, N, d, H, d_k, dd, D_R, seed0=31 * N + w)
    out, _, _, _ = project(inp, H, d_k, fold=fold, pos0=pos0)
    o = dar.dar_attn_prefill_drope(out, w)
    torch.cuda.synchronize()
    P = oracle.project_drope(inp["h"], inp["W_down"], inp["W_up"], inp["W_Q"], inp["W_K"],
                             inp["W_V"], inp["W_QR"], inp["W_KR"], H, d_k, D_R, pos0=pos0)
    check_projections(out, P)
    ref, _ = oracle.attend_drope(P, w)
    err = max_err(host(o), ref)
    log("  max err %.3g (max |o| %.3g)" % (err, np.abs(ref).max()))
    assert err <= TOL["bf16"]


# ------------------------------------------------------------------ attention only
def _attn_inputs(B, H, N, d_k, seed, std=1.0):
    """fp16-representable Gaussian operands of the fused attention: content
    queries and keys [B,H,N,d_k], values [B,H,N,d_k], rotary parts QR
    [B,H,N,d_R] and KR [B,N,d_R] (drawn already rotated)."""
    sh = (B, H, N, d_k)
    P = {k: di.gaussian(seed + i, sh, std, "f16")
         for i, k in enumerate(("QC", "KL", "VL", "KG", "VG"))}
    P["QR"] = di.gaussian(seed + 5, (B, H, N, D_R), std, "f16")
    P["KR"] = di.gaussian(seed + 6, (B, N, D_R), std, "f16")
    return P


def _attn_gpu(P, w):
    t = {k: dev(P[k], "f16") for k in ("QC", "QR", "KR")}
    t["K_loc"], t["K_glob"] = dev(P["KL"], "f16"), dev(P["KG"], "f16")
    # values token-innermost, as dar_project_drope stores them
    t["V_loc"] = dev(P["VL"].transpose(0, 1, 3, 2), "f16")
    t["V_glob"] = dev(P["VG"].transpose(0, 1, 3, 2), "f16")
    o = dar.dar_attn_prefill_drope(t, w)
    torch.cuda.synchronize()
    return host(o)


@pytest.mark.parametrize("B,H,N,d_k,w", [
    (1, 2, 1, 64, 4),          # a single token
    (2, 3, 129, 64, 64),       # one key past a tile
    (1, 2, 300, 128, 0),       # no window
    (1, 2, 255, 128, 255),     # window = N - 0: boundary on the last key
    (2, 1, 640, 64, 200),      # window not a multiple of the tile
])
def test_drope_attention_only(B, H, N, d_k, w):
    P = _attn_inputs(B, H, N, d_k, seed=5 * N + w, std=0.5)
    got = _attn_gpu(P, w)
    ref, rs = oracle.attend_drope(P, w)
    assert np.allclose(rs, 1.0)
    err = max_err(got, ref)
    log("  drope attention B%d H%d N%d dk%d w%d: max err %.3g" % (B, H, N, d_k, w, err))
    assert err <= TOL["bf16"]


def test_drope_attention_rotary_part_matters():
    """The rotary scores move the output: the same content operands with the
    rotary operands zeroed give the content-only attention scaled by
    1/sqrt(d_k + d_R), which differs from the full result."""
    B, H, N, d_k, w = 1, 2, 200, 64, 50
    P = _attn_inputs(B, H, N, d_k, seed=123, std=1.0)
    P0 = dict(P, QR=np.zeros_like(P["QR"]), KR=np.zeros_like(P["KR"]))
    got, got0 = _attn_gpu(P, w), _attn_gpu(P0, w)
    ref0, _ = oracle.attend_drope(P0, w)
    assert max_err(got0, ref0) <= TOL["bf16"]
    assert max_err(got, got0) > 10 * TOL["bf16"]


def test_drope_1b_layer_slices():
    """B4, N8192, d2048, 16 heads of 128 (d_R 64), w512, d_down 512: the
    full-size launch.  Two (batch, head) slices checked in full: every output
    row, the slice's projections and the batch's h^D and rotary keys (the
    oracle runs on one batch and one head at a time)."""
    B, N, d, H, d_k, w, dd = 4, 8192, 2048, 16, 128, 512, 512
    inp = di.drope_prefill_inputs(B, N, d, H, d_k, dd, D_R, seed0=4100)
    out, _, _, _ = project(inp, H, d_k)
    o = dar.dar_attn_prefill_drope(out, w)
    torch.cuda.synchronize()
    for b, hh in [(0, 3), (3, 14)]:
        P = oracle.project_drope(inp["h"][b:b + 1], inp["W_down"], inp["W_up"], inp["W_Q"],
                                 inp["W_K"], inp["W_V"], inp["W_QR"], inp["W_KR"], H, d_k, D_R,
                                 heads=(hh, hh + 1))
        S = {k: np.ascontiguousarray(P[k][:, hh:hh + 1])
             for k in ("QC", "QR", "KL", "VL", "KG", "VG")}
        S["KR"] = P["KR"]
        sl = {k: out[k][b:b + 1, hh:hh + 1]
              for k in ("QC", "QR", "K_loc", "V_loc", "K_glob", "V_glob")}
        sl["h_D"], sl["KR"] = out["h_D"][b:b + 1], out["KR"][b:b + 1]
        check_projections(sl, dict(S, hD=P["hD"]))
        ref, _ = oracle.attend_drope(S, w)
        got = host(o[b:b + 1, :, hh * d_k:(hh + 1) * d_k])
        err = max_err(got, ref)
        log("  drope 1b b%d h%d every row: max err %.3g" % (b, hh, err))
        assert err <= TOL["bf16"]


# ------------------------------------------------------------------ cache and append
@pytest.mark.parametrize("B,N,H,d_k,dd,w,cap", [
    (2, 100, 4, 64, 64, 16, 128),
    (1, 10, 2, 128, 32, 32, 16),     # prompt shorter than the window
    (2, 40, 2, 64, 64, 0, 40),       # no window
])
def test_drope_cache_from_prefill_exact(B, N, H, d_k, dd, w, cap):
    """Latent rows and rotary keys 0..N-1 and the ring slots of positions
    max(0, N-w)..N-1 are the prefill values rounded fp16 -> bf16; every other
    row and slot is left as it was."""
    g = np.random.Generator(np.random.PCG64(3000 + N))
    hD = di.round_f16(g.standard_normal((B, N, dd)))
    KR = di.round_f16(g.standard_normal((B, N, D_R)))
    KL = di.round_f16(g.standard_normal((B, H, N, d_k)))
    VL = di.round_f16(g.standard_normal((B, H, d_k, N)))
    P = {"h_D": dev(hD, "f16"), "KR": dev(KR, "f16"), "K_loc": dev(KL, "f16"),
         "V_loc": dev(VL, "f16")}
    L, Kw, Vw, KRc = dar.dar_cache_from_prefill_drope(P, w, cap=cap)
    torch.cuda.synchronize()
    Lg, KRg = host(L), host(KRc)
    assert np.array_equal(Lg[:, :N], di.round_bf16(hD))
    assert np.array_equal(KRg[:, :N], di.round_bf16(KR))
    assert not Lg[:, N:].any() and not KRg[:, N:].any()
    if w:
        Kg, Vg = host(Kw), host(Vw)
        seen = np.zeros(w, bool)
        for j in range(max(0, N - w), N):
            s = j % w
            seen[s] = True
            assert np.array_equal(Kg[:, :, s], di.round_bf16(KL[:, :, j]))
            assert np.array_equal(Vg[:, :, s], di.round_bf16(VL[:, :, :, j]))
        assert not Kg[:, :, ~seen].any() and not Vg[:, :, ~seen].any()


@pytest.mark.parametrize("B,d,H,d_k,dd,w,pos,cap", [
    (2, 256, 4, 64, 128, 16, 37, 64),
    (1, 512, 2, 128, 256, 0, 5, 8),      # no window
    (3, 256, 8, 64, 64, 1, 0, 4),        # first position, one-slot window
])
def test_drope_decode_append(B, d, H, d_k, dd, w, pos, cap):
    """dar_decode_append_drope writes qC, qR, ring slot pos mod w, latent row
    pos and rotary key pos (the oracle's projections of the token at pos) and
    nothing else."""
    inp = di.drope_prefill_inputs(B, 1, d, H, d_k, dd, D_R, seed0=950 + pos)
    W = wdev(inp)
    g = np.random.Generator(np.random.PCG64(77 + pos))
    K0 = di.round_bf16(g.standard_normal((B, H, max(w, 1), d_k)))
    V0 = di.round_bf16(g.standard_normal((B, H, max(w, 1), d_k)))
    L0 = di.round_bf16(g.standard_normal((B, cap, dd)))
    R0 = di.round_bf16(g.standard_normal((B, cap, D_R)))
    Kd, Vd, Ld, Rd = dev(K0, "bf16"), dev(V0, "bf16"), dev(L0, "bf16"), dev(R0, "bf16")
    qC = torch.empty((B, H, d_k), dtype=torch.bfloat16, device="cuda")
    qR = torch.empty((B, H, D_R), dtype=torch.bfloat16, device="cuda")
    dar.dar_decode_append_drope(dev(inp["h"][:, 0], "bf16"), W["W_down"], W["W_Q"], W["W_K"],
                                W["W_V"], W["W_QR"], W["W_KR"], H, d_k, pos, qC, qR,
                                Kd if w else None, Vd if w else None, Ld, Rd)
    torch.cuda.synchronize()
    P = oracle.project_drope(inp["h"], inp["W_down"], inp["W_up"], inp["W_Q"], inp["W_K"],
                             inp["W_V"], inp["W_QR"], inp["W_KR"], H, d_k, D_R, pos0=pos)
    assert max_err(host(qC), P["QC"][:, :, 0]) <= TOL["bf16"]
    assert max_err(host(qR), P["QR"][:, :, 0]) <= TOL["bf16"]
    mask = np.ones(cap, bool)
    mask[pos] = False
    Lg, Rg = host(Ld), host(Rd)
    assert max_err(Lg[:, pos], P["hD"][:, 0]) <= TOL["bf16"]
    assert max_err(Rg[:, pos], P["KR"][:, 0]) <= TOL["bf16"]
    assert np.array_equal(Lg[:, mask], L0[:, mask])
    assert np.array_equal(Rg[:, mask], R0[:, mask])
    Kg, Vg = host(Kd), host(Vd)
    if w:
        s = pos % w
        assert max_err(Kg[:, :, s], P["KL"][:, :, 0]) <= TOL["bf16"]
        assert max_err(Vg[:, :, s], P["VL"][:, :, 0]) <= TOL["bf16"]
        m2 = np.ones(w, bool)
        m2[s] = False
        assert np.array_equal(Kg[:, :, m2], K0[:, :, m2])
        assert np.array_equal(Vg[:, :, m2], V0[:, :, m2])
    else:
        assert np.array_equal(Kg, K0) and np.array_equal(Vg, V0)


@pytest.mark.parametrize("N,w,d_k,dd", [(700, 100, 64, 128), (333, 512, 128, 256)])
def test_drope_prefill_cache_append_decode(N, w, d_k, dd):
    """The variant's inference loop on the GPU: prefill a prompt of N tokens,
    build the decode cache from it, append token N and decode it; the output
    equals row N of the oracle's prefill of the variant over N+1 tokens."""
    B, d, H = 2, 256, 4
    inp = di.drope_prefill_inputs(B, N + 1, d, H, d_k, dd, D_R, seed0=818 + N)
    h = dev(inp["h"], "bf16")
    out, W, Wk, Wv = project(inp, H, d_k, h=h[:, :N].contiguous())
    o_pre = dar.dar_attn_prefill_drope(out, w)
    L, Kw, Vw, KRc = dar.dar_cache_from_prefill_drope(out, w, cap=N + 1)
    qC = torch.empty((B, H, d_k), dtype=torch.bfloat16, device="cuda")
    qR = torch.empty((B, H, D_R), dtype=torch.bfloat16, device="cuda")
    dar.dar_decode_append_drope(h[:, N].contiguous(), W["W_down"], W["W_Q"], W["W_K"], W["W_V"],
                                W["W_QR"], W["W_KR"], H, d_k, N, qC, qR, Kw, Vw, L, KRc)
    o = dar.dar_attn_decode_drope(qC, qR, Kw, Vw, KRc, L, Wk, Wv, N + 1, w)
    torch.cuda.synchronize()
    ref, _, _ = oracle.prefill_drope(inp, H, d_k, D_R, w)
    err_pre = max_err(host(o_pre), ref[:, :N])
    err = max_err(host(o), ref[:, N])
    log("  drope prefill rows err %.3g; decode of row %d err %.3g" % (err_pre, N, err))
    assert err_pre <= TOL["bf16"]
    assert err <= TOL["bf16"]
