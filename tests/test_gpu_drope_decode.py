"""GPU parity of the decoupled-RoPE variant's decode (dar_attn_decode_drope:
the folded up-projection absorbed into the query, the cache streamed as
[h^D_j ; kR_j]) against the fp64 oracle's cache form (dar_oracle_decode_drope:
content keys of old positions rebuilt from h^D through W_up, W_K in fp64),
through the C ABI.  bf16 I/O, max-abs 2e-2."""
import numpy as np
import pytest
import torch

import dar_inputs as di
import distance_adaptive_dual_amd as dar
import oracle
from gpu_helpers import TOL, dev, dev_w, host, log, max_err

pytestmark = pytest.mark.gpu


def run_drope_decode(inp, ctx, w, H, d_k):
    W_up, W_K, W_V = (dev_w(inp[k], "bf16") for k in ("W_up", "W_K", "W_V"))
    Wk, Wv = dar.dar_fold(W_up, W_K, W_V, H, d_k)
    t = {k: dev(inp[k], "bf16") for k in ("qC", "qR", "K_win", "V_win", "KR", "h_D")}
    o = dar.dar_attn_decode_drope(t["qC"], t["qR"], t["K_win"], t["V_win"], t["KR"], t["h_D"],
                                  Wk, Wv, ctx, w)
    torch.cuda.synchronize()
    return host(o)


def ref_drope_decode(inp, ctx, w, heads=None, b=None):
    sl = slice(None) if b is None else slice(b, b + 1)
    return oracle.decode_drope(inp["qC"][sl], inp["qR"][sl], inp["K_win"][sl],
                               inp["V_win"][sl], inp["KR"][sl], inp["h_D"][sl], inp["W_up"],
                               inp["W_K"], inp["W_V"], ctx, w, heads=heads)


@pytest.mark.parametrize("B,ctx,d,H,d_k,dd,w", [
    (2, 1000, 512, 4, 128, 256, 128),
    (3, 4097, 256, 4, 64, 128, 512),    # ragged context, many chunks
    (2, 300, 256, 2, 128, 256, 0),      # w = 0: every key from the latent stream
    (2, 300, 256, 4, 64, 256, 1),       # w = 1: only the query's own key in the window
    (1, 200, 256, 2, 128, 128, 500),    # w >= ctx: no latent reads
    (2, 1, 128, 2, 64, 128, 4),         # first token
    (1, 65, 512, 8, 64, 256, 64),       # exactly one latent token
    (2, 2000, 512, 16, 128, 256, 100),  # one full group of 16 heads
    (1, 1500, 512, 20, 64, 256, 64),    # two head groups, the second partial
    (2, 3000, 512, 4, 128, 512, 256),   # d_down 512
])
def test_drope_decode_small(B, ctx, d, H, d_k, dd, w):
    d_R = 64
    inp = di.drope_decode_inputs(B, ctx, d, H, d_k, dd, d_R, w, seed0=20 * ctx + w)
    log("drope decode B%d ctx%d d%d H%d dk%d dR%d dd%d w%d" % (B, ctx, d, H, d_k, d_R, dd, w))
    got = run_drope_decode(inp, ctx, w, H, d_k)
    ref = ref_drope_decode(inp, ctx, w)
    err = max_err(got, ref)
    log("  max err %.3g (max |o| %.3g)" % (err, np.abs(ref).max()))
    assert err <= TOL["bf16"]


def test_drope_decode_cap_larger_than_context():
    B, ctx, d, H, d_k, dd, w = 2, 700, 256, 4, 64, 128, 64
    inp = di.drope_decode_inputs(B, ctx, d, H, d_k, dd, 64, w, cap=1024, seed0=99)
    err = max_err(run_drope_decode(inp, ctx, w, H, d_k), ref_drope_decode(inp, ctx, w))
    assert err <= TOL["bf16"]


def test_drope_decode_matches_prefill_row():
    """The cache built from the oracle's own projections of a prompt: the
    decode at position p reproduces row p of the oracle's prefill of the
    variant."""
    B, N, d, H, d_k, dd, w = 2, 600, 256, 4, 64, 128, 100
    d_R = 64
    inp = di.drope_prefill_inputs(B, N, d, H, d_k, dd, d_R, seed0=606)
    o_ref, _, P = oracle.prefill_drope(inp, H, d_k, d_R, w)
    p = N - 1
    r = di.round_bf16
    K_win = np.zeros((B, H, w, d_k))
    V_win = np.zeros((B, H, w, d_k))
    for j in range(p - w + 1, p + 1):
        K_win[:, :, j % w] = P["KL"][:, :, j]
        V_win[:, :, j % w] = P["VL"][:, :, j]
    cache = dict(qC=r(P["QC"][:, :, p]), qR=r(P["QR"][:, :, p]), K_win=r(K_win), V_win=r(V_win),
                 KR=r(P["KR"]), h_D=r(P["hD"]), W_up=inp["W_up"], W_K=inp["W_K"],
                 W_V=inp["W_V"])
    got = run_drope_decode(cache, N, w, H, d_k)
    err = max_err(got, o_ref[:, p])
    log("  drope decode vs prefill row err %.3g" % err)
    assert err <= TOL["bf16"]


def test_drope_long_context_decode():
    """B16, ctx 32768, d2048, 16 heads of 128 (d_R 64), w512, d_down 256: the
    full-size launch, one head of every batch against the oracle."""
    B, ctx, d, H, d_k, dd, w = 16, 32768, 2048, 16, 128, 256, 512
    inp = di.drope_decode_inputs(B, ctx, d, H, d_k, dd, 64, w, seed0=8000)
    got = run_drope_decode(inp, ctx, w, H, d_k)
    for b in range(B):
        hh = (5 * b + 3) % H
        ref = ref_drope_decode(inp, ctx, w, heads=(hh, hh + 1), b=b)
        sl = slice(hh * d_k, (hh + 1) * d_k)
        err = max_err(got[b, sl], ref[0, sl])
        log("  drope long decode b%d h%d max err %.3g" % (b, hh, err))
        assert err <= TOL["bf16"]


def test_drope_decode_deterministic():
    B, ctx, d, H, d_k, dd, w = 2, 3000, 256, 4, 128, 256, 256
    inp = di.drope_decode_inputs(B, ctx, d, H, d_k, dd, 64, w, seed0=77)
    assert np.array_equal(run_drope_decode(inp, ctx, w, H, d_k),
                          run_drope_decode(inp, ctx, w, H, d_k))
