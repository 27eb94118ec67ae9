"""Ragged batches through the C ABI: sequences of different lengths in one
call (dar_cache_from_prefill_varlen, dar_decode_append_varlen,
dar_attn_decode_varlen).  Each is checked against the same call made one
sequence at a time (bit-exact where the work is the same per row) or against
the fp64 oracle per sequence (bf16 I/O, max-abs 2e-2)."""
import numpy as np
import pytest
import torch

import dar_inputs as di
import distance_adaptive_dual_amd as dar
import oracle
from gpu_helpers import TOL, dev, dev_w, host, log, max_err, prefill_case

pytestmark = pytest.mark.gpu


def ivec(vals):
    return torch.tensor(vals, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("lens,d,H,d_k,dd,w", [
    ((1000, 37, 513, 129), 512, 4, 128, 256, 128),   # one short of, one past, the window
    ((1, 700, 64, 65), 256, 4, 64, 64, 64),           # first token; exactly one latent
    ((300, 2100), 256, 2, 128, 512, 256),             # d_down 512
    ((50, 400, 999), 256, 4, 64, 128, 0),             # no window: every key rebuilt
])
def test_decode_varlen_matches_oracle_per_sequence(lens, d, H, d_k, dd, w):
    B, max_ctx = len(lens), max(lens)
    inp = di.decode_inputs(B, max_ctx, d, H, d_k, dd, w, seed0=7000 + max_ctx + w)
    log("decode varlen lens %s d%d H%d dk%d dd%d w%d" % (lens, d, H, d_k, dd, w))
    W_up, W_K, W_V = (dev_w(inp[k], "bf16") for k in ("W_up", "W_K", "W_V"))
    Wk, Wv = dar.dar_fold(W_up, W_K, W_V, H, d_k)
    q, h_D = dev(inp["q"], "bf16"), dev(inp["h_D"], "bf16")
    K_win = dev(inp["K_win"], "bf16") if w else None
    V_win = dev(inp["V_win"], "bf16") if w else None
    o = dar.dar_attn_decode_varlen(q, K_win, V_win, h_D, Wk, Wv, ivec(lens), max_ctx, w)
    o_uni = [dar.dar_attn_decode(q[b:b + 1].contiguous(),
                                 K_win[b:b + 1].contiguous() if w else None,
                                 V_win[b:b + 1].contiguous() if w else None,
                                 h_D[b:b + 1].contiguous(), Wk, Wv, lens[b], w)
             for b in range(B)]
    torch.cuda.synchronize()
    got = host(o)
    for b in range(B):
        sl = slice(b, b + 1)
        ref = oracle.decode(inp["q"][sl], inp["K_win"][sl] if w else None,
                            inp["V_win"][sl] if w else None, inp["h_D"][sl], inp["W_up"],
                            inp["W_K"], inp["W_V"], lens[b], w)
        err = max_err(got[sl], ref)
        err_u = max_err(got[sl], host(o_uni[b]))
        log("  seq %d ctx %d: vs oracle %.3g, vs one-sequence call %.3g" % (b, lens[b], err, err_u))
        assert err <= TOL["bf16"]
        assert err_u <= 1e-2


def test_append_varlen_matches_per_sequence_calls():
    B, d, H, d_k, dd, w, cap = 3, 256, 4, 64, 64, 16, 200
    pos = (5, 130, 16)
    rng = np.random.default_rng(77)
    W = {k: dev_w(rng.standard_normal(s) / np.sqrt(s[0]), "bf16") for k, s in
         (("W_down", (d, dd)), ("W_Q", (d, H * d_k)), ("W_K", (d, H * d_k)),
          ("W_V", (d, H * d_k)))}
    h = dev(rng.standard_normal((B, d)), "bf16")

    def fresh():  # random caches, so untouched rows and slots are compared too
        g = torch.Generator(device="cuda").manual_seed(5)
        mk = lambda *s: torch.randn(*s, generator=g, device="cuda").to(torch.bfloat16)
        return (mk(B, H, d_k), mk(B, H, w, d_k), mk(B, H, w, d_k), mk(B, cap, dd))

    q, Kw, Vw, Lc = fresh()
    dar.dar_decode_append_varlen(h, W["W_down"], W["W_Q"], W["W_K"], W["W_V"], H, d_k, ivec(pos),
                                 q, Kw, Vw, Lc)
    q2, Kw2, Vw2, Lc2 = fresh()
    for b in range(B):
        qb = torch.empty((1, H, d_k), dtype=torch.bfloat16, device="cuda")
        Kb, Vb, Lb = (x[b:b + 1].clone() for x in (Kw2, Vw2, Lc2))
        dar.dar_decode_append(h[b:b + 1].contiguous(), W["W_down"], W["W_Q"], W["W_K"],
                              W["W_V"], H, d_k, pos[b], qb, Kb, Vb, Lb)
        q2[b], Kw2[b], Vw2[b], Lc2[b] = qb[0], Kb[0], Vb[0], Lb[0]
    torch.cuda.synchronize()
    for name, a, e in (("q", q, q2), ("K_win", Kw, Kw2), ("V_win", Vw, Vw2), ("h_D", Lc, Lc2)):
        assert torch.equal(a, e), name


@pytest.mark.parametrize("lens,w,d_k", [((300, 17, 150), 64, 64), ((90, 200), 128, 128)])
def test_cache_varlen_matches_per_sequence_calls(lens, w, d_k):
    B, N, d, H, dd = len(lens), max(lens), 256, 2, 64
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=31 + N)
    W = {k: dev_w(inp[k], "bf16") for k in ("W_down", "W_up", "W_Q", "W_K", "W_V")}
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    out = dar.dar_project(dev(inp["h"], "bf16"), W["W_down"], W["W_up"], W["W_Q"], W["W_K"],
                          W["W_V"], H, d_k, W_upK=Wk, W_upV=Wv)
    Lc, Kw, Vw = dar.dar_cache_from_prefill_varlen(out["h_D"], out["K_loc"], out["V_loc"],
                                                   ivec(lens), w, cap=N + 4)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        Lb, Kb, Vb = dar.dar_cache_from_prefill(
            out["h_D"][b:b + 1, :n].contiguous(), out["K_loc"][b:b + 1, :, :n].contiguous(),
            out["V_loc"][b:b + 1, :, :, :n].contiguous(), w, cap=N + 4)
        torch.cuda.synchronize()
        assert torch.equal(Lc[b, :n], Lb[0, :n])
        assert torch.equal(Kw[b], Kb[0]) and torch.equal(Vw[b], Vb[0])


@pytest.mark.parametrize("lens,w,d_k,dd", [((300, 41, 177), 64, 64, 128),
                                           ((129, 400), 128, 128, 64)])
def test_ragged_batch_inference_loop(lens, w, d_k, dd):
    """A padded batch of prompts of lengths N_b: prefill, the ragged cache,
    one appended token per sequence at its own position N_b, and the ragged
    decode give row N_b of each sequence's own prefill (oracle)."""
    B, d, H = len(lens), 256, 4
    Nmax = max(lens)
    inp = prefill_case(B, Nmax + 1, d, H, d_k, dd, "bf16", seed=4040 + Nmax)
    W = {k: dev_w(inp[k], "bf16") for k in ("W_down", "W_up", "W_Q", "W_K", "W_V")}
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    h = dev(inp["h"], "bf16")
    out = dar.dar_project(h[:, :Nmax].contiguous(), W["W_down"], W["W_up"], W["W_Q"], W["W_K"],
                          W["W_V"], H, d_k, W_upK=Wk, W_upV=Wv)
    n_b = ivec(lens)
    Lc, Kw, Vw = dar.dar_cache_from_prefill_varlen(out["h_D"], out["K_loc"], out["V_loc"], n_b,
                                                   w, cap=Nmax + 1)
    nxt = torch.stack([h[b, lens[b]] for b in range(B)]).contiguous()
    q = torch.empty((B, H, d_k), dtype=torch.bfloat16, device="cuda")
    dar.dar_decode_append_varlen(nxt, W["W_down"], W["W_Q"], W["W_K"], W["W_V"], H, d_k, n_b, q,
                                 Kw, Vw, Lc)
    o = dar.dar_attn_decode_varlen(q, Kw, Vw, Lc, Wk, Wv, ivec([n + 1 for n in lens]), Nmax + 1,
                                   w)
    torch.cuda.synchronize()
    ref, _, _ = oracle.prefill(inp, H, d_k, w)
    got = host(o)
    for b, n in enumerate(lens):
        err = max_err(got[b:b + 1], ref[b:b + 1, n])
        log("  seq %d: decode at position %d vs prefill row: err %.3g" % (b, n, err))
        assert err <= TOL["bf16"]
