"""dar_attn_decode_noalloc (the decode for callers that cannot allocate:
its scratch is the library's static per-GPU array) against dar_attn_decode
with a caller workspace, through the C ABI: identical bytes, on two calls in a
row, the second on a smaller problem (other shapes, fewer chunks, so stale
partials of the first call would show), then the first problem again.  Also
checked against the fp64 oracle at 2e-2."""
import numpy as np
import pytest
import torch

import dar_inputs as di
import distance_adaptive_dual_amd as dar
import oracle
from gpu_helpers import TOL, dev, dev_w, host, log, max_err

pytestmark = pytest.mark.gpu


def _case(B, ctx, d, H, d_k, dd, w, seed):
    inp = di.decode_inputs(B, ctx, d, H, d_k, dd, w, seed0=seed)
    W_up, W_K, W_V = (dev_w(inp[k], "bf16") for k in ("W_up", "W_K", "W_V"))
    Wk, Wv = dar.dar_fold(W_up, W_K, W_V, H, d_k)
    t = {k: dev(inp[k], "bf16") for k in ("q", "K_win", "V_win", "h_D")}
    return inp, t, Wk, Wv


def _both(t, Wk, Wv, ctx, w):
    B, H, d_k = t["q"].shape
    o_ws = dar.dar_attn_decode(t["q"], t["K_win"], t["V_win"], t["h_D"], Wk, Wv, ctx, w)
    o_na = torch.full((B, H * d_k), float("nan"), dtype=torch.bfloat16, device="cuda")
    dar.dar_attn_decode_noalloc(t["q"], t["K_win"], t["V_win"], t["h_D"], Wk, Wv, ctx, w, o_na)
    torch.cuda.synchronize()
    return o_ws, o_na


def test_noalloc_decode_matches_workspace_decode():
    big = (4, 5000, 512, 8, 128, 256, 256)
    small = (2, 1200, 256, 4, 64, 128, 64)
    cases = [("big", big, 71), ("small", small, 72), ("big again", big, 73)]
    for name, (B, ctx, d, H, d_k, dd, w), seed in cases:
        log("noalloc decode %s: B%d ctx%d H%d dk%d dd%d w%d" % (name, B, ctx, H, d_k, dd, w))
        inp, t, Wk, Wv = _case(B, ctx, d, H, d_k, dd, w, seed)
        o_ws, o_na = _both(t, Wk, Wv, ctx, w)
        assert torch.equal(o_ws, o_na), name
        ref = oracle.decode(inp["q"], inp["K_win"], inp["V_win"], inp["h_D"], inp["W_up"],
                            inp["W_K"], inp["W_V"], ctx, w)
        err = max_err(host(o_na), ref)
        log("  max err vs oracle %.3g" % err)
        assert err <= TOL["bf16"]
