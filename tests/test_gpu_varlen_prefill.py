"""GPU parity of the ragged (unpadded) prefill: dar_project_varlen and
dar_attn_prefill_varlen over prompts of different lengths packed without
padding, each prompt against the fp64 oracle's prefill of that prompt alone
(its own positions from 0), through the C ABI.  bf16 I/O, max-abs 2e-2.
dar_cache_from_prefill_packed is checked bit-exact (index moves and one
fp16 -> bf16 rounding) and through the whole loop to the next token's decode."""
import numpy as np
import pytest
import torch

import dar_inputs as di
import distance_adaptive_dual_amd as dar
import oracle
from gpu_helpers import TOL, dev, dev_w, host, log, max_err

pytestmark = pytest.mark.gpu

WNAMES = ("W_down", "W_up", "W_Q", "W_K", "W_V")


def ragged_case(lens, d, H, d_k, dd, seed):
    """Shared weights (prefill_inputs' draws) and one Gaussian h per prompt."""
    base = di.prefill_inputs(1, 1, d, H, d_k, dd, dtype="bf16", seed0=seed)
    hs = [di.gaussian(seed + 100 + b, (1, n, d), 1.0, "bf16") for b, n in enumerate(lens)]
    return base, hs


def run_ragged(base, hs, lens, H, d_k, w):
    W = {k: dev_w(base[k], "bf16") for k in WNAMES}
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    h = dev(np.concatenate([x[0] for x in hs], axis=0), "bf16")
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu = torch.from_numpy(starts).cuda()
    P = dar.dar_project_varlen(h, W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"], H, d_k,
                               cu, max(lens), W_upK=Wk, W_upV=Wv)
    o = dar.dar_attn_prefill_varlen(P, cu, max(lens), H, d_k, w)
    torch.cuda.synchronize()
    return P, o, starts


def check_block(name, got, ref):
    """A projection block against the oracle's, with the 16-bit storage term
    the dense projection tests use (scaled by the row's rms)."""
    axis = -2 if name in ("V_loc", "V_glob") else -1  # a token's d_k values
    rms = np.sqrt(np.mean(ref ** 2, axis=axis, keepdims=True))
    bound = TOL["bf16"] + 1e-2 * np.abs(ref) + 1e-2 * rms
    err = np.abs(got - ref)
    assert np.all(err <= bound), "%s: max err %.3g" % (name, err.max())


@pytest.mark.parametrize("lens,d,H,d_k,dd,w", [
    ([300, 77, 1, 512, 129], 256, 4, 64, 64, 100),
    ([64, 200, 33], 256, 2, 128, 128, 0),       # w = 0: every pair global
    ([500, 17, 250], 512, 4, 128, 256, 1),     # w = 1
    ([96, 96], 256, 4, 64, 64, 1000),          # w beyond every length: all local
    ([1], 128, 2, 64, 32, 4),                  # one prompt of one token
])
def test_ragged_prefill(lens, d, H, d_k, dd, w):
    log("ragged prefill lens %s d%d H%d dk%d dd%d w%d" % (lens, d, H, d_k, dd, w))
    base, hs = ragged_case(lens, d, H, d_k, dd, seed=41 * len(lens) + w)
    P, o, starts = run_ragged(base, hs, lens, H, d_k, w)
    og = host(o)
    names = {"Q": "Q", "K_loc": "KL", "V_loc": "VL", "K_glob": "KG", "V_glob": "VG"}
    for b, n in enumerate(lens):
        inp = dict(base, h=hs[b])
        ref, _, R = oracle.prefill(inp, H, d_k, w)
        err = max_err(og[starts[b]:starts[b + 1]], ref[0])
        log("  prompt %d (%d tokens): max err %.3g" % (b, n, err))
        assert err <= TOL["bf16"]
        for k, rk in names.items():
            tr = k in ("V_loc", "V_glob")
            got = host(dar.varlen_block(P[k], starts, b, H, d_k, transposed=tr))
            refb = R[rk][0].transpose(0, 2, 1) if tr else R[rk][0]
            check_block(k, got, refb)
        check_block("h_D", host(P["h_D"][starts[b]:starts[b + 1]]), R["hD"][0])


def test_ragged_matches_padded_batch():
    """The same prompts prefilled padded (dar_project + dar_attn_prefill at the
    longest length, shorter prompts zero-padded at the end) give the same
    rows up to rounding: causality keeps padding out of the real rows.  (Not
    bit for bit: the RoPE epilogue forms the angles of groups of four
    consecutive rows by one table lookup and complex steps, and the groups
    fall differently in the two layouts.)"""
    lens, d, H, d_k, dd, w = [150, 64, 233], 256, 4, 64, 64, 50
    base, hs = ragged_case(lens, d, H, d_k, dd, seed=515)
    _, o, starts = run_ragged(base, hs, lens, H, d_k, w)
    N = max(lens)
    hp = np.zeros((len(lens), N, d))
    for b, n in enumerate(lens):
        hp[b, :n] = hs[b][0]
    W = {k: dev_w(base[k], "bf16") for k in WNAMES}
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    out = dar.dar_project(dev(hp, "bf16"), W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"], H,
                          d_k, W_upK=Wk, W_upV=Wv)
    op = dar.dar_attn_prefill(out["Q"], out["K_loc"], out["V_loc"], out["K_glob"], out["V_glob"],
                              w)
    torch.cuda.synchronize()
    og, opd = host(o), host(op)
    for b, n in enumerate(lens):
        err = max_err(og[starts[b]:starts[b + 1]], opd[b, :n])
        log("  prompt %d: ragged vs padded max diff %.3g" % (b, err))
        assert err <= 4e-3, b


def test_ragged_prefill_1b_width():
    """d2048, 16 heads of 128, d_down 512, w512 over 10 297 packed tokens (the
    first projection runs the wide-tile GEMM): two prompts checked on one head
    each, every row, and that head's projection blocks."""
    lens, d, H, d_k, dd, w = [4096, 3000, 1, 2500, 700], 2048, 16, 128, 512, 512
    base, hs = ragged_case(lens, d, H, d_k, dd, seed=1234)
    P, o, starts = run_ragged(base, hs, lens, H, d_k, w)
    og = host(o)
    for b, hh in [(1, 5), (4, 12)]:
        inp = dict(base, h=hs[b])
        R = oracle.project(inp["h"], inp["W_down"], inp["W_up"], inp["W_Q"], inp["W_K"],
                           inp["W_V"], H, d_k, heads=(hh, hh + 1))
        S = {k: np.ascontiguousarray(R[k][:, hh:hh + 1]) for k in ("Q", "KL", "VL", "KG", "VG")}
        ref, _ = oracle.attend(S, w)
        got = og[starts[b]:starts[b + 1], hh * d_k:(hh + 1) * d_k]
        err = max_err(got, ref[0])
        log("  1b-width prompt %d head %d: max err %.3g" % (b, hh, err))
        assert err <= TOL["bf16"]
        for k, rk in (("Q", "Q"), ("K_glob", "KG"), ("V_loc", "VL")):
            tr = k == "V_loc"
            blk = host(dar.varlen_block(P[k], starts, b, H, d_k, transposed=tr))[hh]
            refb = S[rk][0, 0].T if tr else S[rk][0, 0]
            check_block(k, blk, refb)


@pytest.mark.parametrize("lens,w,d_k,dd", [([300, 17, 1, 150], 64, 64, 64),
                                           ([90, 200], 128, 128, 128),
                                           ([5, 40], 0, 64, 32)])
def test_packed_cache_exact(lens, w, d_k, dd):
    """dar_cache_from_prefill_packed on seeded fp16 packed blocks: every latent
    row and ring slot is the fp16 value rounded to bf16, and every row and slot
    it must not write keeps its earlier contents."""
    log("packed cache lens %s w%d dk%d dd%d" % (lens, w, d_k, dd))
    H, B, T, N = 3, len(lens), sum(lens), max(lens)
    cap = N + 7
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    g = torch.Generator().manual_seed(97 + T + w)
    P = {k: torch.randn(T * H * d_k, generator=g).to(torch.float16) for k in ("K_loc", "V_loc")}
    P["h_D"] = torch.randn((T, dd), generator=g).to(torch.float16)
    Lc0 = torch.randn((B, cap, dd), generator=g).to(torch.bfloat16)
    Kw0 = torch.randn((B, H, max(w, 1), d_k), generator=g).to(torch.bfloat16)
    Vw0 = torch.randn((B, H, max(w, 1), d_k), generator=g).to(torch.bfloat16)
    Pd = {k: v.cuda() for k, v in P.items()}
    Lc, Kw, Vw = Lc0.cuda(), Kw0.cuda(), Vw0.cuda()
    dar.dar_cache_from_prefill_packed(Pd, torch.from_numpy(starts).cuda(), N, H, d_k, w, cap=cap,
                                      h_D_cache=Lc, K_win=Kw if w else None,
                                      V_win=Vw if w else None)
    torch.cuda.synchronize()
    eL, eK, eV = Lc0.clone(), Kw0.clone(), Vw0.clone()
    for b, n in enumerate(lens):
        eL[b, :n] = P["h_D"][starts[b]:starts[b + 1]].to(torch.bfloat16)
        if w == 0:
            continue
        K = varlen_cpu(P["K_loc"], starts, b, H, d_k, False)
        V = varlen_cpu(P["V_loc"], starts, b, H, d_k, True)
        for j in range(max(0, n - w), n):
            eK[b, :, j % w] = K[:, j].to(torch.bfloat16)
            eV[b, :, j % w] = V[:, :, j].to(torch.bfloat16)
    assert torch.equal(Lc.cpu(), eL)
    if w:
        assert torch.equal(Kw.cpu(), eK) and torch.equal(Vw.cpu(), eV)


def varlen_cpu(x, starts, b, H, d_k, transposed):
    lo, hi = int(starts[b]), int(starts[b + 1])
    blk = x[lo * H * d_k:hi * H * d_k]
    return blk.view(H, d_k, hi - lo) if transposed else blk.view(H, hi - lo, d_k)


@pytest.mark.parametrize("lens,w,d_k,dd", [([300, 41, 1, 177], 64, 64, 128),
                                           ([129, 400], 128, 128, 64)])
def test_packed_prefill_inference_loop(lens, w, d_k, dd):
    """Prompts prefilled packed, their decode cache from the packed outputs, one
    appended token per prompt at position len_b and the ragged decode give row
    len_b of each prompt's own prefill (oracle, len_b + 1 tokens)."""
    log("packed prefill -> cache -> append -> decode lens %s w%d dk%d dd%d" % (lens, w, d_k, dd))
    d, H, B = 256, 4, len(lens)
    N = max(lens)
    base, hs = ragged_case([n + 1 for n in lens], d, H, d_k, dd, seed=808 + N)
    W = {k: dev_w(base[k], "bf16") for k in WNAMES}
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    h = dev(np.concatenate([x[0, :n] for x, n in zip(hs, lens)], axis=0), "bf16")
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu = torch.from_numpy(starts).cuda()
    P = dar.dar_project_varlen(h, W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"], H, d_k,
                               cu, N, W_upK=Wk, W_upV=Wv)
    Lc, Kw, Vw = dar.dar_cache_from_prefill_packed(P, cu, N, H, d_k, w, cap=N + 1)
    nxt = dev(np.stack([x[0, n] for x, n in zip(hs, lens)]), "bf16")
    pos = torch.tensor(lens, dtype=torch.int32, device="cuda")
    q = torch.empty((B, H, d_k), dtype=torch.bfloat16, device="cuda")
    dar.dar_decode_append_varlen(nxt, W["W_down"], W["W_Q"], W["W_K"], W["W_V"], H, d_k, pos, q,
                                 Kw, Vw, Lc)
    ctx = torch.tensor([n + 1 for n in lens], dtype=torch.int32, device="cuda")
    o = dar.dar_attn_decode_varlen(q, Kw, Vw, Lc, Wk, Wv, ctx, N + 1, w)
    torch.cuda.synchronize()
    got = host(o)
    for b, n in enumerate(lens):
        ref, _, _ = oracle.prefill(dict(base, h=hs[b]), H, d_k, w)
        err = max_err(got[b:b + 1], ref[0:1, n])
        log("  prompt %d: decode at position %d vs prefill row: err %.3g" % (b, n, err))
        assert err <= TOL["bf16"]
