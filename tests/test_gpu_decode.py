"""GPU parity of the mixed-cache decode step (dar_attn_decode) against the
fp64 oracle, through the C ABI.  bf16 I/O, max-abs 2e-2."""
import numpy as np
import pytest
import torch

import dar_inputs as di
import distance_adaptive_dual_amd as dar
import oracle
from gpu_helpers import TOL, dev, dev_w, host, log, max_err, prefill_case

pytestmark = pytest.mark.gpu


def run_decode(inp, ctx, w, H, d_k):
    W_up, W_K, W_V = (dev_w(inp[k], "bf16") for k in ("W_up", "W_K", "W_V"))
    Wk, Wv = dar.dar_fold(W_up, W_K, W_V, H, d_k)
    q = dev(inp["q"], "bf16")
    K_win = dev(inp["K_win"], "bf16")
    V_win = dev(inp["V_win"], "bf16")
    h_D = dev(inp["h_D"], "bf16")
    o = dar.dar_attn_decode(q, K_win, V_win, h_D, Wk, Wv, ctx, w)
    torch.cuda.synchronize()
    return host(o)


@pytest.mark.parametrize("B,ctx,d,H,d_k,dd,w", [
    (2, 1000, 512, 4, 128, 256, 128),
    (3, 4097, 256, 4, 64, 64, 512),     # ragged context, many chunks
    (2, 300, 256, 2, 128, 128, 0),      # w = 0: every key rebuilt from the latent
    (2, 300, 256, 4, 64, 32, 1),        # w = 1: only the query's own key is full
    (1, 200, 256, 2, 128, 128, 500),    # w >= ctx: no latent reads at all
    (2, 1, 128, 2, 64, 64, 4),          # first token
    (1, 65, 512, 8, 64, 256, 64),       # exactly one latent token
    (2, 2000, 512, 16, 128, 256, 100),  # 16 heads (several head groups)
    (2, 3000, 512, 4, 128, 512, 256),   # d_down 512: two latent slices per frequency block
    (2, 1500, 256, 4, 64, 512, 64),     # d_down 512 with 64-wide heads
])
def test_decode_small(B, ctx, d, H, d_k, dd, w):
    inp = di.decode_inputs(B, ctx, d, H, d_k, dd, w, seed0=10 * ctx + w)
    log("decode B%d ctx%d d%d H%d dk%d dd%d w%d" % (B, ctx, d, H, d_k, dd, w))
    got = run_decode(inp, ctx, w, H, d_k)
    ref = oracle.decode(inp["q"], inp["K_win"], inp["V_win"], inp["h_D"], inp["W_up"],
                        inp["W_K"], inp["W_V"], ctx, w)
    err = max_err(got, ref)
    log("  max err %.3g" % err)
    assert err <= TOL["bf16"]


def test_decode_cap_larger_than_context():
    """The latent cache may hold more rows than the context uses."""
    B, ctx, d, H, d_k, dd, w = 2, 700, 256, 4, 64, 128, 64
    inp = di.decode_inputs(B, ctx, d, H, d_k, dd, w, cap=1024, seed0=4242)
    got = run_decode(inp, ctx, w, H, d_k)
    ref = oracle.decode(inp["q"], inp["K_win"], inp["V_win"], inp["h_D"], inp["W_up"],
                        inp["W_K"], inp["W_V"], ctx, w)
    assert max_err(got, ref) <= TOL["bf16"]


def test_decode_matches_prefill_row():
    """The decode step at position p reproduces row p of the full prefill
    (oracle), with the cache filled from the oracle's own projections."""
    B, N, d, H, d_k, dd, w = 2, 600, 256, 4, 64, 128, 100
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=606)
    o_ref, _, P = oracle.prefill(inp, H, d_k, w)
    p = N - 1
    r = di.round_bf16
    K_win = np.zeros((B, H, w, d_k))
    V_win = np.zeros((B, H, w, d_k))
    for j in range(p - w + 1, p + 1):
        K_win[:, :, j % w] = P["KL"][:, :, j]
        V_win[:, :, j % w] = P["VL"][:, :, j]
    cache = dict(q=r(P["Q"][:, :, p]), K_win=r(K_win), V_win=r(V_win), h_D=r(P["hD"]),
                 W_up=inp["W_up"], W_K=inp["W_K"], W_V=inp["W_V"])
    got = run_decode(cache, N, w, H, d_k)
    err = max_err(got, o_ref[:, p])
    log("  decode vs prefill row err %.3g" % err)
    assert err <= TOL["bf16"]


def _long_decode_check(inp, got, pairs, ctx, w, d_k, label):
    for b, hh in pairs:
        ref = oracle.decode(inp["q"][b:b + 1], inp["K_win"][b:b + 1], inp["V_win"][b:b + 1],
                            inp["h_D"][b:b + 1], inp["W_up"], inp["W_K"], inp["W_V"], ctx, w,
                            heads=(hh, hh + 1))
        sl = slice(hh * d_k, (hh + 1) * d_k)
        err = max_err(got[b, sl], ref[0, sl])
        log("  %s b%d h%d max err %.3g (max |o| %.3g)" % (label, b, hh, err,
                                                          np.abs(ref[0, sl]).max()))
        assert err <= TOL["bf16"]


LONG = dict(B=16, ctx=32768, d=2048, H=16, d_k=128, dd=256, w=512)


def test_long_context_decode_planted():
    """B16, ctx 32768, d2048, 16 heads of 128, w512, d_down 256: the full-size
    launch on a cache where, for one head of every even batch, latent rows
    (at both sides of the 2016-token chunk edges, the first and the last
    global position) and window slots (oldest, middle, the query's own) carry
    keys aligned with the query, so o is of order 1 and depends on every
    part of the cache (tests/test_planted_decode_bites.py shows the
    mistakes this exposes on the CPU).  8 (batch, head) pairs, all heads
    distinct."""
    import planted
    from test_planted_decode_bites import planted_positions
    c = LONG
    inp = di.decode_inputs(c["B"], c["ctx"], c["d"], c["H"], c["d_k"], c["dd"], c["w"],
                           seed0=5000)
    pairs = [(b, (5 * b + 3) % 16) for b in range(0, 16, 2)]
    inp = planted.plant(inp, c["ctx"], c["w"], c["d_k"], pairs,
                        *planted_positions(c["ctx"], c["w"]))
    got = run_decode(inp, c["ctx"], c["w"], c["H"], c["d_k"])
    _long_decode_check(inp, got, pairs, c["ctx"], c["w"], c["d_k"], "planted decode")


def test_long_context_decode_gaussian():
    """The same launch on the workload's Gaussian cache (softmax spread over
    thousands of keys, |o| ~ 0.02): one head of every odd batch, so the two
    tests together cover every batch and every head."""
    c = LONG
    inp = di.decode_inputs(c["B"], c["ctx"], c["d"], c["H"], c["d_k"], c["dd"], c["w"],
                           seed0=5000)
    got = run_decode(inp, c["ctx"], c["w"], c["H"], c["d_k"])
    pairs = [(b, (5 * b + 3) % 16) for b in range(1, 16, 2)]
    _long_decode_check(inp, got, pairs, c["ctx"], c["w"], c["d_k"], "gaussian decode")


def test_decode_deterministic():
    B, ctx, d, H, d_k, dd, w = 2, 3000, 256, 4, 128, 128, 256
    inp = di.decode_inputs(B, ctx, d, H, d_k, dd, w, seed0=77)
    a = run_decode(inp, ctx, w, H, d_k)
    b = run_decode(inp, ctx, w, H, d_k)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("B,d,H,d_k,dd,w,pos,cap", [
    (2, 256, 4, 64, 64, 16, 100, 200),
    (3, 512, 4, 128, 128, 512, 5000, 5001),
    (2, 256, 2, 128, 32, 0, 7, 8),
])
def test_decode_append(B, d, H, d_k, dd, w, pos, cap):
    """dar_decode_append writes q, ring slot pos mod w of K/V and latent row
    pos (oracle projections of the token at position pos) and nothing else."""
    inp = prefill_case(B, 1, d, H, d_k, dd, "bf16", seed=900 + pos)
    Wd = {k: dev_w(inp[k], "bf16") for k in ("W_down", "W_Q", "W_K", "W_V")}
    h = dev(inp["h"][:, 0], "bf16")
    g = np.random.Generator(np.random.PCG64(pos))
    K0 = di.round_bf16(g.standard_normal((B, H, w, d_k)))
    V0 = di.round_bf16(g.standard_normal((B, H, w, d_k)))
    L0 = di.round_bf16(g.standard_normal((B, cap, dd)))
    K_win, V_win, h_D = dev(K0, "bf16"), dev(V0, "bf16"), dev(L0, "bf16")
    q = torch.empty((B, H, d_k), dtype=torch.bfloat16, device="cuda")
    dar.dar_decode_append(h, Wd["W_down"], Wd["W_Q"], Wd["W_K"], Wd["W_V"], H, d_k, pos, q,
                          K_win if w else None, V_win if w else None, h_D)
    torch.cuda.synchronize()
    P = oracle.project(inp["h"], inp["W_down"], inp["W_up"], inp["W_Q"], inp["W_K"], inp["W_V"],
                       H, d_k, pos0=pos)
    assert max_err(host(q), P["Q"][:, :, 0]) <= TOL["bf16"]
    Lg = host(h_D)
    assert max_err(Lg[:, pos], P["hD"][:, 0]) <= TOL["bf16"]
    mask = np.ones(cap, bool)
    mask[pos] = False
    assert np.array_equal(Lg[:, mask], L0[:, mask])
    if w:
        s = pos % w
        Kg, Vg = host(K_win), host(V_win)
        assert max_err(Kg[:, :, s], P["KL"][:, :, 0]) <= TOL["bf16"]
        assert max_err(Vg[:, :, s], P["VL"][:, :, 0]) <= TOL["bf16"]
        m2 = np.ones(w, bool)
        m2[s] = False
        assert np.array_equal(Kg[:, :, m2], K0[:, :, m2])
        assert np.array_equal(Vg[:, :, m2], V0[:, :, m2])


def test_append_then_decode_matches_prefill_row():
    """Cache for positions < p from the oracle's projections (bf16), the token
    at p appended on the GPU, then the GPU decode step: equals row p of the
    oracle's full prefill."""
    B, N, d, H, d_k, dd, w = 2, 500, 256, 4, 128, 64, 64
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=707)
    o_ref, _, P = oracle.prefill(inp, H, d_k, w)
    p = N - 1
    r = di.round_bf16
    K_win = np.zeros((B, H, w, d_k))
    V_win = np.zeros((B, H, w, d_k))
    for j in range(p - w + 1, p):
        K_win[:, :, j % w] = P["KL"][:, :, j]
        V_win[:, :, j % w] = P["VL"][:, :, j]
    hD = r(P["hD"])
    hD[:, p] = 0.0
    Kd, Vd, Ld = dev(r(K_win), "bf16"), dev(r(V_win), "bf16"), dev(hD, "bf16")
    Wd = {k: dev_w(inp[k], "bf16") for k in ("W_down", "W_up", "W_Q", "W_K", "W_V")}
    q = torch.empty((B, H, d_k), dtype=torch.bfloat16, device="cuda")
    dar.dar_decode_append(dev(inp["h"][:, p], "bf16"), Wd["W_down"], Wd["W_Q"], Wd["W_K"],
                          Wd["W_V"], H, d_k, p, q, Kd, Vd, Ld)
    Wk, Wv = dar.dar_fold(Wd["W_up"], Wd["W_K"], Wd["W_V"], H, d_k)
    o = dar.dar_attn_decode(q, Kd, Vd, Ld, Wk, Wv, N, w)
    torch.cuda.synchronize()
    err = max_err(host(o), o_ref[:, p])
    log("  append+decode vs prefill row err %.3g" % err)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("B,N,H,d_k,dd,w,cap", [
    (2, 100, 4, 64, 64, 16, 128),
    (2, 77, 2, 128, 128, 32, 80),    # ragged N (not a multiple of 8)
    (1, 10, 2, 64, 32, 32, 16),      # prompt shorter than the window
    (2, 40, 2, 64, 64, 0, 40),       # no window
])
def test_cache_from_prefill_exact(B, N, H, d_k, dd, w, cap):
    """Latent rows 0..N-1 and ring slots of positions max(0, N-w)..N-1 are the
    prefill values rounded fp16 -> bf16; every other row and slot is left as
    it was."""
    g = np.random.Generator(np.random.PCG64(1000 + N))
    hD = di.round_f16(g.standard_normal((B, N, dd)))
    KL = di.round_f16(g.standard_normal((B, H, N, d_k)))
    VL = di.round_f16(g.standard_normal((B, H, d_k, N)))
    L0 = di.round_bf16(g.standard_normal((B, cap, dd)))
    K0 = di.round_bf16(g.standard_normal((B, H, max(w, 1), d_k)))
    V0 = di.round_bf16(g.standard_normal((B, H, max(w, 1), d_k)))
    Lc = dev(L0, "bf16")
    Kw = dev(K0, "bf16") if w else None
    Vw = dev(V0, "bf16") if w else None
    dar.dar_cache_from_prefill(dev(hD, "f16"), dev(KL, "f16"), dev(VL, "f16"), w, cap=cap,
                               h_D_cache=Lc, K_win=Kw, V_win=Vw)
    torch.cuda.synchronize()
    Lg = host(Lc)
    assert np.array_equal(Lg[:, :N], di.round_bf16(hD))
    assert np.array_equal(Lg[:, N:], L0[:, N:])
    if w:
        Kg, Vg = host(Kw), host(Vw)
        K_exp, V_exp = K0.copy(), V0.copy()
        for j in range(max(0, N - w), N):
            K_exp[:, :, j % w] = di.round_bf16(KL[:, :, j])
            V_exp[:, :, j % w] = di.round_bf16(VL[:, :, :, j])
        assert np.array_equal(Kg, K_exp)
        assert np.array_equal(Vg, V_exp)


@pytest.mark.parametrize("N,w,d_k,dd", [(700, 100, 64, 128), (333, 512, 128, 64)])
def test_prefill_cache_append_decode_matches_prefill_row(N, w, d_k, dd):
    """The inference loop on the GPU: prefill a prompt of N tokens, build the
    decode cache from it, append token N and decode it; the output equals row
    N of the oracle's prefill over all N+1 tokens."""
    B, d, H = 2, 256, 4
    inp = prefill_case(B, N + 1, d, H, d_k, dd, "bf16", seed=808 + N)
    W = {k: dev_w(inp[k], "bf16") for k in ("W_down", "W_up", "W_Q", "W_K", "W_V")}
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    h = dev(inp["h"], "bf16")
    out = dar.dar_project(h[:, :N].contiguous(), W["W_down"], W["W_up"], W["W_Q"], W["W_K"],
                          W["W_V"], H, d_k, W_upK=Wk, W_upV=Wv)
    Lc, Kw, Vw = dar.dar_cache_from_prefill(out["h_D"], out["K_loc"], out["V_loc"], w, cap=N + 1)
    q = torch.empty((B, H, d_k), dtype=torch.bfloat16, device="cuda")
    dar.dar_decode_append(h[:, N].contiguous(), W["W_down"], W["W_Q"], W["W_K"], W["W_V"], H, d_k,
                          N, q, Kw, Vw, Lc)
    o = dar.dar_attn_decode(q, Kw, Vw, Lc, Wk, Wv, N + 1, w)
    torch.cuda.synchronize()
    ref, _, _ = oracle.prefill(inp, H, d_k, w)
    err = max_err(host(o), ref[:, N])
    log("  prefill -> cache -> append -> decode vs prefill row %d: err %.3g" % (N, err))
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("chunks,w,d_k,dd,H", [
    ((150, 200, 130), 100, 64, 64, 4),     # window shorter than a chunk
    ((100, 64, 250), 300, 128, 128, 2),    # window longer than the prefix
    ((60, 1, 70), 16, 64, 32, 4),          # a one-token chunk
    ((128, 100), 0, 64, 64, 4),            # no window: every pair global
])
def test_chunked_prefill_matches_prefill_rows(chunks, w, d_k, dd, H):
    """A prompt prefilled chunk by chunk over the mixed cache gives every row of
    the oracle's prefill over the whole prompt; decoding the next token after
    the last chunk gives the oracle's next row."""
    run_chunks(chunks, w, d_k, dd, H)


@pytest.mark.parametrize("chunks,w,d_k,dd,H", [
    ((128, 192, 256), 100, 128, 128, 2),   # local arrays rounded down to a key tile
    ((64, 320, 64), 300, 128, 64, 2),      # window longer than the first prefixes
    ((192, 256), 0, 128, 64, 2),           # every pair global
    ((256, 64, 128), 1, 128, 64, 2),       # only the diagonal local
])
def test_chunked_prefill_ring_tiles(chunks, w, d_k, dd, H):
    """Chunks whose ends are multiples of 64 at d_k 128 run the ring kernel
    (whole key tiles, the local arrays starting at p0 - w + 1 rounded down to
    a tile, the rows below it zero): every row matches the oracle's prefill."""
    run_chunks(chunks, w, d_k, dd, H)


def _chunk_sweep_cases(n=8, seed=4242):
    """Seeded chunk splits: d_k 128 or 64, 1-4 heads, windows from 0 to past
    the prompt, chunk ends mostly on multiples of 64 (the ring kernel at d_k
    128) and sometimes not."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        d_k = int(rng.choice([128, 64]))
        H = int(rng.integers(1, 5))
        chunks = []
        for _ in range(int(rng.integers(2, 5))):
            c = 64 * int(rng.integers(1, 6))
            if rng.random() < 0.25:
                c += int(rng.integers(1, 64))
            chunks.append(c)
        w = int(rng.choice([0, 1, int(rng.integers(2, 200)), int(rng.integers(200, 900))]))
        cases.append((tuple(chunks), w, d_k, int(rng.choice([64, 128])), H))
    return cases


@pytest.mark.parametrize("chunks,w,d_k,dd,H", _chunk_sweep_cases())
def test_chunked_prefill_seeded_sweep(chunks, w, d_k, dd, H):
    run_chunks(chunks, w, d_k, dd, H)


def test_1b_prompt_in_chunks_slice():
    """The 1B-width prompt (N 8192, d 2048, 16 heads of 128, w 512, d_down 512)
    in four chunks of 2048 at full size (the ring kernel on every chunk, with
    many query-tile pairs per (batch, head) and the local arrays rounded down
    to a key tile): every row of one (batch, head) slice of the second
    sequence, chunk by chunk, against the oracle's whole prefill of that
    slice."""
    B, N, d, H, d_k, dd, w, C = 2, 8192, 2048, 16, 128, 512, 512, 2048
    b, hh = 1, 11
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=4100)
    W = {k: dev_w(inp[k], "bf16") for k in ("W_down", "W_up", "W_Q", "W_K", "W_V")}
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    h = dev(inp["h"], "bf16")
    Lc = torch.zeros((B, N, dd), dtype=torch.bfloat16, device="cuda")
    Kw = torch.zeros((B, H, w, d_k), dtype=torch.bfloat16, device="cuda")
    Vw = torch.zeros((B, H, w, d_k), dtype=torch.bfloat16, device="cuda")
    outs = []
    for p0 in range(0, N, C):
        o = dar.dar_prefill_chunk(h[:, p0:p0 + C].contiguous(), W["W_down"], W["W_Q"], W["W_K"],
                                  W["W_V"], Wk, Wv, H, d_k, p0, Lc, Kw, Vw, w)
        outs.append(host(o[b:b + 1, :, hh * d_k:(hh + 1) * d_k]))
    torch.cuda.synchronize()
    one = dict(inp, h=inp["h"][b:b + 1])
    P = oracle.project(one["h"], one["W_down"], one["W_up"], one["W_Q"], one["W_K"], one["W_V"],
                       H, d_k, heads=(hh, hh + 1))
    S = {k: np.ascontiguousarray(P[k][:, hh:hh + 1]) for k in ("Q", "KL", "VL", "KG", "VG")}
    ref, _ = oracle.attend(S, w)
    for c, got in enumerate(outs):
        err = max_err(got, ref[:, c * C:(c + 1) * C])
        log("  1b chunk %d (b%d h%d) every row: max err %.3g" % (c, b, hh, err))
        assert err <= TOL["bf16"]


def run_chunks(chunks, w, d_k, dd, H):
    B, d = 2, 256
    N = sum(chunks)
    inp = prefill_case(B, N + 1, d, H, d_k, dd, "bf16", seed=900 + N + w)
    W = {k: dev_w(inp[k], "bf16") for k in ("W_down", "W_up", "W_Q", "W_K", "W_V")}
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    h = dev(inp["h"], "bf16")
    cap = N + 1
    Lc = torch.zeros((B, cap, dd), dtype=torch.bfloat16, device="cuda")
    Kw = torch.zeros((B, H, max(w, 1), d_k), dtype=torch.bfloat16, device="cuda") if w else None
    Vw = torch.zeros((B, H, max(w, 1), d_k), dtype=torch.bfloat16, device="cuda") if w else None
    ref, _, _ = oracle.prefill(inp, H, d_k, w)
    p0 = 0
    for C in chunks:
        o = dar.dar_prefill_chunk(h[:, p0:p0 + C].contiguous(), W["W_down"], W["W_Q"], W["W_K"],
                                  W["W_V"], Wk, Wv, H, d_k, p0, Lc, Kw, Vw, w)
        torch.cuda.synchronize()
        err = max_err(host(o), ref[:, p0:p0 + C])
        log("  chunk p0=%d C=%d max err %.3g" % (p0, C, err))
        assert err <= TOL["bf16"]
        p0 += C
    q = torch.empty((B, H, d_k), dtype=torch.bfloat16, device="cuda")
    dar.dar_decode_append(h[:, N].contiguous(), W["W_down"], W["W_Q"], W["W_K"], W["W_V"], H, d_k,
                          N, q, Kw, Vw, Lc)
    od = dar.dar_attn_decode(q, Kw, Vw, Lc, Wk, Wv, N + 1, w)
    torch.cuda.synchronize()
    err = max_err(host(od), ref[:, N])
    log("  decode after the chunks: max err %.3g" % err)
    assert err <= TOL["bf16"]
