"""GPU parity of the sigmoid-bottleneck variant (dar_project_sigmoid: h^D =
sigmoid(h W_down), the variant named after Eq. (1) of "Dual Dimensionality for
Local and Global Attention") against the fp64 oracle, through the C ABI.

Same bars as the linear path: max-abs 2e-2 on o in bf16 mode (fp16 latents
in (0, 1), fp32 accumulation) and 1e-4 in fp32 mode; the projections with the
same per-element bounds as the linear path's tests."""
import numpy as np
import pytest
import torch

import distance_adaptive_dual_amd as dar
import oracle
from gpu_helpers import TOL, dev, host, log, max_err, prefill_case, weights_dev

pytestmark = pytest.mark.gpu


def _run(inp, H, d_k, w, dtype, fold=True, pos0=0, sigmoid=True):
    W = weights_dev(inp, dtype)
    h = dev(inp["h"], dtype)
    Wk = Wv = None
    if fold:
        Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    out = dar.dar_project(h, W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"], H, d_k,
                          W_upK=Wk, W_upV=Wv, pos0=pos0, sigmoid=sigmoid)
    o = dar.dar_attn_prefill(out["Q"], out["K_loc"], out["V_loc"], out["K_glob"], out["V_glob"],
                             w)
    torch.cuda.synchronize()
    return o, out


def _check_proj(out, P, dtype):
    tol = TOL[dtype]
    pairs = [("Q", P["Q"]), ("K_loc", P["KL"]), ("V_loc", P["VL"].transpose(0, 1, 3, 2)),
             ("h_D", P["hD"]), ("K_glob", P["KG"]), ("V_glob", P["VG"].transpose(0, 1, 3, 2))]
    for name, ref in pairs:
        got = host(out[name])
        err = np.abs(got - ref)
        axis = 2 if name in ("V_loc", "V_glob") else -1
        rms = np.sqrt(np.mean(ref ** 2, axis=axis, keepdims=True))
        bound = (tol + 1e-2 * np.abs(ref) + 1e-2 * rms if dtype == "bf16"
                 else tol * (1 + np.abs(ref)))
        assert np.all(err <= bound), "%s: max err %.3g" % (name, err.max())


@pytest.mark.parametrize("fold", [True, False])
def test_fp32_layer(fold):
    B, N, d, H, d_k, dd, w = 1, 384, 256, 4, 64, 64, 96
    inp = prefill_case(B, N, d, H, d_k, dd, "f32", seed=9100)
    log("sigmoid fp32 fold=%s" % fold)
    o, out = _run(inp, H, d_k, w, "f32", fold=fold)
    ref, _, P = oracle.prefill(inp, H, d_k, w, act="sigmoid")
    _check_proj(out, P, "f32")
    err = max_err(host(o), ref)
    log("  max err %.3g" % err)
    assert err <= TOL["f32"]


@pytest.mark.parametrize("B,N,d,H,d_k,dd,w,pos0", [
    (2, 300, 256, 4, 64, 64, 77, 0),      # ragged N
    (1, 257, 128, 2, 128, 32, 0, 0),      # d_k 128, every pair global
    (2, 200, 256, 4, 64, 96, 1, 500),     # d_down not a power of two, nonzero start
    (1, 7, 128, 2, 64, 32, 3, 0),         # shorter than one tile
])
def test_bf16_small(B, N, d, H, d_k, dd, w, pos0):
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=9200 + N + w)
    log("sigmoid bf16 B%d N%d d%d H%d dk%d dd%d w%d pos0 %d" % (B, N, d, H, d_k, dd, w, pos0))
    o, out = _run(inp, H, d_k, w, "bf16", pos0=pos0)
    ref, _, P = oracle.prefill(inp, H, d_k, w, pos0=pos0, act="sigmoid")
    _check_proj(out, P, "bf16")
    err = max_err(host(o), ref)
    log("  max err %.3g" % err)
    assert err <= TOL["bf16"]


def test_pythia70m_layer():
    """B8, N2048, d512, 8 heads of 64, w128, d_down 128 (the bench workload):
    every output against the oracle."""
    B, N, d, H, d_k, w, dd = 8, 2048, 512, 8, 64, 128, 128
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=9300)
    log("sigmoid pythia70m")
    o, out = _run(inp, H, d_k, w, "bf16")
    ref, _, P = oracle.prefill(inp, H, d_k, w, act="sigmoid")
    _check_proj(out, P, "bf16")
    err = max_err(host(o), ref)
    log("  max err %.3g" % err)
    assert err <= TOL["bf16"]


def test_only_the_latent_path_changes():
    """The local path and the queries are those of dar_project, bit for bit;
    the latents lie in (0, 1) and differ from the linear ones."""
    B, N, d, H, d_k, dd, w = 2, 130, 256, 2, 64, 64, 16
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=9400)
    _, lin = _run(inp, H, d_k, w, "bf16", sigmoid=False)
    _, sig = _run(inp, H, d_k, w, "bf16", sigmoid=True)
    for k in ("Q", "K_loc", "V_loc"):
        assert torch.equal(lin[k], sig[k]), k
    hs = host(sig["h_D"])
    assert np.all((hs > 0) & (hs < 1))
    assert not torch.equal(lin["h_D"], sig["h_D"])


@pytest.mark.parametrize("N,w,d_k,dd", [(300, 64, 64, 64), (700, 512, 128, 128),
                                        (129, 0, 64, 32)])
def test_inference_loop_matches_prefill_row(N, w, d_k, dd):
    """The whole inference loop of a sigmoid-bottleneck model on the GPU:
    dar_project_sigmoid over a prompt of N tokens, dar_cache_from_prefill,
    dar_decode_append_sigmoid of token N, dar_attn_decode; the output equals
    row N of the oracle's sigmoid-variant prefill over all N+1 tokens, and the
    appended latent row is sigma(h_N W_down)."""
    from gpu_helpers import dev_w
    B, d, H = 2, 256, 4
    inp = prefill_case(B, N + 1, d, H, d_k, dd, "bf16", seed=9500 + N)
    W = {k: dev_w(inp[k], "bf16") for k in ("W_down", "W_up", "W_Q", "W_K", "W_V")}
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    h = dev(inp["h"], "bf16")
    out = dar.dar_project(h[:, :N].contiguous(), W["W_down"], W["W_up"], W["W_Q"], W["W_K"],
                          W["W_V"], H, d_k, W_upK=Wk, W_upV=Wv, sigmoid=True)
    Lc, Kw, Vw = dar.dar_cache_from_prefill(out["h_D"], out["K_loc"], out["V_loc"], w, cap=N + 1)
    q = torch.empty((B, H, d_k), dtype=torch.bfloat16, device="cuda")
    dar.dar_decode_append(h[:, N].contiguous(), W["W_down"], W["W_Q"], W["W_K"], W["W_V"], H,
                          d_k, N, q, Kw, Vw, Lc, sigmoid=True)
    o = dar.dar_attn_decode(q, Kw, Vw, Lc, Wk, Wv, N + 1, w)
    torch.cuda.synchronize()
    ref, _, P = oracle.prefill(inp, H, d_k, w, act="sigmoid")
    lat = host(Lc)[:, N]
    assert max_err(lat, P["hD"][:, N]) <= 2.0 ** -8  # bf16 rounding of a value in (0, 1)
    err = max_err(host(o), ref[:, N])
    log("  sigmoid loop N%d w%d: decode vs prefill row err %.3g" % (N, w, err))
    assert err <= TOL["bf16"]


def test_ragged_append_writes_sigmoid_latents():
    """dar_decode_append_varlen_sigmoid: sequence b's latent row pos[b] is
    sigma(h_b W_down), its q and ring slot those of the linear call, and the
    other rows are untouched."""
    from gpu_helpers import dev_w
    B, d, H, d_k, dd, w, cap = 3, 256, 2, 64, 64, 32, 100
    inp = prefill_case(B, 1, d, H, d_k, dd, "bf16", seed=9600)
    W = {k: dev_w(inp[k], "bf16") for k in ("W_down", "W_Q", "W_K", "W_V")}
    h = dev(inp["h"][:, 0], "bf16")
    pos = torch.tensor([5, 77, 31], dtype=torch.int32, device="cuda")
    outs = {}
    for sig in (False, True):
        L = torch.zeros((B, cap, dd), dtype=torch.bfloat16, device="cuda")
        Kw = torch.zeros((B, H, w, d_k), dtype=torch.bfloat16, device="cuda")
        Vw = torch.zeros((B, H, w, d_k), dtype=torch.bfloat16, device="cuda")
        q = torch.empty((B, H, d_k), dtype=torch.bfloat16, device="cuda")
        dar.dar_decode_append_varlen(h, W["W_down"], W["W_Q"], W["W_K"], W["W_V"], H, d_k, pos,
                                     q, Kw, Vw, L, sigmoid=sig)
        outs[sig] = (q, Kw, Vw, L)
    torch.cuda.synchronize()
    for t_lin, t_sig in zip(outs[False][:3], outs[True][:3]):
        assert torch.equal(t_lin, t_sig)
    L = host(outs[True][3])
    for b, p in enumerate((5, 77, 31)):
        P = oracle.project(inp["h"][b:b + 1], inp["W_down"], inp["W_up"], inp["W_Q"],
                           inp["W_K"], inp["W_V"], H, d_k, pos0=p, act="sigmoid")
        assert max_err(L[b, p], P["hD"][0, 0]) <= 2.0 ** -8
        rest = np.ones(cap, bool)
        rest[p] = False
        assert not L[b, rest].any()


@pytest.mark.parametrize("chunks,w,d_k,dd,H", [((150, 200, 130), 100, 64, 64, 4),
                                                ((100, 64, 250), 300, 128, 128, 2)])
def test_chunked_prefill_matches_prefill_rows(chunks, w, d_k, dd, H):
    """dar_prefill_chunk_sigmoid chunk by chunk gives every row of the oracle's
    sigmoid-variant prefill over the whole prompt, and the decode of the next
    token (appended with dar_decode_append_sigmoid) gives the next row."""
    from gpu_helpers import dev_w
    B, d = 2, 256
    N = sum(chunks)
    inp = prefill_case(B, N + 1, d, H, d_k, dd, "bf16", seed=9700 + N + w)
    W = {k: dev_w(inp[k], "bf16") for k in ("W_down", "W_up", "W_Q", "W_K", "W_V")}
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    h = dev(inp["h"], "bf16")
    cap = N + 1
    Lc = torch.zeros((B, cap, dd), dtype=torch.bfloat16, device="cuda")
    Kw = torch.zeros((B, H, w, d_k), dtype=torch.bfloat16, device="cuda")
    Vw = torch.zeros((B, H, w, d_k), dtype=torch.bfloat16, device="cuda")
    ref, _, _ = oracle.prefill(inp, H, d_k, w, act="sigmoid")
    p0 = 0
    for C in chunks:
        o = dar.dar_prefill_chunk(h[:, p0:p0 + C].contiguous(), W["W_down"], W["W_Q"], W["W_K"],
                                  W["W_V"], Wk, Wv, H, d_k, p0, Lc, Kw, Vw, w, sigmoid=True)
        torch.cuda.synchronize()
        err = max_err(host(o), ref[:, p0:p0 + C])
        log("  sigmoid chunk p0 %d C %d: err %.3g" % (p0, C, err))
        assert err <= TOL["bf16"]
        p0 += C
    q = torch.empty((B, H, d_k), dtype=torch.bfloat16, device="cuda")
    dar.dar_decode_append(h[:, N].contiguous(), W["W_down"], W["W_Q"], W["W_K"], W["W_V"], H,
                          d_k, N, q, Kw, Vw, Lc, sigmoid=True)
    od = dar.dar_attn_decode(q, Kw, Vw, Lc, Wk, Wv, N + 1, w)
    torch.cuda.synchronize()
    assert max_err(host(od), ref[:, N]) <= TOL["bf16"]
