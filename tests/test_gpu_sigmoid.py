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
