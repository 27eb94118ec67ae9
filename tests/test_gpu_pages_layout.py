"""The equations' weight layout at the boundary: a caller holding W_down,
W_up, W_Q, W_K, W_V row-major as Eqs. (1)-(4) write them (W in R^{in x out},
right-multiplied by row vectors) packs them once with dar_pack_weight and
runs the layer through the C ABI; the result matches the fp64 oracle at 1e-4
(fp32 mode) and 2e-2 (bf16 mode)."""
import numpy as np
import pytest
import torch

import dar_inputs as di
import distance_adaptive_dual_amd as dar
import oracle
from gpu_helpers import TOL, dev, host, log, max_err, prefill_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", [(512, 128), (100, 70), (1, 33), (64, 1), (257, 1031)])
def test_pack_is_exact_transpose(dtype, rows, cols):
    g = np.random.Generator(np.random.PCG64(rows * 7 + cols))
    W = g.standard_normal((rows, cols))
    W = di.round_bf16(W) if dtype == "bf16" else di.round_f32(W)
    got = dar.dar_pack_weight(dev(W, dtype))
    torch.cuda.synchronize()
    assert tuple(got.shape) == (cols, rows)
    assert np.array_equal(host(got), W.T)


@pytest.mark.parametrize("dtype,B,N,d,H,d_k,dd,w", [
    ("f32", 1, 512, 512, 8, 64, 128, 128),    # the single fp32 layer
    ("bf16", 2, 700, 512, 8, 64, 128, 128),
    ("bf16", 1, 300, 256, 2, 128, 64, 50),
])
def test_layer_from_the_equations_layout(dtype, B, N, d, H, d_k, dd, w):
    inp = prefill_case(B, N, d, H, d_k, dd, dtype, seed=616 + N)
    # the matrices exactly as the equations hold them: [in, out], rows contiguous
    W = {k: dar.dar_pack_weight(dev(inp[k], dtype))
         for k in ("W_down", "W_up", "W_Q", "W_K", "W_V")}
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    out = dar.dar_project(dev(inp["h"], dtype), W["W_down"], W["W_up"], W["W_Q"], W["W_K"],
                          W["W_V"], H, d_k, W_upK=Wk, W_upV=Wv)
    o = dar.dar_attn_prefill(out["Q"], out["K_loc"], out["V_loc"], out["K_glob"], out["V_glob"],
                             w)
    torch.cuda.synchronize()
    ref, _, _ = oracle.prefill(inp, H, d_k, w)
    err = max_err(host(o), ref)
    log("  %s layer from row-major weights: max err %.3g" % (dtype, err))
    assert err <= TOL[dtype]
