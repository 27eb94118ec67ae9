"""The library's calls captured into a HIP graph (torch.cuda.CUDAGraph) give,
on every replay, exactly the bytes of the eager calls.  Replays are separated
by eager work of the program (other library calls into other buffers, torch
ops) and synchronizations, and each replay's output is checked."""
import pytest
import torch

import dar_inputs as di
import distance_adaptive_dual_amd as dar
from gpu_helpers import dev, dev_w, log, prefill_case

pytestmark = pytest.mark.gpu


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_prefill_graph_replays_match_eager():
    B, N, d, H, d_k, dd, w = 2, 700, 256, 4, 64, 64, 100
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=31)
    W = {k: dev_w(inp[k], "bf16") for k in ("W_down", "W_up", "W_Q", "W_K", "W_V")}
    h = dev(inp["h"], "bf16")
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    ws = torch.empty(dar.project_workspace_bytes(B, N, d, dd, H, d_k), dtype=torch.uint8,
                     device="cuda")
    out = dar.dar_project(h, W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"], H, d_k,
                          W_upK=Wk, W_upV=Wv, workspace=ws)
    o = dar.dar_attn_prefill(out["Q"], out["K_loc"], out["V_loc"], out["K_glob"], out["V_glob"], w)
    torch.cuda.synchronize()
    ref_o = o.clone()
    ref_out = {k: v.clone() for k, v in out.items()}

    def step():
        dar.dar_project(h, W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"], H, d_k,
                        W_upK=Wk, W_upV=Wv, out=out, workspace=ws)
        dar.dar_attn_prefill(out["Q"], out["K_loc"], out["V_loc"], out["K_glob"], out["V_glob"],
                             w, o=o)

    g = capture(step)
    other = dev(di.prefill_inputs(B, N, d, H, d_k, dd, seed0=77)["h"], "bf16")
    for rep in range(4):
        o.zero_()
        for v in out.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log("prefill graph replay %d" % rep)
        assert torch.equal(o, ref_o)
        for k in ref_out:
            assert torch.equal(out[k], ref_out[k]), k
        # eager work between replays: the same library calls on another input
        p2 = dar.dar_project(other, W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"], H, d_k,
                             W_upK=Wk, W_upV=Wv)
        o2 = dar.dar_attn_prefill(p2["Q"], p2["K_loc"], p2["V_loc"], p2["K_glob"], p2["V_glob"], w)
        torch.cuda.synchronize()
        assert not torch.equal(o2, ref_o)
        del o2, p2


@pytest.mark.parametrize("C", [192, 150])  # chunk end on a key tile (ring kernel), and not
def test_chunked_prefill_graph_replays_match_eager(C):
    """One prefill chunk after a cached prefix, captured: every replay, from
    the same cache state (restored by eager copies between replays, with other
    eager work), writes the eager output, latent rows and window ring."""
    B, d, H, d_k, dd, w, C0 = 2, 256, 2, 128, 64, 100, 128
    N = C0 + C
    inp = prefill_case(B, N, d, H, d_k, dd, "bf16", seed=950 + C)
    W = {k: dev_w(inp[k], "bf16") for k in ("W_down", "W_up", "W_Q", "W_K", "W_V")}
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    h = dev(inp["h"], "bf16")
    h1 = h[:, C0:].contiguous()
    Lc = torch.zeros((B, N, dd), dtype=torch.bfloat16, device="cuda")
    Kw = torch.zeros((B, H, w, d_k), dtype=torch.bfloat16, device="cuda")
    Vw = torch.zeros((B, H, w, d_k), dtype=torch.bfloat16, device="cuda")
    args = (W["W_down"], W["W_Q"], W["W_K"], W["W_V"], Wk, Wv, H, d_k)
    dar.dar_prefill_chunk(h[:, :C0].contiguous(), *args, 0, Lc, Kw, Vw, w)
    state = [t.clone() for t in (Lc, Kw, Vw)]
    ws = torch.empty(dar.chunk_workspace_bytes(B, C, d, dd, H, d_k, C0, w, N), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((B, C, H * d_k), dtype=torch.bfloat16, device="cuda")

    def restore():
        for t, s0 in zip((Lc, Kw, Vw), state):
            t.copy_(s0)

    dar.dar_prefill_chunk(h1, *args, C0, Lc, Kw, Vw, w, o=o, workspace=ws)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, Lc, Kw, Vw)]
    restore()
    g = capture(lambda: dar.dar_prefill_chunk(h1, *args, C0, Lc, Kw, Vw, w, o=o, workspace=ws))
    for rep in range(3):
        restore()
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("o", "latents", "K ring", "V ring"), (o, Lc, Kw, Vw), ref):
            assert torch.equal(got, want), "replay %d: %s differs" % (rep, name)
        # other eager work between replays
        dar.dar_prefill_chunk(h[:, :C0].contiguous(), *args, 0, Lc, Kw, Vw, w)
    log("  chunk C=%d: 3 replays equal the eager call" % C)


def test_decode_graph_replays_match_eager():
    B, ctx, d, H, d_k, dd, w = 2, 3000, 512, 4, 128, 128, 256
    inp = di.decode_inputs(B, ctx, d, H, d_k, dd, w, seed0=88)
    W_up, W_K, W_V = (dev_w(inp[k], "bf16") for k in ("W_up", "W_K", "W_V"))
    Wk, Wv = dar.dar_fold(W_up, W_K, W_V, H, d_k)
    q, K_win, V_win, h_D = (dev(inp[k], "bf16") for k in ("q", "K_win", "V_win", "h_D"))
    ws = torch.empty(dar.decode_workspace_bytes(B, ctx, ctx, H, d_k, dd, w), dtype=torch.uint8,
                     device="cuda")
    o = dar.dar_attn_decode(q, K_win, V_win, h_D, Wk, Wv, ctx, w, workspace=ws)
    torch.cuda.synchronize()
    ref = o.clone()
    g = capture(lambda: dar.dar_attn_decode(q, K_win, V_win, h_D, Wk, Wv, ctx, w, o=o,
                                            workspace=ws))
    for rep in range(4):
        o.zero_()
        ws.fill_(0x7F)  # the partials must be rewritten by every replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log("decode graph replay %d" % rep)
        assert torch.equal(o, ref)
        o2 = dar.dar_attn_decode(q, K_win, V_win, h_D, Wk, Wv, ctx - 7, w)
        torch.cuda.synchronize()
        assert not torch.equal(o2, ref)


def test_ragged_decode_graph_follows_device_lengths():
    """A captured ragged decode reads the per-sequence lengths from device
    memory at every replay: changing them in place between replays gives the
    eager result for the new lengths."""
    B, max_ctx, d, H, d_k, dd, w = 3, 2500, 512, 4, 128, 128, 256
    inp = di.decode_inputs(B, max_ctx, d, H, d_k, dd, w, seed0=99)
    W_up, W_K, W_V = (dev_w(inp[k], "bf16") for k in ("W_up", "W_K", "W_V"))
    Wk, Wv = dar.dar_fold(W_up, W_K, W_V, H, d_k)
    q, K_win, V_win, h_D = (dev(inp[k], "bf16") for k in ("q", "K_win", "V_win", "h_D"))
    lens = torch.tensor([2500, 300, 1200], dtype=torch.int32, device="cuda")
    ws = torch.empty(dar.decode_workspace_bytes(B, max_ctx, max_ctx, H, d_k, dd, w),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty((B, H * d_k), dtype=torch.bfloat16, device="cuda")
    g = capture(lambda: dar.dar_attn_decode_varlen(q, K_win, V_win, h_D, Wk, Wv, lens, max_ctx,
                                                   w, o=o, workspace=ws))
    for rep, new in enumerate(([2500, 300, 1200], [17, 2499, 256], [1, 257, 2000])):
        lens.copy_(torch.tensor(new, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = dar.dar_attn_decode_varlen(q, K_win, V_win, h_D, Wk, Wv, lens, max_ctx, w)
        torch.cuda.synchronize()
        log("ragged decode graph replay %d lens %s" % (rep, new))
        assert torch.equal(o, ref)


def test_training_step_graph_replays_match_eager():
    """Forward with lse and the backward captured together: every replay gives
    the eager gradients exactly; the backward is also deterministic."""
    B, H, N, d_k, w = 2, 2, 600, 64, 100
    g_ = [dev(di.gaussian(900 + i, (B, H, N, d_k), 1.0, "f16"), "f16") for i in range(3)]
    Q, KL, KG = g_
    VL = dev(di.gaussian(905, (B, H, d_k, N), 1.0, "f16"), "f16")
    VG = dev(di.gaussian(906, (B, H, d_k, N), 1.0, "f16"), "f16")
    dO = dev(di.gaussian(907, (B, N, H * d_k), 1.0, "bf16"), "bf16")
    o, lse = dar.dar_attn_prefill_lse(Q, KL, VL, KG, VG, w)
    ws = torch.empty(max(dar.attn_backward_workspace_bytes(B, N, H, d_k), 256), dtype=torch.uint8,
                     device="cuda")
    grads = dar.dar_attn_prefill_backward(Q, KL, VL, KG, VG, o, dO, w, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in grads.items()}
    ref_o, ref_lse = o.clone(), lse.clone()
    again = dar.dar_attn_prefill_backward(Q, KL, VL, KG, VG, o, dO, w, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(again[k], ref[k]), k

    def step():
        dar.dar_attn_prefill_lse(Q, KL, VL, KG, VG, w, o=o, lse=lse)
        dar.dar_attn_prefill_backward(Q, KL, VL, KG, VG, o, dO, w, lse=lse, out=grads,
                                      workspace=ws)

    g = capture(step)
    for rep in range(3):
        for v in list(grads.values()) + [o, lse]:
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log("training graph replay %d" % rep)
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse)
        for k in ref:
            assert torch.equal(grads[k], ref[k]), k
        # eager work of the program between replays
        dar.dar_attn_prefill(Q, KG, VG, KL, VL, w)
        torch.cuda.synchronize()


def test_calls_on_a_side_stream_match_the_current_stream():
    """Every binding call given `stream` allocates its outputs and workspace on
    that stream and launches there: a prompt -> cache -> append -> decode
    sequence issued on a side stream (while the current stream is kept busy)
    gives exactly the bytes of the same sequence on the current stream."""
    B, N, d, H, d_k, dd, w = 2, 300, 256, 4, 64, 64, 64
    inp = prefill_case(B, N + 1, d, H, d_k, dd, "bf16", seed=808)
    W = {k: dev_w(inp[k], "bf16") for k in ("W_down", "W_up", "W_Q", "W_K", "W_V")}
    h = dev(inp["h"], "bf16")
    # inputs are made before the side stream is ordered after the current one:
    # a caller's inputs must be ready on the stream it passes
    h_prompt, h_next = h[:, :N].contiguous(), h[:, N].contiguous()

    def sequence(stream):
        Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k, stream=stream)
        out = dar.dar_project(h_prompt, W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"],
                              H, d_k, W_upK=Wk, W_upV=Wv, stream=stream)
        o = dar.dar_attn_prefill(out["Q"], out["K_loc"], out["V_loc"], out["K_glob"],
                                 out["V_glob"], w, stream=stream)
        cache, K_win, V_win = dar.dar_cache_from_prefill(out["h_D"], out["K_loc"],
                                                         out["V_loc"], w, cap=N + 1,
                                                         stream=stream)
        with torch.cuda.stream(stream) if stream is not None else torch.cuda.stream(
                torch.cuda.current_stream()):
            q = torch.empty((B, H, d_k), dtype=torch.bfloat16, device="cuda")
        dar.dar_decode_append(h_next, W["W_down"], W["W_Q"], W["W_K"], W["W_V"], H, d_k, N, q,
                              K_win, V_win, cache, stream=stream)
        od = dar.dar_attn_decode(q, K_win, V_win, cache, Wk, Wv, N + 1, w, stream=stream)
        return [o, od, cache, K_win, V_win]

    ref = [t.clone() for t in sequence(None)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    busy = torch.randn(4096, 4096, device="cuda")
    for _ in range(8):  # keep the current stream busy meanwhile
        busy = busy @ busy
        busy /= busy.norm()
    got = sequence(side)
    side.synchronize()
    res = [t.clone() for t in got]
    torch.cuda.synchronize()
    for a, b in zip(ref, res):
        assert torch.equal(a, b)
