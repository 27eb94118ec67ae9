"""Benchmark of the DAR attention forward pass on one MI355X.

A step is one prefill pass of the layer (dar_project + dar_attn_prefill, the
folded weights prepared once beforehand) over one batch of synthetic input
already resident in HBM.  Headline workload: the 1B-scale layer (batch 4,
N 8192, d 2048, 16 heads of 128, w 512, d_down 512, bf16), the largest
prefill configuration.  The same run also times the Pythia-70M- and
410M-shaped layers, the d_down sweep, chunked prefill, the attention backward
and the long-context decode step (batch 16, context 32768, d 2048, 16 heads
of 128, w 512, d_down 256), and times the fp64 oracle on a bounded sample of
the headline workload on the host cores (a reported baseline).

Prints ONE JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg):
    print(msg, file=sys.stderr, flush=True)


CSRC = os.path.join(ROOT, "distance_adaptive_dual_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel_key, files):
    """HBM bytes per launch measured by rocprofv3 FETCH_SIZE + WRITE_SIZE runs
    (profiles/*.md, line 'traffic <key> <bytes> sha <hash>'), or None when the
    kernel's sources changed since the counters were taken."""
    sha = source_sha(files)
    if not os.path.isdir(PROFILES):
        return None
    for name in sorted(os.listdir(PROFILES)):
        if not name.endswith(".md"):
            continue
        for line in open(os.path.join(PROFILES, name)):
            m = re.match(r"^traffic (\S+) (\d+) sha (\w+)", line.strip())
            if m and m.group(1) == kernel_key and m.group(3) == sha:
                return int(m.group(2))
    return None


def prefill_flops(B, N, d, d_down):
    """Algorithmic FLOPs of one prefill pass on the minimal route: the fused
    projection h [W_Q|W_K|W_V|W_down], the folded global projection
    h^D [W_upK|W_upV] and causal attention (each pair once)."""
    proj = 2.0 * B * N * (3 * d * d + 3 * d * d_down)
    attn = 2.0 * B * d * N * (N + 1)
    return proj, attn


def prefill_bytes(B, N, d, d_down, H, d_k):
    """Algorithmic HBM bytes (bf16): read h and the weights, write o."""
    return 2.0 * (B * N * d + d * (3 * d + d_down) + 2 * d_down * d + B * N * H * d_k)


def decode_work(B, ctx, d, d_down, w, H):
    """Per-step decode bytes (latents + window K/V + folded weights + q + o) and
    FLOPs: per latent token the key rebuild (2 d d_down), the scores (2 d) and
    the latent-space value sum (2 H d_down); per window token 4 d; per
    sequence one lift by W_upV (2 d_down d)."""
    n_lat = ctx - w
    byts = 2.0 * (B * n_lat * d_down + B * w * 2 * d + 2 * d_down * d + 2 * B * d)
    flops = (B * n_lat * (2.0 * d * d_down + 2.0 * d + 2.0 * H * d_down)
             + B * w * 4.0 * d + B * 2.0 * d_down * d)
    return byts, flops


def make_prefill(torch, dar, di, B, N, d, H, d_k, d_down, seed):
    inp = di.prefill_inputs(B, N, d, H, d_k, d_down, dtype="bf16", seed0=seed)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(
            torch.bfloat16).cuda()

    W = {k: dev(inp[k].T) for k in ("W_down", "W_up", "W_Q", "W_K", "W_V")}
    h = dev(inp["h"])
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    kw = dict(dtype=torch.float16, device="cuda")  # the fp16 intermediates of bf16 mode
    out = dict(Q=torch.empty((B, H, N, d_k), **kw), K_loc=torch.empty((B, H, N, d_k), **kw),
               V_loc=torch.empty((B, H, d_k, N), **kw), h_D=torch.empty((B, N, d_down), **kw),
               K_glob=torch.empty((B, H, N, d_k), **kw), V_glob=torch.empty((B, H, d_k, N), **kw))
    o = torch.empty((B, N, H * d_k), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(dar.project_workspace_bytes(B, N, d, d_down, H, d_k), 256),
                     dtype=torch.uint8, device="cuda")
    return inp, dict(h=h, W=W, Wk=Wk, Wv=Wv, out=out, o=o, ws=ws)


def prefill_step(dar, s, H, d_k, w):
    W = s["W"]
    dar.dar_project(s["h"], W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"], H, d_k,
                    W_upK=s["Wk"], W_upV=s["Wv"], out=s["out"], workspace=s["ws"],
                    sigmoid=s.get("sigmoid", False))
    out = s["out"]
    dar.dar_attn_prefill(out["Q"], out["K_loc"], out["V_loc"], out["K_glob"], out["V_glob"], w,
                         o=s["o"])


def capture(torch, fn, copies=1):
    """HIP graph of `copies` back-to-back calls of fn (the library never
    allocates and records no memset, so its launches capture as plain kernel
    nodes).  One eager call on the capture stream first finishes any lazy
    set-up."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(copies):
            fn()
    torch.cuda.synchronize()
    return g


def settle(torch, g, seconds=1.0):
    """Replays graph g for about `seconds` before anything is timed.  The GPU's
    clocks ramp up under sustained load: the same step graph measured right
    after set-up runs about 15% slower than a second later, so the timed
    region should start from the settled state."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        g.replay()
        torch.cuda.synchronize()


def graph_launch_ms(torch, fn, copies=10, reps=3):
    """Average duration of one call of fn: a graph of `copies` back-to-back
    calls, replayed `reps` times between HIP events on the launch stream."""
    g = capture(torch, fn, copies)
    g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (copies * reps)
    del g
    return ms


def time_prefill(torch, dar, s, H, d_k, w, steps, warmup):
    """The K timed steps (two library calls, four kernels each) are captured as
    one HIP graph, as a model's forward pass would hold its layers, and
    replayed once between synchronizations after W untimed steps.  Returns
    (ms per step by the wall clock, by HIP events, dar_project ms, dar_attn_prefill ms)."""
    step = lambda: prefill_step(dar, s, H, d_k, w)
    warm = capture(torch, step, max(warmup, 1))
    timed = capture(torch, step, steps)
    settle(torch, warm)
    if warmup > 0:
        warm.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    timed.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    ev = e0.elapsed_time(e1) / steps
    del warm, timed
    W = s["W"]
    out = s["out"]
    proj = lambda: dar.dar_project(s["h"], W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"],
                                   H, d_k, W_upK=s["Wk"], W_upV=s["Wv"], out=out,
                                   workspace=s["ws"], sigmoid=s.get("sigmoid", False))
    attn = lambda: dar.dar_attn_prefill(out["Q"], out["K_loc"], out["V_loc"], out["K_glob"],
                                        out["V_glob"], w, o=s["o"])
    return wall, ev, graph_launch_ms(torch, proj), graph_launch_ms(torch, attn)


def time_prefill_drope(torch, dar, di, cfg, d_R, steps, warmup):
    """One prefill pass of the decoupled-RoPE variant (dar_project_drope +
    dar_attn_prefill_drope) at cfg, timed like the headline step (a graph of
    the timed steps).  Algorithmic FLOP: the projections (content, values and
    latent; the rotary queries and the shared rotary key; the folded global
    content keys and values) and, per causal pair and head, 2 (d_k + d_R) for
    the score and 2 d_k for the value sum."""
    B, N, d, H, d_k, w, d_down = cfg
    inp = di.drope_prefill_inputs(B, N, d, H, d_k, d_down, d_R, seed0=4100)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(
            torch.bfloat16).cuda()

    W = {k: dev(inp[k].T) for k in ("W_down", "W_up", "W_Q", "W_K", "W_V", "W_QR", "W_KR")}
    h = dev(inp["h"])
    del inp
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    out = dar.dar_project_drope(h, W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"],
                                W["W_QR"], W["W_KR"], H, d_k, W_upK=Wk, W_upV=Wv)
    o = torch.empty((B, N, H * d_k), dtype=torch.bfloat16, device="cuda")
    # RoPE tables of width d_R: (64 + N/64) rows of d_R/2 (cos, sin) pairs, well under 1 MiB
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")

    def step():
        dar.dar_project_drope(h, W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"],
                              W["W_QR"], W["W_KR"], H, d_k, W_upK=Wk, W_upV=Wv, out=out,
                              workspace=ws)
        dar.dar_attn_prefill_drope(out, w, o=o)
    warm = capture(torch, step, max(warmup, 1))
    timed = capture(torch, step, steps)
    settle(torch, warm)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    timed.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del warm, timed
    attn_ms = graph_launch_ms(torch, lambda: dar.dar_attn_prefill_drope(out, w, o=o))
    proj_f = (2.0 * B * N * d * (3 * H * d_k + d_down + H * d_R + d_R)
              + 4.0 * B * N * d_down * H * d_k)
    attn_f = B * H * N * (N + 1) / 2.0 * (4.0 * d_k + 2.0 * d_R)
    return {"workload": "decoupled-RoPE prefill B%d N%d d%d H%d dk%d dR%d w%d d_down%d"
                        % (B, N, d, H, d_k, d_R, w, d_down),
            "ms": ms, "TFLOP/s": (proj_f + attn_f) / ms / 1e9, "attn_ms": attn_ms,
            "attn_TFLOP/s": attn_f / attn_ms / 1e9,
            "attn_mfma_frac": attn_f / attn_ms / 1e9 / PEAK_BF16_TFLOPS}


def time_ragged_prefill(torch, dar, di, lens, d, H, d_k, w, d_down, reps):
    """A batch of prompts of different lengths prefilled without padding
    (dar_project_varlen + dar_attn_prefill_varlen) and, for comparison, padded
    to the longest (dar_project + dar_attn_prefill).  Both report the
    algorithmic FLOPs of the real tokens only."""
    B, N, T = len(lens), max(lens), sum(lens)
    inp = di.prefill_inputs(1, 1, d, H, d_k, d_down, dtype="bf16", seed0=6000)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(
            torch.bfloat16).cuda()

    W = {k: dev(inp[k].T) for k in ("W_down", "W_up", "W_Q", "W_K", "W_V")}
    Wk, Wv = dar.dar_fold(W["W_up"], W["W_K"], W["W_V"], H, d_k)
    h = torch.randn((T, d), device="cuda").to(torch.bfloat16)
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu = torch.from_numpy(starts).cuda()
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    P = dar.dar_project_varlen(h, W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"], H, d_k,
                               cu, N, W_upK=Wk, W_upV=Wv, workspace=ws)
    o = dar.dar_attn_prefill_varlen(P, cu, N, H, d_k, w)

    def ragged():
        dar.dar_project_varlen(h, W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"], H, d_k,
                               cu, N, W_upK=Wk, W_upV=Wv, out=P, workspace=ws)
        dar.dar_attn_prefill_varlen(P, cu, N, H, d_k, w, o=o)
    hp = torch.zeros((B, N, d), dtype=torch.bfloat16, device="cuda")
    for b, n in enumerate(lens):
        hp[b, :n] = h[starts[b]:starts[b + 1]]
    outp = dar.dar_project(hp, W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"], H, d_k,
                           W_upK=Wk, W_upV=Wv)
    op = torch.empty((B, N, H * d_k), dtype=torch.bfloat16, device="cuda")
    wsp = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")

    def padded():
        dar.dar_project(hp, W["W_down"], W["W_up"], W["W_Q"], W["W_K"], W["W_V"], H, d_k,
                        W_upK=Wk, W_upV=Wv, out=outp, workspace=wsp)
        dar.dar_attn_prefill(outp["Q"], outp["K_loc"], outp["V_loc"], outp["K_glob"],
                             outp["V_glob"], w, o=op)
    flops = sum(2.0 * n * (3 * d * d + 3 * d * d_down) + 2.0 * d * n * (n + 1) for n in lens)
    res = {"workload": "ragged prefill of %d prompts, %d..%d tokens (%d in all), d%d H%d dk%d "
                       "w%d d_down%d" % (B, min(lens), N, T, d, H, d_k, w, d_down)}
    for name, fn in (("ragged", ragged), ("padded", padded)):
        g = capture(torch, fn, reps)
        settle(torch, g, 0.5)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name + "_ms"] = ms
        res[name + "_TFLOP/s"] = flops / ms / 1e9
        del g
    return res


def chunk_flops(B, C, p0, d, d_down):
    """Algorithmic FLOP of one prefill chunk of C tokens after p0 cached ones:
    the chunk's projections, the prefix's global keys/values rebuilt from the
    latents (2 d_down d per token per key and value), and the chunk's queries
    against every key at or before them (4 d per pair)."""
    pairs = C * p0 + C * (C + 1) // 2
    return (2.0 * B * C * (3 * d * d + 3 * d * d_down) + 4.0 * B * p0 * d * d_down
            + 4.0 * B * d * pairs)


def time_chunked(torch, dar, di, cfg, chunk, reps):
    """The prompt of cfg prefilled in chunks of `chunk` tokens over the mixed
    cache (each chunk: dar_prefill_chunk), timed as a whole with HIP events."""
    B, N, d, H, d_k, w, d_down = cfg
    inp, s = make_prefill(torch, dar, di, B, N, d, H, d_k, d_down, seed=3000)
    W = s["W"]
    cache = torch.zeros((B, N, d_down), dtype=torch.bfloat16, device="cuda")
    Kw = torch.zeros((B, H, w, d_k), dtype=torch.bfloat16, device="cuda")
    Vw = torch.zeros_like(Kw)
    hs = [s["h"][:, p0:p0 + chunk].contiguous() for p0 in range(0, N, chunk)]
    o = torch.empty((B, chunk, H * d_k), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(dar.chunk_workspace_bytes(B, chunk, d, d_down, H, d_k, N - chunk, w, N),
                         256), dtype=torch.uint8, device="cuda")

    def run():
        for i, hc in enumerate(hs):
            dar.dar_prefill_chunk(hc, W["W_down"], W["W_Q"], W["W_K"], W["W_V"], s["Wk"],
                                  s["Wv"], H, d_k, i * chunk, cache, Kw, Vw, w, o=o, workspace=ws)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = sum(chunk_flops(B, chunk, p0, d, d_down) for p0 in range(0, N, chunk))
    del inp, s, cache, Kw, Vw, hs, o, ws
    return {"ms": ms, "TFLOP/s": flops / ms / 1e9, "chunks": N // chunk, "chunk": chunk}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def sample_flops(N, d, d_down, nh, d_k):
    """Algorithmic FLOP of one sequence restricted to nh heads, counted as the
    GPU metric counts a whole step: the shared latent h W_down, the nh heads'
    columns of W_Q, W_K, W_V and of the folded W_upK, W_upV, and their causal
    attention."""
    hd = nh * d_k
    return 2.0 * N * (d * d_down + 3 * d * hd + 2 * d_down * hd) + 2.0 * hd * N * (N + 1)


def cpu_baseline(oracle, inp, H, d_k, w, budget_s=10.0, heads=2):
    """The fp64 oracle on a bounded sample of the step's own input: sequence 0
    in full (all N positions), its first `heads` heads (projections, then the
    attention of Eqs. 3-4), repeated until about budget_s seconds of host
    time have passed."""
    h1 = inp["h"][:1]
    _, N, d = h1.shape
    d_down = inp["W_down"].shape[1]
    reps, t0 = 0, time.perf_counter()
    while True:
        P = oracle.project(h1, inp["W_down"], inp["W_up"], inp["W_Q"], inp["W_K"], inp["W_V"],
                           H, d_k, heads=(0, heads))
        S = {k: np.ascontiguousarray(P[k][:, :heads]) for k in ("Q", "KL", "VL", "KG", "VG")}
        oracle.attend(S, w)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s:
            break
    f = sample_flops(N, d, d_down, heads, d_k)
    return {"value": reps * f / dt / 1e12, "unit": "TFLOP/s",
            "cores": oracle.threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "seconds": dt,
            "sample": "sequence 0 of the headline batch (N %d, d %d), heads 0..%d of %d: "
                      "projections (incl. the shared h W_down) and causal attention in fp64, "
                      "%d times; algorithmic FLOP of that sample counted as the GPU metric "
                      "counts a step" % (N, d, heads - 1, H, reps)}


def cache_flusher(torch):
    """A 1 GiB device read (libdar_calib.so) run before each timed decode call:
    it replaces the 256 MB Infinity Cache's contents with clean lines of an
    unrelated buffer, so the call reads its cache from HBM.  (A write-based
    flush would leave dirty lines whose write-back then lands inside the
    timed call.)"""
    import ctypes
    L = ctypes.CDLL(os.path.join(ROOT, "distance_adaptive_dual_amd", "libdar_calib.so"))
    L.dar_calib_read.restype = ctypes.c_int
    L.dar_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                 ctypes.c_void_p]
    buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")

    def flush():
        st = L.dar_calib_read(buf.data_ptr(), buf.numel(), sink.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError("dar_calib_read failed")
    flush.keep = (buf, sink)
    return flush


def timed_after_flush(torch, call, flush, steps, warmup):
    """GPU time of one decode step read from a cold cache: each timed step is
    the cache flush, then HIP events on the launch stream around the step's
    kernels.  The step's launches are enqueued while the flush (a 1 GiB read)
    still runs, so the events bracket the kernels back to back, with no host
    launch time inside (a graph replay behind the flush added about 6 us of
    start-up per step on this ROCm).  Sustained replays first settle the
    clocks."""
    t0 = time.time()
    while time.time() - t0 < 1.0:
        for _ in range(20):
            call()
        torch.cuda.synchronize()
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return times


def time_decode_drope(torch, dar, di, steps, warmup, cfg):
    """The decoupled-RoPE variant's decode step (dar_attn_decode_drope) at the
    long-context shape, timed like time_decode.  Bytes: the latent and rotary
    caches (d_down + d_R per position), the window's content keys and values
    and its rotary keys, the folded weights, q and o."""
    B, ctx, d, H, d_k, d_down, w, d_R = cfg
    inp = di.drope_decode_inputs(B, ctx, d, H, d_k, d_down, d_R, w, seed0=8000)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(
            torch.bfloat16).cuda()

    W_up, W_K, W_V = (dev(inp[k].T) for k in ("W_up", "W_K", "W_V"))
    Wk, Wv = dar.dar_fold(W_up, W_K, W_V, H, d_k)
    t = {k: dev(inp[k]) for k in ("qC", "qR", "K_win", "V_win", "KR", "h_D")}
    del inp
    o = torch.empty((B, H * d_k), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(dar.decode_drope_workspace_bytes(B, ctx, ctx, H, d_k, d_R, d_down, w),
                     dtype=torch.uint8, device="cuda")
    flush = cache_flusher(torch)

    def call():
        dar.dar_attn_decode_drope(t["qC"], t["qR"], t["K_win"], t["V_win"], t["KR"], t["h_D"], Wk,
                                  Wv, ctx, w, o=o, workspace=ws)
    times = timed_after_flush(torch, call, flush, steps, warmup)
    ms = float(np.median(times))
    n_lat = ctx - w
    byts = 2.0 * (B * n_lat * (d_down + d_R) + B * w * (2 * H * d_k + d_R) + 2 * d_down * H * d_k
                  + B * H * (d_k + d_R) + B * H * d_k)
    flops = (B * n_lat * H * (2.0 * (d_down + d_R) + 2.0 * d_down) + B * w * H * (4.0 * d_k + 2.0 * d_R)
             + 2.0 * B * H * d_k * d_down * 2)
    return {"workload": "decoupled-RoPE decode B%d ctx%d d%d H%d dk%d dR%d w%d d_down%d"
                        % (B, ctx, d, H, d_k, d_R, w, d_down),
            "ms": ms, "GB/s": byts / ms / 1e6, "TFLOP/s": flops / ms / 1e9,
            "bytes": byts, "flops": flops,
            "roofline": {"bound": "hbm", "achieved": byts / ms / 1e6, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": byts / ms / 1e6 / PEAK_HBM_GBS}}


def time_decode(torch, dar, di, steps, warmup, cfg, lens=None):
    """The mixed-cache decode step of cfg (B sequences at context ctx), or with
    lens, a ragged batch: sequence b at context lens[b] <= ctx
    (dar_attn_decode_varlen)."""
    B, ctx, d, H, d_k, d_down, w = cfg
    inp = di.decode_inputs(B, ctx, d, H, d_k, d_down, w, dtype="bf16", seed0=5000)

    def dev(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(
            torch.bfloat16).cuda()

    W_up, W_K, W_V = (dev(inp[k].T) for k in ("W_up", "W_K", "W_V"))
    Wk, Wv = dar.dar_fold(W_up, W_K, W_V, H, d_k)
    q, K_win, V_win, h_D = (dev(inp[k]) for k in ("q", "K_win", "V_win", "h_D"))
    del inp
    o = torch.empty((B, H * d_k), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(dar.decode_workspace_bytes(B, ctx, ctx, H, d_k, d_down, w),
                     dtype=torch.uint8, device="cuda")
    flush = cache_flusher(torch)
    if lens is None:
        def call():
            dar.dar_attn_decode(q, K_win, V_win, h_D, Wk, Wv, ctx, w, o=o, workspace=ws)
    else:
        lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda")

        def call():
            dar.dar_attn_decode_varlen(q, K_win, V_win, h_D, Wk, Wv, lens_d, ctx, w, o=o,
                                       workspace=ws)
    times = timed_after_flush(torch, call, flush, steps, warmup)
    ms = float(np.median(times))
    if lens is None:
        byts, flops = decode_work(B, ctx, d, d_down, w, H)
        name = "decode B%d ctx%d d%d H%d dk%d w%d d_down%d" % (B, ctx, d, H, d_k, w, d_down)
    else:
        n_lat = sum(max(0, c - w) for c in lens)
        n_win = sum(min(w, c) for c in lens)
        byts = 2.0 * (n_lat * d_down + n_win * 2 * d + 2 * d_down * d + 2 * B * d)
        flops = (n_lat * (2.0 * d * d_down + 2.0 * d + 2.0 * H * d_down) + n_win * 4.0 * d
                 + B * 2.0 * d_down * d)
        name = ("ragged decode B%d ctx %d..%d (mean %d) d%d H%d dk%d w%d d_down%d"
                % (B, min(lens), max(lens), sum(lens) // B, d, H, d_k, w, d_down))
    return {"workload": name,
            "ms": ms, "GB/s": byts / ms / 1e6, "hbm_frac": byts / ms / 1e6 / PEAK_HBM_GBS,
            "TFLOP/s": flops / ms / 1e9, "mfma_frac": flops / ms / 1e9 / PEAK_BF16_TFLOPS,
            "bytes": byts, "flops": flops}


def time_backward(torch, dar, di, cfg, reps):
    """dar_attn_prefill_backward on seeded fp16 Q/K/V, the forward's o and a
    seeded bf16 dO, with the forward's lse (dar_attn_prefill_lse), as a training
    step would run it.  Algorithmic work: four products of 2 d_k FLOP per causal
    pair (dV, dP, dQ, dK); the MFMA kernels also recompute the scores (in dq
    and in dK/dV) and dP (twice)."""
    B, N, H, d_k, w = cfg

    def g(i, shape, t):
        x = torch.from_numpy(di.gaussian(7000 + i, shape, 1.0, t)).to(torch.float32)
        return x.to(torch.float16 if t == "f16" else torch.bfloat16).cuda()

    qk = (B, H, N, d_k)
    vt = (B, H, d_k, N)
    Q, KL, KG = g(0, qk, "f16"), g(1, qk, "f16"), g(2, qk, "f16")
    VL, VG = g(3, vt, "f16"), g(4, vt, "f16")
    dO = g(5, (B, N, H * d_k), "bf16")
    o, lse = dar.dar_attn_prefill_lse(Q, KL, VL, KG, VG, w)
    out = {k: torch.empty(qk, dtype=torch.float32, device="cuda")
           for k in ("dQ", "dK_loc", "dV_loc", "dK_glob", "dV_glob")}
    ws = torch.empty(max(dar.attn_backward_workspace_bytes(B, N, H, d_k), 256),
                     dtype=torch.uint8, device="cuda")
    fn = lambda: dar.dar_attn_prefill_backward(Q, KL, VL, KG, VG, o, dO, w, lse=lse, out=out,
                                               workspace=ws)
    ms = graph_launch_ms(torch, fn, copies=3, reps=reps)
    flops = 4.0 * B * H * d_k * N * (N + 1)
    tf = flops / ms / 1e9
    return {"workload": "attention backward B%d N%d H%d dk%d w%d (bf16 inputs, fp32 grads)"
                        % (B, N, H, d_k, w),
            "ms": ms, "TFLOP/s": tf, "flops": flops, "bound": "mfma",
            "peak": PEAK_BF16_TFLOPS, "frac": tf / PEAK_BF16_TFLOPS}


def calibrate(torch):
    """Measured peaks on this device: dense fp16 MFMA rate and HBM copy
    bandwidth (libdar_calib.so), to read the kernels' rates against."""
    import ctypes
    L = ctypes.CDLL(os.path.join(ROOT, "distance_adaptive_dual_amd", "libdar_calib.so"))
    L.dar_calib_mfma_flops.restype = ctypes.c_double
    L.dar_calib_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.dar_calib_mfma.restype = ctypes.c_int
    L.dar_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p]
    L.dar_calib_copy.restype = ctypes.c_int
    L.dar_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    wgs, iters = 2048, 2000
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    rates = {}
    for shape, name in ((0, "32x32x16"), (1, "16x16x32")):
        def mfma():
            if L.dar_calib_mfma(sink.data_ptr(), wgs, iters, shape, stream) != 0:
                raise RuntimeError("dar_calib_mfma failed")

        rates[name] = L.dar_calib_mfma_flops(wgs, iters, shape) / timed(mfma) / 1e9
    tflops = max(rates.values())
    nbytes = 1 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)

    def copy():
        if L.dar_calib_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream) != 0:
            raise RuntimeError("dar_calib_copy failed")

    ms_c = timed(copy)
    L.dar_calib_read.restype = ctypes.c_int
    L.dar_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                 ctypes.c_void_p]
    rsink = torch.zeros(8192, dtype=torch.int32, device="cuda")

    def read():
        if L.dar_calib_read(src.data_ptr(), nbytes, rsink.data_ptr(), stream) != 0:
            raise RuntimeError("dar_calib_read failed")

    ms_r = timed(read)
    del src, dst, sink, rsink
    torch.cuda.empty_cache()
    return {"mfma_f16_tflops": tflops, "mfma_f16_tflops_by_shape": rates,
            "hbm_copy_gbs": 2 * nbytes / ms_c / 1e6, "hbm_read_gbs": nbytes / ms_r / 1e6,
            "vendor_mfma_tflops": PEAK_BF16_TFLOPS, "vendor_hbm_gbs": PEAK_HBM_GBS,
            "how": "fp16 MFMA loops from registers (the faster of 32x32x16 and 16x16x32), "
                   "2048 workgroups; 1 GiB device copy with 16-byte loads/stores (read + "
                   "write bytes); 1 GiB device read with 16-byte loads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["all", "prefill", "decode", "backward"], default="all")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline leg")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="one 256 MiB device-to-device copy first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import dar_inputs as di
    import distance_adaptive_dual_amd as dar

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dar.lib()
    if args.calib_copy:
        # known traffic for the counter runs: a 256 MiB copy, and a 256 MiB
        # read by direct-to-LDS loads (the DAR kernels' staging path)
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        import ctypes
        CL = ctypes.CDLL(os.path.join(ROOT, "distance_adaptive_dual_amd", "libdar_calib.so"))
        CL.dar_calib_read_lds.restype = ctypes.c_int
        CL.dar_calib_read_lds.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        if CL.dar_calib_read_lds(src.data_ptr(), src.numel(),
                                 torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("dar_calib_read_lds failed")
        torch.cuda.synchronize()
        del src, dst

    log("calibration: measured MFMA and copy peaks")
    cal = calibrate(torch)
    res = {"metric": "DAR prefill TFLOP/s (% bf16 MFMA peak); decode GB/s (% HBM peak)",
           "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}

    if args.only in ("all", "prefill"):
        # headline: the 1B-scale layer
        B, N, d, H, d_k, w, d_down = 4, 8192, 2048, 16, 128, 512, 512
        log("prefill 1b layer: building inputs")
        inp, s = make_prefill(torch, dar, di, B, N, d, H, d_k, d_down, seed=4000)
        ms, ev_ms, proj_ms, attn_ms = time_prefill(torch, dar, s, H, d_k, w, args.steps,
                                                   args.warmup)
        proj_f, attn_f = prefill_flops(B, N, d, d_down)
        tflops = (proj_f + attn_f) / ms / 1e9
        log("prefill 1b: %.3f ms/step, %.1f TFLOP/s (proj %.3f ms, attn %.3f ms)"
            % (ms, tflops, proj_ms, attn_ms))
        res.update(value=tflops, ms_per_step=ms)
        res["gpu_ms_per_step"] = ev_ms
        res["config"] = {"workload": "1b-layer prefill B%d N%d d%d H%d dk%d w%d d_down%d"
                         % (B, N, d, H, d_k, w, d_down), "global_batch": B, "seq_len": N,
                         "parallelism": "none (1 GPU)"}
        res["mfma_frac"] = tflops / PEAK_BF16_TFLOPS
        res["kernels"] = {"dar_project_ms": proj_ms, "dar_project_TFLOP/s": proj_f / proj_ms / 1e9,
                          "dar_attn_prefill_ms": attn_ms,
                          "dar_attn_prefill_TFLOP/s": attn_f / attn_ms / 1e9}
        # The fused attention kernel is the only launch of dar_attn_prefill and
        # the largest kernel of the step: HIP events on its launch stream around
        # a graph of back-to-back calls time that kernel.
        achieved = attn_f / attn_ms / 1e9
        res["roofline"] = {"kernel": "attn_prefill_ring<128>", "bound": "mfma",
                           "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": achieved / PEAK_BF16_TFLOPS,
                           "traffic": recorded_traffic("attn_prefill_ring<128>@1b",
                                                       ["attn_prefill.hip", "dar_common.hpp"]),
                           "flops_per_launch": attn_f, "launch_ms": attn_ms,
                           "peak_measured": cal["mfma_f16_tflops"],
                           "frac_measured": achieved / cal["mfma_f16_tflops"]}
        if not args.no_cpu:
            import oracle
            log("cpu baseline: the oracle on sequence 0, two heads, of the headline input")
            res["cpu_baseline"] = cpu_baseline(oracle, inp, H, d_k, w)
        del s, inp
        torch.cuda.empty_cache()
        # the Pythia-70M-shaped layer (d_down 128), with its own roofline line
        B, N, d, H, d_k, w, d_down = 8, 2048, 512, 8, 64, 128, 128
        _, s = make_prefill(torch, dar, di, B, N, d, H, d_k, d_down, seed=2000 + d_down)
        ms2, _, p2, a2 = time_prefill(torch, dar, s, H, d_k, w, args.steps, args.warmup)
        pf, af = prefill_flops(B, N, d, d_down)
        res["pythia70m"] = {"workload": "pythia70m-layer prefill B8 N2048 d512 H8 dk64 w128 "
                                        "d_down128", "ms": ms2,
                            "TFLOP/s": (pf + af) / ms2 / 1e9, "proj_ms": p2, "attn_ms": a2,
                            "roofline": {"kernel": "attn_prefill_f16<64>", "bound": "mfma",
                                         "achieved": af / a2 / 1e9, "peak": PEAK_BF16_TFLOPS,
                                         "unit": "TFLOP/s",
                                         "frac": af / a2 / 1e9 / PEAK_BF16_TFLOPS,
                                         "traffic": recorded_traffic(
                                             "attn_prefill_f16<64>@pythia70m",
                                             ["attn_prefill.hip", "dar_common.hpp"])}}
        log("pythia70m: %.3f ms, %.1f TFLOP/s" % (ms2, (pf + af) / ms2 / 1e9))
        del s
        if not args.no_sweep:
            sweep = {}
            for dd in (256, 64):
                _, s2 = make_prefill(torch, dar, di, B, N, d, H, d_k, dd, seed=2000 + dd)
                ms2, _, p2, a2 = time_prefill(torch, dar, s2, H, d_k, w, args.steps,
                                              args.warmup)
                pf, af = prefill_flops(B, N, d, dd)
                sweep["pythia70m d_down%d" % dd] = {"ms": ms2, "TFLOP/s": (pf + af) / ms2 / 1e9}
                del s2
            # the sigmoid-bottleneck variant on the same workload (the sigmoid is
            # B N d_down exponentials in the projection epilogue; FLOP count as above)
            _, s2 = make_prefill(torch, dar, di, B, N, d, H, d_k, d_down, seed=2000 + d_down)
            s2["sigmoid"] = True
            ms2, _, p2, a2 = time_prefill(torch, dar, s2, H, d_k, w, args.steps, args.warmup)
            pf, af = prefill_flops(B, N, d, d_down)
            sweep["pythia70m sigmoid d_down%d" % d_down] = {
                "ms": ms2, "TFLOP/s": (pf + af) / ms2 / 1e9, "proj_ms": p2, "attn_ms": a2}
            del s2
            name, cfg = ("pythia410m B8 N2048 d1024 H16 dk64 w128 d_down256",
                         (8, 2048, 1024, 16, 64, 128, 256))
            b_, n_, d_, h_, k_, w_, dd_ = cfg
            _, s3 = make_prefill(torch, dar, di, b_, n_, d_, h_, k_, dd_, seed=3000)
            ms3, _, p3, a3 = time_prefill(torch, dar, s3, h_, k_, w_, max(3, args.steps // 2), 2)
            pf, af = prefill_flops(b_, n_, d_, dd_)
            sweep[name] = {"ms": ms3, "TFLOP/s": (pf + af) / ms3 / 1e9,
                           "proj_ms": p3, "attn_ms": a3,
                           "attn_TFLOP/s": af / a3 / 1e9, "proj_TFLOP/s": pf / p3 / 1e9}
            log("%s: %.3f ms, %.1f TFLOP/s" % (name, ms3, (pf + af) / ms3 / 1e9))
            del s3
            res["sweep"] = sweep
            cfg1b = (4, 8192, 2048, 16, 128, 512, 512)
            pd = time_prefill_drope(torch, dar, di, cfg1b, 64, max(3, args.steps // 2), 2)
            res["prefill_drope"] = pd
            log("prefill (decoupled RoPE): %.3f ms, %.1f TFLOP/s (attention %.3f ms, %.1f%% of "
                "MFMA peak)" % (pd["ms"], pd["TFLOP/s"], pd["attn_ms"], 100 * pd["attn_mfma_frac"]))
            torch.cuda.empty_cache()
            # a serving-like batch: 16 prompts spread over the 332 .. 1394-token
            # contexts of the pages' downstream evaluations, at the 1B width
            lens = [int(x) for x in np.linspace(332, 1394, 16)]
            rp = time_ragged_prefill(torch, dar, di, lens, 2048, 16, 128, 512, 512,
                                     max(3, args.steps // 2))
            res["prefill_ragged"] = rp
            log("ragged prefill: %.3f ms (%.1f TFLOP/s of real tokens) vs padded %.3f ms"
                % (rp["ragged_ms"], rp["ragged_TFLOP/s"], rp["padded_ms"]))
            torch.cuda.empty_cache()
            ch = time_chunked(torch, dar, di, cfg1b, 2048, max(2, args.steps // 8))
            ch["workload"] = "1b prompt B4 N8192 in chunks of 2048 over the mixed cache"
            res["chunked_prefill"] = ch
            log("chunked prefill: %.3f ms, %.1f TFLOP/s" % (ch["ms"], ch["TFLOP/s"]))
        torch.cuda.empty_cache()
    if args.only in ("all", "backward") and not args.no_sweep:
        bw = time_backward(torch, dar, di, (8, 2048, 8, 64, 128), 2)
        res["backward"] = bw
        log("backward: %.3f ms, %.1f TFLOP/s" % (bw["ms"], bw["TFLOP/s"]))
        bw1 = time_backward(torch, dar, di, (4, 8192, 16, 128, 512), 1)
        res["backward_1b"] = bw1
        log("backward 1b: %.3f ms, %.1f TFLOP/s" % (bw1["ms"], bw1["TFLOP/s"]))
        torch.cuda.empty_cache()
        torch.cuda.empty_cache()
    if args.only in ("all", "decode"):
        log("decode: building the 32k-context cache")
        dec = time_decode(torch, dar, di, max(3, args.steps // 2), 2,
                          (16, 32768, 2048, 16, 128, 256, 512))
        log("decode: %.3f ms, %.0f GB/s, %.1f TFLOP/s" % (dec["ms"], dec["GB/s"], dec["TFLOP/s"]))
        dec["hbm_frac_measured"] = dec["GB/s"] / cal["hbm_read_gbs"]
        dec["mfma_frac_measured"] = dec["TFLOP/s"] / cal["mfma_f16_tflops"]
        res["decode"] = dec
        dd = time_decode_drope(torch, dar, di, max(3, args.steps // 2), 2,
                               (16, 32768, 2048, 16, 128, 256, 512, 64))
        dd["roofline"]["frac_measured"] = dd["GB/s"] / cal["hbm_read_gbs"]
        dd["roofline"]["peak_measured"] = cal["hbm_read_gbs"]
        res["decode_drope"] = dd
        log("decode (decoupled RoPE): %.3f ms, %.0f GB/s (%.1f%% of HBM)"
            % (dd["ms"], dd["GB/s"], 100 * dd["roofline"]["frac"]))
        if not args.no_sweep:
            # a serving-like batch: 16 contexts spread over 1k .. 32k
            lens = [int(x) for x in np.linspace(1024, 32768, 16)[::-1]]
            rg = time_decode(torch, dar, di, max(3, args.steps // 2), 2,
                             (16, 32768, 2048, 16, 128, 256, 512), lens=lens)
            log("ragged decode: %.3f ms, %.0f GB/s, %.1f TFLOP/s" % (rg["ms"], rg["GB/s"],
                                                                   rg["TFLOP/s"]))
            res["decode_ragged"] = rg
        if res["value"] is None:
            res.update(value=dec["GB/s"], unit="GB/s", ms_per_step=dec["ms"])
            res["config"] = {"workload": dec["workload"], "global_batch": 16, "seq_len": 32768,
                             "parallelism": "none (1 GPU)"}
    res["calibration"] = cal
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
