"""Seeded synthetic inputs for the DAR attention layer.

This module only draws random numbers and rounds them to the storage type of
a run (bf16 or fp32).  It holds none of the method's arithmetic, so both the
fp64 oracle (``oracle/``) and the HIP path (``distance_adaptive_dual_amd``)
can consume exactly the same values.

Values are returned as float64 numpy arrays whose entries are exactly
representable in the run's storage type, plus helpers that turn them into the
bit patterns a device buffer needs.

Distributions (the pages train these layers from scratch, so the synthetic
stand-in uses the usual fan-in scaling):
  h                      ~ N(0, 1)
  W_down, W_Q, W_K, W_V  ~ N(0, 1/d)         (fan-in d)
  W_up                   ~ N(0, 1/d_down)    (fan-in d_down)
Seeds: ``seed = 1000 * cfg + k`` with k = 0..5 for (h, W_down, W_up, W_Q, W_K, W_V).
"""
from __future__ import annotations

import numpy as np

# Workloads (batch, sequence, model width, heads, per-head width, window,
# bottleneck width) of the layers the pages train: Pythia-70M / 410M shapes
# (d = 512 / 1024, w = 128, sequence length 2048), a 1B-scale layer
# (d = 2048) and a long-context decode step.
WORKLOADS = {
    1: dict(name="dar-fp32-B1-N512-d512", B=1, N=512, d=512, H=8, d_k=64, w=128,
            d_down=128, dtype="f32", kind="prefill"),
    2: dict(name="pythia70m-B8-N2048-d512", B=8, N=2048, d=512, H=8, d_k=64, w=128,
            d_down=256, dtype="bf16", kind="prefill"),
    3: dict(name="pythia410m-B8-N2048-d1024", B=8, N=2048, d=1024, H=16, d_k=64, w=128,
            d_down=256, dtype="bf16", kind="prefill"),
    4: dict(name="1b-B4-N8192-d2048", B=4, N=8192, d=2048, H=16, d_k=128, w=512,
            d_down=512, dtype="bf16", kind="prefill"),
    5: dict(name="decode-B16-ctx32768-d2048", B=16, N=32768, d=2048, H=16, d_k=128,
            w=512, d_down=256, dtype="bf16", kind="decode"),
}
ROPE_BASE = 10000.0


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as float64."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def round_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_f16(x) -> np.ndarray:
    """Round float64 values to the nearest IEEE half (ties to even), as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def round_to(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f16":
        return round_f16(x)
    if dtype == "f32":
        return round_f32(x)
    raise ValueError(dtype)


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of values already representable in bf16."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bits_to_f64(bits) -> np.ndarray:
    """float64 values of bf16 bit patterns."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def gaussian(seed: int, shape, std: float, dtype: str) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    return round_to(g.standard_normal(size=shape) * std, dtype)


def prefill_inputs(B, N, d, H, d_k, d_down, dtype="bf16", seed0=2000, q_scale=1.0,
                   hot_rows=0):
    """h [B,N,d] and the five weights in the pages' right-multiplication layout.

    ``q_scale`` multiplies W_Q (a sharper softmax); ``hot_rows`` > 0 scales that
    many seeded rows of h by 8 (large scores, exercising max subtraction).
    """
    hd = H * d_k
    h = np.random.Generator(np.random.PCG64(seed0 + 0)).standard_normal((B, N, d))
    if hot_rows:
        g = np.random.Generator(np.random.PCG64(seed0 + 6))
        idx = g.choice(B * N, size=min(hot_rows, B * N), replace=False)
        h.reshape(B * N, d)[idx] *= 8.0
    out = dict(
        h=round_to(h, dtype),
        W_down=gaussian(seed0 + 1, (d, d_down), d ** -0.5, dtype),
        W_up=gaussian(seed0 + 2, (d_down, d), d_down ** -0.5, dtype),
        W_Q=round_to(np.random.Generator(np.random.PCG64(seed0 + 3)).standard_normal((d, hd))
                     * (d ** -0.5) * q_scale, dtype),
        W_K=gaussian(seed0 + 4, (d, hd), d ** -0.5, dtype),
        W_V=gaussian(seed0 + 5, (d, hd), d ** -0.5, dtype),
    )
    return out


def decode_inputs(B, ctx, d, H, d_k, d_down, w, cap=None, dtype="bf16", seed0=5000):
    """Mixed decode cache for one new query per sequence at position p = ctx - 1.

    q      [B, H, d_k]        the query (already rotated: values are drawn directly)
    K_win  [B, H, w, d_k]     window keys, ring slot s holds the position == s (mod w)
    V_win  [B, H, w, d_k]     window values, same ring
    h_D    [B, cap, d_down]   latents; only rows 0 .. p - w are read
    W_up, W_K, W_V            weights (pages' layout); W_down, W_Q complete the set
    """
    cap = ctx if cap is None else cap
    hd = H * d_k
    return dict(
        q=gaussian(seed0 + 0, (B, H, d_k), 1.0, dtype),
        K_win=gaussian(seed0 + 1, (B, H, w, d_k), 1.0, dtype),
        V_win=gaussian(seed0 + 2, (B, H, w, d_k), 1.0, dtype),
        h_D=gaussian(seed0 + 3, (B, cap, d_down), 1.0, dtype),
        W_up=gaussian(seed0 + 4, (d_down, d), d_down ** -0.5, dtype),
        W_K=gaussian(seed0 + 5, (d, hd), d ** -0.5, dtype),
        W_V=gaussian(seed0 + 6, (d, hd), d ** -0.5, dtype),
        # not read by the decode step itself; the packed weight set holds them
        W_down=gaussian(seed0 + 7, (d, d_down), d ** -0.5, dtype),
        W_Q=gaussian(seed0 + 8, (d, hd), d ** -0.5, dtype),
    )


def drope_prefill_inputs(B, N, d, H, d_k, d_down, d_R, dtype="bf16", seed0=7000, q_scale=1.0):
    """prefill_inputs plus the rotary weights of the decoupled-RoPE variant:
    W_QR [d, H d_R] and W_KR [d, d_R], both ~ N(0, 1/d) (fan-in d)."""
    out = prefill_inputs(B, N, d, H, d_k, d_down, dtype=dtype, seed0=seed0, q_scale=q_scale)
    out["W_QR"] = gaussian(seed0 + 7, (d, H * d_R), d ** -0.5, dtype)
    out["W_KR"] = gaussian(seed0 + 8, (d, d_R), d ** -0.5, dtype)
    return out


def drope_decode_inputs(B, ctx, d, H, d_k, d_down, d_R, w, cap=None, dtype="bf16",
                        seed0=8000):
    """Mixed cache of the decoupled-RoPE variant for one query per sequence at
    p = ctx - 1 (every value drawn directly; rotated parts are drawn already
    rotated):
    qC [B,H,d_k], qR [B,H,d_R]; K_win, V_win [B,H,w,d_k] (content keys and
    values, ring slot = position mod w); KR [B,cap,d_R] (rotary keys of every
    position); h_D [B,cap,d_down]; W_up, W_K, W_V (pages' layout)."""
    cap = ctx if cap is None else cap
    hd = H * d_k
    return dict(
        qC=gaussian(seed0 + 0, (B, H, d_k), 1.0, dtype),
        qR=gaussian(seed0 + 1, (B, H, d_R), 1.0, dtype),
        K_win=gaussian(seed0 + 2, (B, H, w, d_k), 1.0, dtype),
        V_win=gaussian(seed0 + 3, (B, H, w, d_k), 1.0, dtype),
        KR=gaussian(seed0 + 4, (B, cap, d_R), 1.0, dtype),
        h_D=gaussian(seed0 + 5, (B, cap, d_down), 1.0, dtype),
        W_up=gaussian(seed0 + 6, (d_down, d), d_down ** -0.5, dtype),
        W_K=gaussian(seed0 + 7, (d, hd), d ** -0.5, dtype),
        W_V=gaussian(seed0 + 8, (d, hd), d ** -0.5, dtype),
    )
