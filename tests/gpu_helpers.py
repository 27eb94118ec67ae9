"""Shared helpers for the GPU tests: move seeded inputs to the device in the
library's layouts and compare against the fp64 oracle.  Holds no arithmetic
of the method."""
from __future__ import annotations

import numpy as np
import torch

import dar_inputs as di

TOL = {"bf16": 2e-2, "f32": 1e-4}


def tdtype(dtype: str):
    return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]


def dev(x, dtype: str):
    """float64 numpy (already representable in `dtype`) -> device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(tdtype(dtype)).cuda()


def dev_w(W, dtype: str):
    """A weight W in R^{in x out} -> the column-major device layout ([out, in])."""
    return dev(np.ascontiguousarray(np.asarray(W).T), dtype)


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def weights_dev(inp, dtype):
    return {k: dev_w(inp[k], dtype) for k in ("W_down", "W_up", "W_Q", "W_K", "W_V")}


def max_err(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def log(msg: str):
    print(msg, flush=True)


def prefill_case(B, N, d, H, d_k, d_down, dtype, seed, q_scale=1.0, hot_rows=0):
    return di.prefill_inputs(B, N, d, H, d_k, d_down, dtype=dtype, seed0=seed, q_scale=q_scale,
                             hot_rows=hot_rows)
