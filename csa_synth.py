"""Seeded synthetic inputs for the CSA/HCA attention forward.

This module only draws random numbers. It holds none of the method's
arithmetic (no compression, quantisation, scoring, selection or attention),
so both the CPU oracle and the HIP path can take their inputs from it.

Generation: NumPy ``Generator(PCG64(seed))`` on the host in float32, with
``seed = 1000 * workload_id + tensor_id``. Tensors stored in bf16 on the device
are drawn in float32 and then snapped to the nearest bf16 value (round to
nearest, ties to even) here, so the float32 array handed to either side holds
exactly the values the device sees.

The workloads mirror the shapes and distributions of the 1M-token-context
workloads the DeepSeek-V4 write-ups describe (cf-1.com write-up §3.1-§3.4,
yfxerp.com write-up §3): 4:1 overlapped gated compression, 128:1 compression,
top-k 512/1024, a 128-token window and a per-head sink logit. No public dataset
is involved; these synthetic tensors stand in for real activations.
"""
from __future__ import annotations

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Snap float32 values to bf16-representable float32 values (RNE)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def normal(seed: int, shape, scale: float = 1.0, bf16: bool = False) -> np.ndarray:
    x = rng(seed).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return round_bf16(x) if bf16 else x


def uniform(seed: int, shape, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    x = rng(seed).random(size=shape, dtype=np.float32)
    if lo != 0.0 or hi != 1.0:
        x = (x * np.float32(hi - lo) + np.float32(lo)).astype(np.float32)
    return x


def integers(seed: int, shape, lo: int, hi: int) -> np.ndarray:
    """Integers in [lo, hi] as float32 (exact)."""
    return rng(seed).integers(lo, hi + 1, size=shape).astype(np.float32)


def grid_weights(seed: int, shape) -> np.ndarray:
    """Weights on the grid {0, 1/8, ..., 1} (exact in every float format used)."""
    return (rng(seed).integers(0, 9, size=shape).astype(np.float32) / np.float32(8.0)).astype(np.float32)


def fp4_grid(seed: int, shape) -> np.ndarray:
    """Values drawn from the e2m1 grid {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)
    g = rng(seed)
    v = mags[g.integers(0, 8, size=shape)]
    s = np.where(g.integers(0, 2, size=shape) == 1, np.float32(-1.0), np.float32(1.0))
    return (v * s).astype(np.float32)


# ---------------------------------------------------------------------------
# Workload recipes. Each returns a dict of float32 host arrays plus scalars.
# Shapes follow the five workloads of the measurement plan; ``scale_down``
# shrinks the long axes for parity tests the oracle finishes in seconds.
# ---------------------------------------------------------------------------

def csa_prefill(wid: int, T: int, H: int, H_I: int, d_I: int, bf16: bool, d: int = 128,
                grid: bool = False) -> dict:
    """CSA prefill: raw KV/gate streams, indexer streams, queries, weights, sinks.

    KV streams C_a, C_b and gate logits Z_a, Z_b are [T, d] N(0,1); the
    indexer streams (same four roles) are [T, d_I] N(0,1); queries [T, H, d]
    N(0,1)/sqrt(d); indexer queries [T, H_I, d_I] N(0,1); indexer weights
    [T, H_I] U(0,1); sink logits [H] N(0,1).
    With ``grid=True`` the indexer queries are integers in [-4, 4] and the
    weights lie on {0, 1/8, ..., 1}.
    """
    s = 1000 * wid
    out = {
        "c_a": normal(s + 1, (T, d), bf16=bf16), "c_b": normal(s + 2, (T, d), bf16=bf16),
        "z_a": normal(s + 3, (T, d), bf16=bf16), "z_b": normal(s + 4, (T, d), bf16=bf16),
        "ci_a": normal(s + 5, (T, d_I), bf16=bf16), "ci_b": normal(s + 6, (T, d_I), bf16=bf16),
        "zi_a": normal(s + 7, (T, d_I), bf16=bf16), "zi_b": normal(s + 8, (T, d_I), bf16=bf16),
        "q": normal(s + 9, (T, H, d), scale=1.0 / np.sqrt(d), bf16=bf16),
        "sink": normal(s + 12, (H,)),
    }
    if grid:
        out["q_i"] = integers(s + 10, (T, H_I, d_I), -4, 4)
        out["w"] = grid_weights(s + 11, (T, H_I))
    else:
        out["q_i"] = normal(s + 10, (T, H_I, d_I), bf16=bf16)
        out["w"] = uniform(s + 11, (T, H_I))
    return out


def hca_prefill(wid: int, T: int, H: int, bf16: bool, d: int = 128) -> dict:
    """HCA prefill: raw stream C, gate logits Z [T, d] N(0,1); q [T, H, d]; sinks [H]."""
    s = 1000 * wid
    return {
        "c": normal(s + 1, (T, d), bf16=bf16), "z": normal(s + 2, (T, d), bf16=bf16),
        "q": normal(s + 3, (T, H, d), scale=1.0 / np.sqrt(d), bf16=bf16),
        "sink": normal(s + 4, (H,)),
    }


def csa_decode(wid: int, B: int, N: int, H: int, H_I: int, d_I: int, T_win: int = 128,
               d: int = 128, key_grid: str | None = None) -> dict:
    """CSA decode caches sampled directly (the compressor is not on the decode path).

    E [B, N, d] bf16 N(0,1); indexer keys [B, N, d_I] N(0,1) before quantisation;
    window rows [B, T_win, d] bf16 N(0,1); q [B, H, d] N(0,1)/sqrt(d) bf16;
    indexer queries [B, H_I, d_I] N(0,1); weights [B, H_I] U(0,1); sinks [H].
    ``key_grid`` = "int" (integers in [-4, 4]) or "fp4" (e2m1 grid values)
    gives scores that are exact in float32 under any summation order.
    """
    s = 1000 * wid
    out = {
        "kv": normal(s + 1, (B, N, d), bf16=True),
        "x_win": normal(s + 3, (B, T_win, d), bf16=True),
        "q": normal(s + 4, (B, H, d), scale=1.0 / np.sqrt(d), bf16=True),
        "sink": normal(s + 7, (H,)),
    }
    if key_grid == "int":
        out["k_i"] = integers(s + 2, (B, N, d_I), -4, 4)
        out["q_i"] = integers(s + 5, (B, H_I, d_I), -4, 4)
        out["w"] = grid_weights(s + 6, (B, H_I))
    elif key_grid == "fp4":
        out["k_i"] = fp4_grid(s + 2, (B, N, d_I))
        out["q_i"] = fp4_grid(s + 5, (B, H_I, d_I))
        out["w"] = grid_weights(s + 6, (B, H_I))
    else:
        out["k_i"] = normal(s + 2, (B, N, d_I))
        out["q_i"] = normal(s + 5, (B, H_I, d_I))
        out["w"] = uniform(s + 6, (B, H_I))
    return out


def hca_decode(wid: int, B: int, N: int, H: int, T_win: int = 128, d: int = 128) -> dict:
    """HCA decode cache [B, N, d] bf16 N(0,1), window rows, q, sinks (tensor ids 11..)."""
    s = 1000 * wid
    return {
        "kv": normal(s + 11, (B, N, d), bf16=True),
        "x_win": normal(s + 12, (B, T_win, d), bf16=True),
        "q": normal(s + 13, (B, H, d), scale=1.0 / np.sqrt(d), bf16=True),
        "sink": normal(s + 14, (H,)),
    }


# ---------------------------------------------------------------------------
# Device-side generation for the benchmark's large tensors (hundreds of MB):
# torch's seeded Philox generator on the GPU. Both the HIP path and the
# oracle's timed sample read the same tensors (the oracle gets host copies).
# ---------------------------------------------------------------------------

def normal_device(seed: int, shape, device, dtype=None, scale: float = 1.0):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x if dtype is None else x.to(dtype)


def uniform_device(seed: int, shape, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.rand(*shape, generator=g, device=device, dtype=torch.float32)
