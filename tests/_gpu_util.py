"""Helpers for the GPU parity tests: device copies of the seeded inputs and
comparison against the oracle. Inputs always come from ``workloads`` (or
seeded numpy draws here); expected values always come from ``oracle``."""
import sys

import numpy as np
import torch

import workloads

TOL_BF16 = 1e-2      # max |O_gpu - O_oracle| for bf16 inputs
TOL_F32 = 1e-4       # ... for fp32 inputs
TOL_LSE_BF16 = 1e-3
TOL_LSE_F32 = 1e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to_device(arr: np.ndarray, dtype: str) -> torch.Tensor:
    return dev_bf16(arr) if dtype == "bf16" else dev_f32(arr)


def exact_values(arr: np.ndarray, dtype: str) -> np.ndarray:
    """The exact values the GPU consumes, as float32 (bf16 widens exactly)."""
    return workloads.bf16_to_f32(arr) if dtype == "bf16" else np.asarray(arr, np.float32)


def random_qkv(H, N, d, dtype, seed):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((H, N, d), dtype=np.float32) for _ in range(3))
    if dtype == "bf16":
        return workloads.bf16_bits(q), workloads.bf16_bits(k), workloads.bf16_bits(v)
    return q, k, v


def alloc_out(H, N, d, dtype, fill=float("nan")):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    o = torch.full((H, N, d), fill, dtype=tdt, device="cuda")
    lse = torch.full((H, N), fill, dtype=torch.float32, device="cuda")
    return o, lse


def host64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    """Max |a - b| where equal infinities count as 0 and any NaN as infinite."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.abs(a - b)
    d[same_inf] = 0.0
    if np.isnan(d).any():
        return float("inf")
    return float(d.max()) if d.size else 0.0
