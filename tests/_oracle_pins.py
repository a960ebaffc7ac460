"""Independent references used to pin the oracle (CPU only).

None of these call into ``oracle``: they restate what the pages and the
mathematics fix with different means (PyTorch's scaled-dot-product attention
with an explicit token mask, scipy's logsumexp, pure-Python loops, closed
forms), so that a mistake in the oracle shows up as a disagreement.
"""
import math
from fractions import Fraction

import numpy as np
import scipy.special
import torch


def token_mask(block_mask: np.ndarray, N: int, B: int) -> np.ndarray:
    """Expand an [nb, nb] block mask to the [N, N] token mask M[i//B, j//B]."""
    idx = np.arange(N) // B
    return np.asarray(block_mask, dtype=bool)[np.ix_(idx, idx)]


def sdpa_reference(q, k, v, tok_mask, scale):
    """torch.nn.functional.scaled_dot_product_attention in fp64 on the CPU.

    Rows without any kept key are returned as NaN (SDPA leaves them undefined).
    """
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))[None]
    kt = torch.from_numpy(np.asarray(k, dtype=np.float64))[None]
    vt = torch.from_numpy(np.asarray(v, dtype=np.float64))[None]
    m = None if tok_mask is None else torch.from_numpy(np.asarray(tok_mask, dtype=bool))[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)[0].numpy()
    if tok_mask is not None:
        o = o.copy()
        o[~np.asarray(tok_mask, dtype=bool).any(axis=1)] = np.nan
    return o


def logsumexp_reference(q, k, tok_mask, scale):
    s = scale * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    s = np.where(tok_mask, s, -np.inf)
    return scipy.special.logsumexp(s, axis=1)


def brute_force_attention(q, k, v, tok_mask, scale):
    """Pure-Python loops over tokens (tiny inputs only)."""
    N, d = len(q), len(q[0])
    out, lse = [], []
    for i in range(N):
        keys = [j for j in range(N) if tok_mask[i][j]]
        if not keys:
            out.append([0.0] * d)
            lse.append(-math.inf)
            continue
        scores = [scale * sum(float(q[i][t]) * float(k[j][t]) for t in range(d)) for j in keys]
        m = max(scores)
        e = [math.exp(s - m) for s in scores]
        tot = sum(e)
        out.append([sum(e[n] * float(v[j][t]) for n, j in enumerate(keys)) / tot for t in range(d)])
        lse.append(m + math.log(tot))
    return np.array(out), np.array(lse)


def parse_value(tok: str) -> float:
    """Values in the golden files: integers, fractions a/b, ln<int>."""
    tok = tok.strip()
    if tok.startswith("ln"):
        return math.log(int(tok[2:]))
    return float(Fraction(tok))


def max_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.shape != b.shape:
        return math.inf
    both_nan = np.isnan(a) & np.isnan(b)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        d = np.abs(a - b)
    d[both_nan | same_inf] = 0.0
    if np.isnan(d).any():
        return math.inf
    return float(d.max()) if d.size else 0.0
