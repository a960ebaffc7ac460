"""Calibration oracle: block energies, per-prompt selection, keep frequency.
TEST INFRASTRUCTURE ONLY (see package docstring).

[Notes] Key Design 1 (block energy selection): for a fixed timestep, layer and
head, post-softmax attention P is summed over each (query block, key block)
pair at FlashAttention block granularity; a block's energy sums attention over
its keys and averages that sum over its queries (Eq. 5). For each query block
the energies are sorted in descending order and the shortest prefix whose
cumulative mass reaches the threshold is kept; mapping the kept entries back to
their positions gives the prompt's binary mask.
[Notes] Key Design 2 (cross-prompt aggregation, Eq. 8-9): the binary masks of
the calibration prompts are averaged elementwise into a keep frequency, and a
block is retained when its frequency is at least the agreement threshold rho.
A Worked Example: with 64 prompts and rho = 0.5 a block selected at least 32
times is retained.

Readings applied here (the pages leave these open):

* Eq. 5 divides by the block side B; for a partial last query block that would
  make the energies of that block sum to less than one, while the notes state
  that a query block's energies sum to one. The average is taken over the
  block's actual query count |I_r| (equal to B for every full block).
* Sort order: descending energy, ties by ascending key-block index.
* "Reaches the threshold" is cumulative mass >= tau. The cumulative mass is
  summed exactly: each fp32 energy E contributes floor(E * 2^48) units (an
  exact integer for E >= 2^-25, a truncation below), the threshold is
  ceil(tau * 2^48) units. The decision is then independent of summation order,
  so any parallel scan takes it identically. A block at sorted position s is
  kept iff the mass of the blocks before it is below the threshold; when the
  whole row stays below it, every block of the row is kept.
* Selection takes fp32 energies (the precision the kernels produce them in).
* Keep frequency: block retained iff count >= rho * |D|, evaluated exactly
  (count and |D| integers, rho an fp32 number; the product is exact in fp64).
"""
from __future__ import annotations

import math

import numpy as np

FIXED_POINT_BITS = 48


def block_energy(q, k, B: int, scale: float, blocks=None) -> np.ndarray:
    """Energies E [nb, nb] (fp64) of one head for one prompt, written from Eq. 5.

    q, k: [N, d] exact input values. P = softmax_rows(scale * q k^T) over all
    N keys; E[r, c] = (1 / |I_r|) * sum_{i in I_r} sum_{j in J_c} P[i, j].
    blocks: optional query blocks to evaluate (other rows stay NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    N = q.shape[0]
    nb = -(-N // B)
    E = np.full((nb, nb), np.nan)
    for r in (range(nb) if blocks is None else blocks):
        rows = slice(r * B, min((r + 1) * B, N))
        s = scale * (q[rows] @ k.T)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        n_q = p.shape[0]
        for c in range(nb):
            E[r, c] = p[:, c * B:min((c + 1) * B, N)].sum() / n_q
    return E


def energy_units(e32: np.ndarray) -> np.ndarray:
    """floor(E * 2^48) of fp32 energies, as int64 (the exact cumulative-mass units)."""
    e = np.asarray(e32, dtype=np.float32).astype(np.float64)
    if np.any(e < 0) or not np.all(np.isfinite(e)):
        raise ValueError("energies must be finite and >= 0")
    return np.floor(e * float(1 << FIXED_POINT_BITS)).astype(np.int64)


def threshold_units(tau: float) -> int:
    return int(math.ceil(float(np.float32(tau)) * float(1 << FIXED_POINT_BITS)))


def select_blocks(e32: np.ndarray, tau: float) -> np.ndarray:
    """Per-prompt binary mask from fp32 energies [..., nb] (last axis = key blocks).

    For every row: sort descending (ties by index), keep each block whose
    preceding cumulative mass is still below tau.
    """
    e32 = np.asarray(e32, dtype=np.float32)
    shape = e32.shape
    rows = e32.reshape(-1, shape[-1])
    units = energy_units(rows)
    need = threshold_units(tau)
    out = np.zeros(rows.shape, dtype=np.uint8)
    for i in range(rows.shape[0]):
        ranked = sorted(range(shape[-1]), key=lambda c: (-float(rows[i, c]), c))
        before = 0
        for c in ranked:
            if before >= need:
                break
            out[i, c] = 1
            before += int(units[i, c])
    return out.reshape(shape)


def keep_counts(masks) -> np.ndarray:
    """Elementwise number of prompts that selected each block (masks: [P, ...])."""
    return np.sum(np.asarray(masks) != 0, axis=0).astype(np.int32)


def keep_frequency_mask(counts, n_prompts: int, rho: float) -> np.ndarray:
    """Eq. 8-9: retained iff counts / |D| >= rho, i.e. counts >= rho * |D| (exact)."""
    bound = float(np.float32(rho)) * float(n_prompts)
    return (np.asarray(counts).astype(np.float64) >= bound).astype(np.uint8)
