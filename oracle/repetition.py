"""Spatial-repetition oracle: row similarities and repetition flags.
TEST INFRASTRUCTURE ONLY (see package docstring).

[Notes] Key Design 3 (spatial repetition detection): a separate calibration
branch compares attention distributions across spatial rows of the same
frame. The attention of each spatial row is flattened, compared by cosine
similarity with the nearest anchor row, and the similarities are averaged
over frames, rows and calibration prompts; a (timestep, layer, head) is marked
repetitive only when that mean exceeds the threshold (five equally spaced
anchor rows and 0.87 by default).

Readings applied here (the pages leave these open):

* The attention of spatial row r of frame f is the C x N block of
  post-softmax probabilities P[(f, r, c), j] (all C tokens of the row, all N
  keys), flattened into one vector.
* The nearest anchor is the one the broadcast uses: argmin |r - a|, ties to
  the smaller a (same reading as the anchor path).
* The mean runs over the non-anchor rows of every frame (the rows whose output
  the broadcast would replace); anchor rows would only add a trivial 1.
* "Exceeds" is strict: repetitive iff mean > threshold.
"""
from __future__ import annotations

import numpy as np

from .attention import nearest_anchor_rows


def _probs(q, k, rows, scale):
    s = scale * (q[rows] @ k.T)
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(axis=1, keepdims=True)


def row_similarity(q, k, F: int, R: int, C: int, anchors, scale: float, frames=None) -> np.ndarray:
    """Cosine similarity [F, R] of each spatial row's flattened attention with its nearest anchor row's.

    q, k: [N, d] exact input values (N = F*R*C). Anchor rows get 1. Rows of
    frames not listed in `frames` stay NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    a_of = nearest_anchor_rows(R, anchors)
    out = np.full((F, R), np.nan)
    for f in (range(F) if frames is None else frames):
        tok = lambda r: (f * R + r) * C + np.arange(C)
        vec = {a: _probs(q, k, tok(a), scale).ravel() for a in sorted(set(int(x) for x in anchors))}
        for r in range(R):
            a = int(a_of[r])
            if r == a:
                out[f, r] = 1.0
                continue
            v = _probs(q, k, tok(r), scale).ravel()
            out[f, r] = float(v @ vec[a]) / float(np.sqrt((v @ v) * (vec[a] @ vec[a])))
    return out


def repetition_mean(sims, anchors) -> np.ndarray:
    """Mean similarity over prompts, frames and non-anchor rows. sims: [P, H, F, R] -> [H]."""
    sims = np.asarray(sims, dtype=np.float64)
    R = sims.shape[-1]
    keep = np.ones(R, dtype=bool)
    keep[np.asarray(anchors, dtype=np.int64)] = False
    return sims[..., keep].mean(axis=(0, 2, 3))


def repetition_flags(sims, anchors, threshold: float) -> np.ndarray:
    """uint8 [H]: 1 where the mean similarity exceeds the threshold."""
    return (repetition_mean(sims, anchors) > float(np.float32(threshold))).astype(np.uint8)
