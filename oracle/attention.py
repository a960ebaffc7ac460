"""Attention oracle in fp64. TEST INFRASTRUCTURE ONLY (see package docstring).

Block-sparse path ([Notes] Overall Architecture and Key Design 4; [Abstract]):
the retained connections are computed densely from the current Q, K, V and
the unselected ones are skipped. For query block r with token set I_r and the
union J of its listed key blocks' token sets,

    S = scale * Q[I_r] K[J]^T,  P = softmax_rows(S),  O[I_r] = P V[J],
    lse[I_r] = log sum_j exp(S_ij).

Anchor-row path ([Notes] Key Design 3, Key Design 4, A Worked Example): only
anchor spatial rows compute attention, over all keys and values; every other
spatial row of the same frame receives the output of its nearest anchor row.

Readings applied here (the pages leave these open):

* Token order: n = (f*R + r)*C + c (frame, spatial row, column).
* Blocks: block b covers tokens [b*B, min((b+1)*B, N)); a partial last block
  simply has fewer tokens (no padding tokens exist).
* A query block whose list is empty gets O = 0 and lse = -inf.
* Nearest anchor: argmin |r - a| over the anchor rows, ties to the smaller a.
* Broadcast unit: the same column c of the same frame f; no cross-frame copy.
* A repetitive head ignores its block mask (the two paths are alternatives).
* lse is returned in natural-log units.
"""
from __future__ import annotations

import numpy as np


def block_tokens(b: int, B: int, N: int) -> np.ndarray:
    """Token indices of block b: [b*B, min((b+1)*B, N))."""
    return np.arange(b * B, min((b + 1) * B, N), dtype=np.int64)


def _softmax_attention(qi: np.ndarray, kj: np.ndarray, vj: np.ndarray, scale: float):
    """Plain softmax attention of the query rows qi over keys kj / values vj (fp64)."""
    s = scale * (qi @ kj.T)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p / l) @ vj
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse, p / l


def block_sparse_head(q, k, v, row_ptr, col_idx, record: int, B: int, scale: float,
                      blocks=None, return_probs: bool = False):
    """Block-sparse attention of one head.

    q, k, v: [N, d] arrays holding the exact input values (widened to fp64).
    row_ptr, col_idx: a compiled skip list; this head's rows are
    record*nb + r for query blocks r < nb = ceil(N/B).
    blocks: optional iterable of query blocks to evaluate (others stay NaN).
    return_probs: also return the dense [N, N] probability matrix (tiny N only),
    with exact zeros wherever a key block was skipped.
    Returns (O [N, d], lse [N]) or (O, lse, P).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    nb = -(-N // B)
    out = np.full((N, d), np.nan)
    lse = np.full(N, np.nan)
    probs = np.zeros((N, N)) if return_probs else None
    for r in (range(nb) if blocks is None else blocks):
        rows = block_tokens(r, B, N)
        row = record * nb + r
        cols = col_idx[row_ptr[row]:row_ptr[row + 1]]
        if len(cols) == 0:
            out[rows] = 0.0
            lse[rows] = -np.inf
            continue
        keys = np.concatenate([block_tokens(int(c), B, N) for c in cols])
        o, l, p = _softmax_attention(q[rows], k[keys], v[keys], scale)
        out[rows] = o
        lse[rows] = l
        if return_probs:
            probs[np.ix_(rows, keys)] = p
    if return_probs:
        return out, lse, probs
    return out, lse


def nearest_anchor_rows(R: int, anchors) -> np.ndarray:
    """For every spatial row r < R, the anchor row it copies from.

    argmin over anchors a of |r - a|; on a tie the smaller anchor row wins.
    """
    anchors = [int(a) for a in anchors]
    out = np.empty(R, dtype=np.int64)
    for r in range(R):
        best = None
        for a in sorted(anchors):
            if best is None or abs(r - a) < abs(r - best):
                best = a
        out[r] = best
    return out


def anchor_head(q, k, v, F: int, R: int, C: int, anchors, scale: float, frames=None):
    """Anchor-row attention with broadcast for one repetitive head.

    For every frame f and anchor row a, the C query tokens (f, a, c) attend to
    all N keys; rows whose nearest anchor is a receive that output (and lse)
    column by column. frames: optional subset of frames to evaluate.
    Returns (O [N, d], lse [N]); tokens of frames not evaluated stay NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    if N != F * R * C:
        raise ValueError("N must equal F*R*C")
    amap = nearest_anchor_rows(R, anchors)
    out = np.full((N, d), np.nan)
    lse = np.full(N, np.nan)
    cols = np.arange(C, dtype=np.int64)
    for f in (range(F) if frames is None else frames):
        for a in sorted({int(x) for x in anchors}):
            toks = (f * R + a) * C + cols
            o, l, _ = _softmax_attention(q[toks], k, v, scale)
            for r in range(R):
                if amap[r] == a:
                    dst = (f * R + r) * C + cols
                    out[dst] = o
                    lse[dst] = l
    return out, lse


def layer_forward(q, k, v, row_ptr, col_idx, T: int, L: int, H: int, B: int, t: int, l: int,
                  rep_flags, F: int, R: int, C: int, anchors, scale: float, heads=None):
    """One attention layer-call: per head, the path chosen by the repetition flag.

    q, k, v: [H, N, d]. rep_flags: [T, L, H] (nonzero = repetitive head).
    The record of head h is (t*L + l)*H + h. heads: optional subset to evaluate.
    Returns (O [H, N, d], lse [H, N]); heads not evaluated stay NaN.
    """
    Hq, N, d = np.shape(q)
    out = np.full((Hq, N, d), np.nan)
    lse = np.full((Hq, N), np.nan)
    rep_flags = np.asarray(rep_flags)
    for h in (range(H) if heads is None else heads):
        if rep_flags[t, l, h]:
            out[h], lse[h] = anchor_head(q[h], k[h], v[h], F, R, C, anchors, scale)
        else:
            rec = (t * L + l) * H + h
            out[h], lse[h] = block_sparse_head(q[h], k[h], v[h], row_ptr, col_idx, rec, B, scale)
    return out, lse
