"""Pins for the spatial-repetition oracle (CPU only).

Similarities: identical spatial rows and uniform attention give exactly 1,
rows attending to disjoint key sets give 0, values lie in [0, 1], and a
pure-Python brute force (its own nearest-anchor search, explicit exp and sums)
agrees on tiny inputs. Flags: a hand-derived fixture (non-anchor mean, strict
threshold). Planted mistakes (ties to the larger anchor, anchor rows in the
mean, a non-strict threshold) are rejected.
"""
import math
import os

import numpy as np
import pytest

from oracle.repetition import repetition_flags, repetition_mean, row_similarity

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture():
    d = {}
    for line in open(os.path.join(GOLDEN, "repetition_small.txt")):
        if line.startswith("#") or not line.strip():
            continue
        key, vals = line.split(":")
        d[key.strip()] = [float(x) for x in vals.split()]
    return d


def _brute(q, k, F, R, C, anchors, scale):
    def nearest(r):
        best = None
        for a in anchors:                       # ascending: strict < keeps the smaller on ties
            if best is None or abs(r - a) < abs(r - best):
                best = a
        return best
    N = len(q)
    def prow(i):
        s = [scale * sum(q[i][x] * k[j][x] for x in range(len(q[i]))) for j in range(N)]
        m = max(s)
        w = [math.exp(v - m) for v in s]
        t = sum(w)
        return [x / t for x in w]
    out = [[0.0] * R for _ in range(F)]
    for f in range(F):
        for r in range(R):
            a = nearest(r)
            dot = nr = na = 0.0
            for c in range(C):
                pr, pa = prow((f * R + r) * C + c), prow((f * R + a) * C + c)
                dot += sum(x * y for x, y in zip(pr, pa))
                nr += sum(x * x for x in pr)
                na += sum(y * y for y in pa)
            out[f][r] = dot / math.sqrt(nr * na)
    return np.array(out)


def _qk(N, d, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((N, d)), rng.standard_normal((N, d))


@pytest.mark.parametrize("F,R,C,anchors", [(2, 4, 3, [1]), (1, 5, 2, [0, 4]), (2, 6, 2, [1, 4]), (1, 16, 1, [4, 12])])
def test_brute_force(F, R, C, anchors):
    q, k = _qk(F * R * C, 3, F * R + C)
    got = row_similarity(q, k, F, R, C, anchors, 0.8)
    want = _brute(q.tolist(), k.tolist(), F, R, C, anchors, 0.8)
    np.testing.assert_allclose(got, want, atol=1e-12)


def test_identical_rows_give_one():
    F, R, C, d = 2, 5, 4, 6
    rng = np.random.default_rng(3)
    q = np.repeat(rng.standard_normal((F, 1, C, d)), R, axis=1).reshape(-1, d)
    k = rng.standard_normal((F * R * C, d))
    np.testing.assert_allclose(row_similarity(q, k, F, R, C, [2], 0.9), 1.0, atol=1e-12)


def test_uniform_attention_gives_one():
    F, R, C = 2, 4, 3
    q = np.zeros((F * R * C, 5))
    k = np.random.default_rng(4).standard_normal((F * R * C, 5))
    np.testing.assert_allclose(row_similarity(q, k, F, R, C, [0, 3], 1.0), 1.0, atol=1e-12)


def test_disjoint_attention_gives_zero():
    # each token carries its spatial row as a one-hot feature: rows attend only to their own row's keys
    F, R, C = 1, 4, 3
    x = np.zeros((F * R * C, R))
    for n in range(F * R * C):
        x[n, (n // C) % R] = 1.0
    sims = row_similarity(x, x, F, R, C, [1], 80.0)
    assert sims[0, 1] == 1.0
    np.testing.assert_allclose(np.delete(sims[0], 1), 0.0, atol=1e-30)


def test_range():
    q, k = _qk(2 * 6 * 5, 4, 9)
    s = row_similarity(q, k, 2, 6, 5, [1, 4], 1.3)
    assert np.all((s >= 0.0) & (s <= 1.0 + 1e-12))


def test_flag_fixture():
    g = _fixture()
    sims = np.array([[[g["sims f0"], g["sims f1"]]]])          # [P=1, H=1, F=2, R=4]
    anchors = [int(a) for a in g["anchors"]]
    np.testing.assert_allclose(repetition_mean(sims, anchors), [5.0 / 6.0], atol=1e-15)
    assert repetition_flags(sims, anchors, 0.8)[0] == g["threshold 0.8"][0]
    assert repetition_flags(sims, anchors, 0.85)[0] == g["threshold 0.85"][0]
    sims2 = np.array([[[g["sims2 f0"]]]])
    assert repetition_flags(sims2, anchors, 0.875)[0] == g["threshold2 0.875"][0]


def test_mistakes_are_caught():
    g = _fixture()
    sims = np.array([[[g["sims f0"], g["sims f1"]]]])
    # anchor rows inside the mean: (6 + 2) / 8 = 0.875 > 0.85 flips the 0.85 decision
    assert (sims.mean() > 0.85) != bool(g["threshold 0.85"][0])
    # ">=" instead of ">" flips the equality case
    sims2 = np.array([[[g["sims2 f0"]]]])
    assert (repetition_mean(sims2, [1])[0] >= 0.875) != bool(g["threshold2 0.875"][0])
    # ties to the larger anchor disagree with brute force where a tie exists (R = 16, row 8)
    import oracle.repetition as orep
    F, R, C, anchors = 1, 16, 1, [4, 12]
    q, k = _qk(F * R * C, 3, 11)
    want = _brute(q.tolist(), k.tolist(), F, R, C, anchors, 0.8)
    real = orep.nearest_anchor_rows
    try:
        orep.nearest_anchor_rows = lambda R, a: np.array([max(a, key=lambda x: (-abs(r - x), x)) for r in range(R)])
        wrong = orep.row_similarity(q, k, F, R, C, anchors, 0.8)
    finally:
        orep.nearest_anchor_rows = real
    assert not np.allclose(wrong, want, atol=1e-9)
