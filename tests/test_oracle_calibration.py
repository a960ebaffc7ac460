"""Pins for the calibration oracle (CPU only): block energies (Eq. 5),
per-prompt top-p selection and cross-prompt keep frequency (Eq. 8-9).

Energies: rows sum to one (the notes' statement, partial last block included),
the closed form of uniform attention, pure-Python brute force on tiny inputs,
and near-identity energies for block-local attention. Selection: a hand-derived
fixture, minimum cardinality against an exact-rational subset search, and the
K-largest property. Keep frequency: the notes' worked example. Planted mistakes
in copies of the oracle's steps are rejected by these pins.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle.calibration as ocal
from oracle.calibration import block_energy, keep_counts, keep_frequency_mask, select_blocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture():
    sel, keep = [], []
    for line in open(os.path.join(GOLDEN, "calibration_small.txt")):
        if line.startswith("#") or not line.strip():
            continue
        head, rest = line.split(":", 1)
        lhs, rhs = rest.split("->")
        vals, want = [float(x) for x in lhs.split()], [int(x) for x in rhs.split()]
        kv = dict(tok.split("=") for tok in head.split()[2:] if "=" in tok) if head.startswith("select") \
            else dict(tok.split("=") for tok in head.split()[1:])
        if head.startswith("select"):
            sel.append((float(kv["tau"]), vals, want))
        else:
            keep.append((int(kv["prompts"]), float(kv["rho"]), [int(v) for v in vals], want))
    return sel, keep


def _qk(N, d, seed, spread=1.0):
    rng = np.random.default_rng(seed)
    return spread * rng.standard_normal((N, d)), spread * rng.standard_normal((N, d))


# ---------------- energies ----------------

@pytest.mark.parametrize("N,B", [(64, 16), (70, 16), (33, 8), (8, 8), (5, 8)])
def test_energy_rows_sum_to_one(N, B):
    q, k = _qk(N, 6, N + B, spread=1.5)
    E = block_energy(q, k, B, 0.7)
    np.testing.assert_allclose(E.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(E >= 0)


def test_uniform_attention_closed_form():
    N, B = 50, 16
    q = np.zeros((N, 4))
    k = np.random.default_rng(1).standard_normal((N, 4))
    E = block_energy(q, k, B, 1.0)
    sizes = np.array([16, 16, 16, 2], dtype=np.float64)
    np.testing.assert_allclose(E, np.tile(sizes / N, (4, 1)), atol=1e-15)


def _brute_energy(q, k, B, scale):
    N = len(q)
    nb = -(-N // B)
    E = [[0.0] * nb for _ in range(nb)]
    for i in range(N):
        s = [scale * sum(q[i][x] * k[j][x] for x in range(len(q[i]))) for j in range(N)]
        m = max(s)
        w = [math.exp(v - m) for v in s]
        tot = sum(w)
        r = i // B
        nq = min((r + 1) * B, N) - r * B
        for j in range(N):
            E[r][j // B] += w[j] / tot / nq
    return np.array(E)


@pytest.mark.parametrize("N,B,d", [(10, 4, 3), (9, 3, 2), (7, 7, 5)])
def test_energy_brute_force(N, B, d):
    q, k = _qk(N, d, 3 * N + d)
    np.testing.assert_allclose(block_energy(q, k, B, 0.9), _brute_energy(q.tolist(), k.tolist(), B, 0.9),
                               atol=1e-13)


def test_block_local_attention_gives_identity_energies():
    # tokens of block b carry feature e_b: each query attends (almost) only to its own block
    N, B = 24, 8
    nb = N // B
    x = np.zeros((N, nb))
    for i in range(N):
        x[i, i // B] = 1.0
    E = block_energy(x, x, B, 60.0)
    np.testing.assert_allclose(E, np.eye(nb), atol=1e-20)


def test_energy_mistakes_are_caught():
    N, B = 20, 8
    q, k = _qk(N, 4, 5)
    # (a) dividing by B instead of |I_r| breaks "rows sum to one" for the partial block
    E = block_energy(q, k, B, 0.8)
    wrong = E.copy()
    wrong[-1] *= (N - 2 * B) / B
    assert not np.allclose(wrong.sum(axis=1), 1.0, atol=1e-12)
    # (b) swapped roles of q and k disagree with brute force
    assert not np.allclose(block_energy(k, q, B, 0.8), _brute_energy(q.tolist(), k.tolist(), B, 0.8), atol=1e-6)
    # (c) a softmax restricted to one key block disagrees with brute force
    def per_block_softmax(q, k, B, scale):
        nb = -(-len(q) // B)
        out = np.zeros((nb, nb))
        for r in range(nb):
            for c in range(nb):
                s = scale * q[r * B:(r + 1) * B] @ k[c * B:(c + 1) * B].T
                p = np.exp(s - s.max(axis=1, keepdims=True))
                out[r, c] = (p / p.sum(axis=1, keepdims=True)).sum() / len(s)
        return out
    assert not np.allclose(per_block_softmax(q, k, B, 0.8), _brute_energy(q.tolist(), k.tolist(), B, 0.8),
                           atol=1e-6)


# ---------------- selection ----------------

def test_selection_fixture():
    sel, _ = _fixture()
    for tau, vals, want in sel:
        got = select_blocks(np.array([vals], dtype=np.float32), tau)[0]
        np.testing.assert_array_equal(got, want, err_msg=f"tau={tau} vals={vals}")


def _min_subset_size(vals, tau):
    """Smallest number of entries whose exact (rational) sum reaches tau."""
    fr = [Fraction(float(v)) for v in vals]
    t = Fraction(float(np.float32(tau)))
    for size in range(len(vals) + 1):
        for sub in itertools.combinations(range(len(vals)), size):
            if sum((fr[i] for i in sub), Fraction(0)) >= t:
                return size
    return len(vals)


@pytest.mark.parametrize("seed", range(12))
def test_selection_is_minimal_and_takes_the_largest(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(1, 8))
    raw = rng.random(nb) ** 3 + 2.0 ** -18          # >= 2^-18: the fixed-point units are exact
    e = (raw / raw.sum()).astype(np.float32)
    if seed % 3 == 0 and nb > 2:
        e[1] = e[0]                                   # a tie
    tau = float(np.float32(rng.choice([0.5, 0.8, 0.9, 0.99, 1.0])))
    m = select_blocks(e[None], tau)[0]
    kept = int(m.sum())
    assert kept == _min_subset_size(e, tau) or (kept == nb and _min_subset_size(e, tau) == nb)
    order = sorted(range(nb), key=lambda c: (-float(e[c]), c))
    np.testing.assert_array_equal(np.flatnonzero(m), sorted(order[:kept]))


def test_selection_mistakes_are_caught():
    sel, _ = _fixture()
    def strict(e, tau):          # "reaches" read as ">" instead of ">="
        out = np.zeros_like(e, dtype=np.uint8)
        for i, row in enumerate(e):
            acc = 0.0
            for c in sorted(range(len(row)), key=lambda c: (-row[c], c)):
                if acc > tau:
                    break
                out[i, c] = 1
                acc += row[c]
        return out
    def ties_high(e, tau):        # ties to the higher index
        out = np.zeros_like(e, dtype=np.uint8)
        for i, row in enumerate(e):
            acc = 0.0
            for c in sorted(range(len(row)), key=lambda c: (-row[c], -c)):
                if acc >= tau:
                    break
                out[i, c] = 1
                acc += row[c]
        return out
    for wrong in (strict, ties_high):
        assert any(not np.array_equal(wrong(np.array([v], np.float32), t)[0], w) for t, v, w in sel)


# ---------------- keep frequency ----------------

def test_keep_frequency_worked_example():
    _, keep = _fixture()
    for n_prompts, rho, counts, want in keep:
        np.testing.assert_array_equal(keep_frequency_mask(np.array(counts), n_prompts, rho), want)


def test_keep_counts_and_extremes():
    rng = np.random.default_rng(4)
    masks = (rng.random((7, 5, 6)) < 0.4).astype(np.uint8)
    counts = keep_counts(masks)
    np.testing.assert_array_equal(counts, masks.sum(axis=0))
    np.testing.assert_array_equal(keep_frequency_mask(counts, 7, 1.0), np.all(masks, axis=0))     # intersection
    np.testing.assert_array_equal(keep_frequency_mask(counts, 7, 1e-6), np.any(masks, axis=0))    # union


def test_units_are_exact_and_monotone():
    e = np.array([1.0, 0.5, 2.0 ** -25, 2.0 ** -30, 0.0], dtype=np.float32)
    np.testing.assert_array_equal(ocal.energy_units(e), [2 ** 48, 2 ** 47, 2 ** 23, 2 ** 18, 0])
    assert ocal.threshold_units(0.5) == 2 ** 47
    with pytest.raises(ValueError):
        ocal.energy_units(np.array([-1.0], np.float32))
