"""Pins for the skip-list compilation oracle (CPU only).

The encoding is pinned by (i) a hand-derived fixture, (ii) brute-force
enumeration with plain Python loops, (iii) structural invariants and (iv) the
round trip back to the dense mask.
"""
import os

import numpy as np
import pytest

from oracle import compile_skiplist, skiplist_to_dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_skiplist_fixture():
    masks = np.zeros((1, 1, 2, 4, 4), dtype=np.uint8)
    out = {}
    for line in open(os.path.join(GOLDEN, "skiplist_small.txt")):
        if line.startswith("#") or not line.strip():
            continue
        key, vals = line.split(":")
        nums = [int(x) for x in vals.split()]
        if key.startswith("mask"):
            _, h, r = key.split()
            masks[0, 0, int(h[1:]), int(r[1:])] = nums
        else:
            out[key.strip()] = np.array(nums)
    return masks, out


def _brute_force(masks):
    T, L, H, nb, _ = masks.shape
    row_ptr = [0]
    col_idx = []
    order = []
    for t in range(T):
        for l in range(L):
            for h in range(H):
                counts = []
                for r in range(nb):
                    kept = [c for c in range(nb) if masks[t, l, h, r, c] != 0]
                    col_idx.extend(kept)
                    row_ptr.append(row_ptr[-1] + len(kept))
                    counts.append(len(kept))
                # selection sort: repeatedly take the largest count, lowest index first
                left = list(range(nb))
                while left:
                    best = left[0]
                    for r in left:
                        if counts[r] > counts[best]:
                            best = r
                    order.append(best)
                    left.remove(best)
    return np.array(row_ptr), np.array(col_idx, dtype=np.int64), np.array(order)


def test_hand_derived_fixture():
    masks, want = _parse_skiplist_fixture()
    row_ptr, col_idx, order = compile_skiplist(masks)
    np.testing.assert_array_equal(row_ptr, want["row_ptr"])
    np.testing.assert_array_equal(col_idx, want["col_idx"])
    np.testing.assert_array_equal(order, want["order"])


@pytest.mark.parametrize("shape,p", [((1, 1, 1, 1), 0.5), ((1, 1, 3, 5), 0.3), ((2, 3, 2, 7), 0.6),
                                     ((1, 2, 2, 16), 0.1), ((1, 1, 2, 33), 0.9)])
def test_brute_force_random(shape, p):
    rng = np.random.default_rng(7 + shape[-1])
    T, L, H, nb = shape
    masks = (rng.random((T, L, H, nb, nb)) < p).astype(np.uint8)
    # values other than 1 are also "keep"
    masks[masks == 1] = rng.integers(1, 256, size=int(masks.sum()), dtype=np.uint8)
    got = compile_skiplist(masks)
    want = _brute_force(masks)
    for g, w in zip(got, want):
        np.testing.assert_array_equal(g, w)
    assert got[0].dtype == np.int64 and got[1].dtype == np.int32 and got[2].dtype == np.int32


@pytest.mark.parametrize("fill", [0, 1])
def test_all_zero_and_all_one(fill):
    masks = np.full((1, 2, 3, 6, 6), fill, dtype=np.uint8)
    row_ptr, col_idx, order = compile_skiplist(masks)
    rows = 2 * 3 * 6
    assert row_ptr.shape == (rows + 1,)
    np.testing.assert_array_equal(row_ptr, np.arange(rows + 1) * (6 * fill))
    if fill:
        np.testing.assert_array_equal(col_idx, np.tile(np.arange(6), rows))
    else:
        assert col_idx.size == 0
    # equal counts: order is the identity in every record
    np.testing.assert_array_equal(order, np.tile(np.arange(6), 6))


def test_invariants_and_round_trip():
    rng = np.random.default_rng(11)
    masks = (rng.random((2, 2, 3, 20, 20)) < 0.3).astype(np.uint8)
    masks[0, 1, 2, 5] = 0  # an empty row
    row_ptr, col_idx, order = compile_skiplist(masks)
    assert row_ptr[0] == 0
    assert np.all(np.diff(row_ptr) >= 0)
    assert row_ptr[-1] == np.count_nonzero(masks)
    assert np.all((col_idx >= 0) & (col_idx < 20))
    for row in range(len(row_ptr) - 1):
        seg = col_idx[row_ptr[row]:row_ptr[row + 1]]
        assert np.all(np.diff(seg) > 0)
    back = skiplist_to_dense(row_ptr, col_idx, 2, 2, 3, 20)
    np.testing.assert_array_equal(back, (masks != 0).astype(np.uint8))
    # order is a permutation of the record's blocks with non-increasing counts
    counts = np.diff(row_ptr)
    for rec in range(2 * 2 * 3):
        o = order[rec * 20:(rec + 1) * 20]
        assert sorted(o.tolist()) == list(range(20))
        c = counts[rec * 20 + o]
        assert np.all(np.diff(c) <= 0)


def test_rejects_non_square():
    with pytest.raises(ValueError):
        compile_skiplist(np.zeros((1, 1, 1, 3, 4), dtype=np.uint8))
