"""Pins for the interval form of the skip-list oracle (CPU only).

The interval encoding (one half-open [lo, hi) pair per maximal run of kept key
blocks) is pinned by (i) a hand-derived fixture, (ii) an independent run
enumeration with itertools.groupby, (iii) the round trip back to the dense
mask, (iv) maximality invariants, (v) agreement of the expanded runs with the
separately pinned index-list form, and (vi) planted mistakes that the pins
reject.
"""
import itertools
import os

import numpy as np
import pytest

from oracle import compile_skiplist
from oracle.skiplist import compile_intervals, intervals_to_dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture():
    masks = np.zeros((1, 1, 2, 4, 4), dtype=np.uint8)
    out = {}
    for line in open(os.path.join(GOLDEN, "intervals_small.txt")):
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


def _groupby_runs(masks):
    """Runs by grouping equal neighbours (a different formulation from the oracle's)."""
    T, L, H, nb, _ = masks.shape
    ptr, runs = [0], []
    for row in masks.reshape(-1, nb):
        pos = 0
        for kept, grp in itertools.groupby(row != 0):
            n = len(list(grp))
            if kept:
                runs.append((pos, pos + n))
            pos += n
        ptr.append(len(runs))
    return np.array(ptr), np.array(runs, dtype=np.int64).reshape(-1, 2)


def _random_masks(seed, shape, p):
    rng = np.random.default_rng(seed)
    masks = (rng.random(shape) < p).astype(np.uint8)
    masks[masks == 1] = rng.integers(1, 256, size=int(masks.sum()), dtype=np.uint8)
    return masks


def _pins_hold(fn):
    """True when a candidate encoder passes every pin used below."""
    masks, want = _fixture()
    iv_ptr, iv, order = fn(masks)
    if not (np.array_equal(iv_ptr, want["iv_ptr"]) and iv.shape == (len(want["iv_lo"]), 2)
            and np.array_equal(iv[:, 0], want["iv_lo"]) and np.array_equal(iv[:, 1], want["iv_hi"])):
        return False
    m = _random_masks(5, (1, 2, 2, 13, 13), 0.5)
    p, v, _ = fn(m)
    gp, gv = _groupby_runs(m)
    return (np.array_equal(p, gp) and np.array_equal(v, gv)
            and np.array_equal(intervals_to_dense(p, v, 1, 2, 2, 13), (m != 0).astype(np.uint8)))


def test_hand_derived_fixture():
    masks, want = _fixture()
    iv_ptr, iv, order = compile_intervals(masks)
    np.testing.assert_array_equal(iv_ptr, want["iv_ptr"])
    np.testing.assert_array_equal(iv[:, 0], want["iv_lo"])
    np.testing.assert_array_equal(iv[:, 1], want["iv_hi"])
    np.testing.assert_array_equal(order, want["order"])


@pytest.mark.parametrize("shape,p", [((1, 1, 1, 1, 1), 0.5), ((1, 1, 3, 5, 5), 0.3), ((2, 3, 2, 7, 7), 0.6),
                                     ((1, 2, 2, 16, 16), 0.1), ((1, 1, 2, 33, 33), 0.9),
                                     ((1, 1, 1, 70, 70), 0.5)])
def test_groupby_enumeration(shape, p):
    masks = _random_masks(17 + shape[-1], shape, p)
    iv_ptr, iv, _ = compile_intervals(masks)
    want_ptr, want_iv = _groupby_runs(masks)
    np.testing.assert_array_equal(iv_ptr, want_ptr)
    np.testing.assert_array_equal(iv, want_iv)
    assert iv_ptr.dtype == np.int64 and iv.dtype == np.int32


def test_round_trip_and_maximality():
    masks = _random_masks(23, (2, 2, 3, 20, 20), 0.45)
    masks[0, 1, 2, 5] = 0        # an empty row
    masks[1, 0, 0, 3] = 7        # a full row
    iv_ptr, iv, _ = compile_intervals(masks)
    back = intervals_to_dense(iv_ptr, iv, 2, 2, 3, 20)
    np.testing.assert_array_equal(back, (masks != 0).astype(np.uint8))
    for row in range(len(iv_ptr) - 1):
        runs = iv[iv_ptr[row]:iv_ptr[row + 1]]
        assert np.all(runs[:, 0] < runs[:, 1])                     # non-empty
        assert np.all(runs[1:, 0] > runs[:-1, 1])                  # separated by a gap: maximal
        assert np.all((runs >= 0) & (runs <= 20))
    row_full = (1 * 2 + 0) * 3 * 20 + 0 * 20 + 3
    np.testing.assert_array_equal(iv[iv_ptr[row_full]:iv_ptr[row_full + 1]], [[0, 20]])


def test_special_rows():
    nb = 10
    masks = np.zeros((1, 1, 1, nb, nb), dtype=np.uint8)
    masks[0, 0, 0, 0] = 1                          # all kept: one run
    masks[0, 0, 0, 1, ::2] = 1                     # alternating: nb/2 single-block runs
    masks[0, 0, 0, 2, nb - 1] = 1                  # only the last block
    iv_ptr, iv, _ = compile_intervals(masks)
    np.testing.assert_array_equal(iv[iv_ptr[0]:iv_ptr[1]], [[0, nb]])
    np.testing.assert_array_equal(iv[iv_ptr[1]:iv_ptr[2]], [[c, c + 1] for c in range(0, nb, 2)])
    np.testing.assert_array_equal(iv[iv_ptr[2]:iv_ptr[3]], [[nb - 1, nb]])
    assert iv_ptr[-1] == 1 + nb // 2 + 1           # every other row is empty


def test_runs_expand_to_index_list():
    masks = _random_masks(29, (1, 2, 2, 24, 24), 0.35)
    iv_ptr, iv, order_iv = compile_intervals(masks)
    row_ptr, col_idx, order = compile_skiplist(masks)
    for row in range(len(row_ptr) - 1):
        expanded = [c for lo, hi in iv[iv_ptr[row]:iv_ptr[row + 1]] for c in range(lo, hi)]
        np.testing.assert_array_equal(expanded, col_idx[row_ptr[row]:row_ptr[row + 1]])
    np.testing.assert_array_equal(order_iv, order)


def test_unmutated_encoder_passes_the_pins():
    assert _pins_hold(compile_intervals)


def test_inclusive_upper_bound_is_caught():
    def wrong(masks):
        p, v, o = compile_intervals(masks)
        v = v.copy()
        v[:, 1] -= 1                                # [lo, hi] closed instead of half-open
        return p, v, o
    assert not _pins_hold(wrong)


def test_non_maximal_runs_are_caught():
    def wrong(masks):
        # one interval per kept block: names the same set, but not maximal runs
        row_ptr, col_idx, order = compile_skiplist(masks)
        return row_ptr, np.stack([col_idx, col_idx + 1], axis=1).astype(np.int32), order
    assert not _pins_hold(wrong)


def test_lost_run_at_row_end_is_caught():
    def wrong(masks):
        masks = np.asarray(masks).copy()
        nb = masks.shape[-1]
        m = masks.reshape(-1, nb)
        p, v, o = compile_intervals(masks)
        keep = [i for i in range(len(v)) if v[i, 1] != nb]   # drops runs that touch the last block
        counts = [sum(1 for i in range(p[r], p[r + 1]) if v[i, 1] != nb) for r in range(len(m))]
        return np.concatenate([[0], np.cumsum(counts)]), v[keep], o
    assert not _pins_hold(wrong)


def test_rejects_non_square():
    with pytest.raises(ValueError):
        compile_intervals(np.zeros((1, 1, 1, 3, 4), dtype=np.uint8))
