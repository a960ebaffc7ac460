"""Pins for the bitmap form of the skip-list oracle (CPU only).

The bitmap encoding (one bit per key block: block c is bit c % 64 of word c // 64 of its query block's
ceil(nb/64) words; bits past nb zero) is pinned by (i) a hand-derived fixture, (ii) pure-Python brute
force over every bit, (iii) the round trip back to the dense mask, (iv) agreement of the expanded bits
with the separately pinned index-list form, and (v) planted mistakes that the pins reject.
"""
import os

import numpy as np
import pytest

from oracle import compile_skiplist
from oracle.skiplist import bitmap_to_dense, compile_bitmap

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture():
    a_masks = np.zeros((1, 1, 2, 4, 4), dtype=np.uint8)
    b_masks = np.zeros((1, 1, 1, 70, 70), dtype=np.uint8)
    a_words, b_words = None, {}
    for line in open(os.path.join(GOLDEN, "bitmap_small.txt")):
        if line.startswith("#") or not line.strip() or "none kept" in line:
            continue
        key, vals = line.split(":")
        nums = [int(x) for x in vals.split()]
        parts = key.split()
        if parts[0] == "A" and parts[1] == "mask":
            a_masks[0, 0, int(parts[2][1:]), int(parts[3][1:])] = nums
        elif parts[0] == "A" and parts[1] == "words":
            a_words = nums
        elif parts[0] == "B" and parts[1] == "kept":
            b_masks[0, 0, 0, int(parts[2][1:]), nums] = 1
        elif parts[0] == "B" and parts[1] == "words":
            b_words[int(parts[2][1:])] = nums
    return a_masks, a_words, b_masks, b_words


def test_golden_fixture():
    a_masks, a_words, b_masks, b_words = _fixture()
    bits = compile_bitmap(a_masks)
    assert bits.shape == (8, 1)
    assert [int(x) for x in bits[:, 0]] == a_words
    bits = compile_bitmap(b_masks)
    assert bits.shape == (70, 2)
    for r, want in b_words.items():
        assert [int(x) for x in bits[r]] == want, r
    assert not bits[4:].any()


def _brute(masks):
    T, L, H, nb, _ = masks.shape
    W = (nb + 63) // 64
    out = []
    for row in masks.reshape(-1, nb):
        words = []
        for w in range(W):
            v = 0
            for b in range(64):
                c = 64 * w + b
                if c < nb and row[c] != 0:
                    v += 2 ** b
            words.append(v)
        out.append(words)
    return out


@pytest.mark.parametrize("shape,p,seed", [((1, 1, 1, 1), 1.0, 0), ((1, 1, 2, 3), 0.5, 1), ((2, 1, 2, 64), 0.3, 2),
                                          ((1, 2, 1, 65), 0.5, 3), ((1, 1, 2, 130), 0.2, 4), ((1, 1, 1, 200), 0.9, 5)])
def test_brute_force(shape, p, seed):
    rng = np.random.default_rng(seed)
    T, L, H, nb = shape
    masks = (rng.random((T, L, H, nb, nb)) < p).astype(np.uint8)
    masks[masks != 0] = rng.integers(1, 256, size=int((masks != 0).sum()))   # any nonzero byte keeps
    got = [[int(x) for x in row] for row in compile_bitmap(masks)]
    assert got == _brute(masks)


@pytest.mark.parametrize("nb", [1, 63, 64, 65, 128, 591])
def test_round_trip_and_index_form(nb):
    rng = np.random.default_rng(nb)
    masks = (rng.random((1, 1, 2, nb, nb)) < 0.3).astype(np.uint8)
    bits = compile_bitmap(masks)
    assert bits.dtype == np.uint64 and bits.shape == (2 * nb, (nb + 63) // 64)
    np.testing.assert_array_equal(bitmap_to_dense(bits, 1, 1, 2, nb), (masks != 0).astype(np.uint8))
    # expanding the set bits in ascending order gives the index-list form
    rp, ci, _ = compile_skiplist(masks)
    for row in range(2 * nb):
        listed = [64 * w + b for w in range(bits.shape[1]) for b in range(64) if (int(bits[row, w]) >> b) & 1]
        assert listed == ci[rp[row]:rp[row + 1]].tolist()
    # padding bits past nb are zero
    if nb % 64:
        assert not (bits[:, -1] >> np.uint64(nb % 64)).any()


def test_planted_mistakes_are_rejected():
    a_masks, a_words, _, _ = _fixture()
    good = compile_bitmap(a_masks)[:, 0]
    # big-endian bit order within the 4 used bits
    flipped = [int("{:04b}".format(int(x))[::-1], 2) for x in good]
    assert flipped != a_words
    # a column shifted by one
    shifted = compile_bitmap(np.roll(a_masks, 1, axis=4))[:, 0]
    assert [int(x) for x in shifted] != a_words
    # word order reversed for a two-word row
    _, _, b_masks, b_words = _fixture()
    bits = compile_bitmap(b_masks)
    assert [int(x) for x in bits[0, ::-1]] != b_words[0]
