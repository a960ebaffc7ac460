"""Pins for the block-sparse attention oracle (CPU only).

What the pages fix: retained key blocks are computed exactly from the current
inputs and skipped blocks contribute nothing. So the oracle must equal softmax
attention with the token mask M[i//B, j//B]; an all-ones mask must give dense
attention; probabilities outside kept blocks must be exactly zero and every
row must sum to one.
"""
import os

import numpy as np
import pytest

from oracle import block_sparse_head, compile_skiplist
from _oracle_pins import (brute_force_attention, logsumexp_reference, max_err, parse_value,
                          sdpa_reference, token_mask)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _single_head(block_mask):
    nb = block_mask.shape[0]
    return compile_skiplist(np.asarray(block_mask, np.uint8).reshape(1, 1, 1, nb, nb))


def _random_case(seed, N, d, B, p):
    rng = np.random.default_rng(seed)
    nb = -(-N // B)
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    m = (rng.random((nb, nb)) < p) | np.eye(nb, dtype=bool)
    return q, k, v, m


def test_hand_derived_fixture():
    rows = {}
    for line in open(os.path.join(GOLDEN, "attention_small.txt")):
        if line.startswith("#") or not line.strip():
            continue
        key, vals = line.split(":", 1)
        rows[key.strip()] = vals
    mask = np.array([[int(x) for x in rows["mask r0"].split()],
                     [int(x) for x in rows["mask r1"].split()]], dtype=np.uint8)

    def mat(s):
        return np.array([[parse_value(t) for t in r.split()] for r in s.split(";")])

    q, k, v, o_want = mat(rows["q"]), mat(rows["k"]), mat(rows["v"]), mat(rows["o"])
    lse_want = np.array([parse_value(t) for t in rows["lse"].split(";")])
    rp, ci, _ = _single_head(mask)
    o, lse = block_sparse_head(q, k, v, rp, ci, 0, 2, 1.0)
    assert max_err(o, o_want) < 1e-14
    assert max_err(lse, lse_want) < 1e-14


@pytest.mark.parametrize("N,d,B", [(64, 16, 8), (96, 32, 32), (50, 8, 8), (130, 16, 64)])
def test_all_ones_equals_dense_sdpa(N, d, B):
    q, k, v, _ = _random_case(N + d, N, d, B, 0.0)
    nb = -(-N // B)
    rp, ci, _ = _single_head(np.ones((nb, nb), np.uint8))
    scale = 1.0 / np.sqrt(d)
    o, lse = block_sparse_head(q, k, v, rp, ci, 0, B, scale)
    assert max_err(o, sdpa_reference(q, k, v, None, scale)) < 1e-12
    assert max_err(lse, logsumexp_reference(q, k, np.ones((N, N), bool), scale)) < 1e-12


@pytest.mark.parametrize("N,d,B,p", [(64, 16, 8, 0.3), (100, 16, 16, 0.5), (50, 8, 8, 0.2),
                                     (257, 32, 64, 0.4)])
def test_masked_equals_sdpa_with_token_mask(N, d, B, p):
    q, k, v, m = _random_case(3 * N + B, N, d, B, p)
    rp, ci, _ = _single_head(m)
    scale = 0.37
    o, lse = block_sparse_head(q, k, v, rp, ci, 0, B, scale)
    tm = token_mask(m, N, B)
    assert max_err(o, sdpa_reference(q, k, v, tm, scale)) < 1e-12
    assert max_err(lse, logsumexp_reference(q, k, tm, scale)) < 1e-12


def test_probabilities_zero_outside_kept_blocks_and_rows_sum_to_one():
    N, d, B = 48, 8, 8
    q, k, v, m = _random_case(5, N, d, B, 0.35)
    rp, ci, _ = _single_head(m)
    _, _, P = block_sparse_head(q, k, v, rp, ci, 0, B, 0.5, return_probs=True)
    tm = token_mask(m, N, B)
    assert np.all(P[~tm] == 0.0)
    assert np.all(P[tm] > 0.0)
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) < 1e-12


@pytest.mark.parametrize("N,d,B", [(24, 4, 4), (30, 3, 8), (17, 5, 4)])
def test_brute_force_tiny(N, d, B):
    q, k, v, m = _random_case(N * d, N, d, B, 0.4)
    m[1, :] = False  # one query block with an empty list
    rp, ci, _ = _single_head(m)
    o, lse = block_sparse_head(q, k, v, rp, ci, 0, B, 0.8)
    ob, lb = brute_force_attention(q.tolist(), k.tolist(), v.tolist(), token_mask(m, N, B), 0.8)
    assert max_err(o, ob) < 1e-12
    assert max_err(lse, lb) < 1e-12


def test_closed_form_zero_queries_average_kept_values():
    N, d, B = 40, 6, 8
    _, k, v, m = _random_case(9, N, d, B, 0.5)
    q = np.zeros((N, d))
    rp, ci, _ = _single_head(m)
    o, lse = block_sparse_head(q, k, v, rp, ci, 0, B, 1.0)
    tm = token_mask(m, N, B)
    for i in range(N):
        np.testing.assert_allclose(o[i], v[tm[i]].mean(axis=0), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[i], np.log(tm[i].sum()), rtol=0, atol=1e-13)


def test_closed_form_constant_values():
    N, d, B = 40, 6, 8
    q, k, _, m = _random_case(10, N, d, B, 0.5)
    c = np.array([0.5, -2.0, 3.25, 0.0, 1.0, -0.125])
    v = np.tile(c, (N, 1))
    rp, ci, _ = _single_head(m)
    o, _ = block_sparse_head(q, k, v, rp, ci, 0, B, 1.0)
    assert np.max(np.abs(o - c)) < 1e-13


def test_closed_form_identical_keys_in_single_diagonal_block():
    N, d, B = 32, 4, 8
    rng = np.random.default_rng(12)
    q, v = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    k = np.repeat(rng.standard_normal((N // B, d)), B, axis=0)  # rows equal inside each block
    m = np.eye(N // B, dtype=np.uint8)
    rp, ci, _ = _single_head(m)
    o, _ = block_sparse_head(q, k, v, rp, ci, 0, B, 1.0)
    for r in range(N // B):
        np.testing.assert_allclose(o[r * B:(r + 1) * B], np.tile(v[r * B:(r + 1) * B].mean(0), (B, 1)),
                                   rtol=0, atol=1e-13)


def test_empty_list_gives_zero_output_and_minus_inf_lse():
    N, d, B = 16, 4, 4
    q, k, v, _ = _random_case(13, N, d, B, 0.0)
    m = np.zeros((4, 4), np.uint8)
    m[0, 0] = 1
    rp, ci, _ = _single_head(m)
    o, lse = block_sparse_head(q, k, v, rp, ci, 0, B, 1.0)
    assert np.all(o[B:] == 0.0) and np.all(np.isneginf(lse[B:]))
    assert np.all(np.isfinite(o[:B]))


def test_partial_last_block_clipped_to_N():
    # N = 50 with B = 16: the last block holds 2 tokens; no padding token may appear.
    N, d, B = 50, 8, 16
    q, k, v, m = _random_case(14, N, d, B, 0.5)
    m[:, -1] = 1
    rp, ci, _ = _single_head(m)
    o, lse = block_sparse_head(q, k, v, rp, ci, 0, B, 0.3)
    tm = token_mask(m, N, B)
    assert max_err(o, sdpa_reference(q, k, v, tm, 0.3)) < 1e-12
    assert max_err(lse, logsumexp_reference(q, k, tm, 0.3)) < 1e-12


def test_record_indexing_selects_the_right_head():
    # Two records with different masks: record 1 must use its own rows of the list.
    N, d, B = 32, 4, 8
    q, k, v, m0 = _random_case(15, N, d, B, 0.2)
    _, _, _, m1 = _random_case(16, N, d, B, 0.7)
    rp, ci, _ = compile_skiplist(np.stack([m0, m1]).astype(np.uint8).reshape(1, 1, 2, 4, 4))
    o1, _ = block_sparse_head(q, k, v, rp, ci, 1, B, 1.0)
    assert max_err(o1, sdpa_reference(q, k, v, token_mask(m1, N, B), 1.0)) < 1e-12


def test_subset_of_blocks():
    N, d, B = 40, 4, 8
    q, k, v, m = _random_case(17, N, d, B, 0.5)
    rp, ci, _ = _single_head(m)
    full, _ = block_sparse_head(q, k, v, rp, ci, 0, B, 1.0)
    part, _ = block_sparse_head(q, k, v, rp, ci, 0, B, 1.0, blocks=[1, 3])
    np.testing.assert_array_equal(part[8:16], full[8:16])
    np.testing.assert_array_equal(part[24:32], full[24:32])
    assert np.all(np.isnan(part[:8]))
