"""Pins for the anchor-row oracle and the per-head dual-path layer oracle (CPU only).

What the pages fix (notes, Key Designs 3 and 4): anchor rows attend to all
keys and values; every spatial row receives its nearest anchor's output within
the same frame; with k anchors a frame computes k*C instead of R*C queries;
the two paths are alternatives chosen per head by the repetition flag.
"""
import os

import numpy as np
import pytest

import workloads
from oracle import anchor_head, block_sparse_head, compile_skiplist, layer_forward, nearest_anchor_rows
from _oracle_pins import max_err, sdpa_reference

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_maps():
    maps = []
    for line in open(os.path.join(GOLDEN, "anchor_rows.txt")):
        if not line.startswith("R="):
            continue
        head, vals = line.split(":")
        R = int(head.split()[0][2:])
        anchors = [int(x) for x in head.split()[1].split("=")[1].split(",")]
        maps.append((R, anchors, [int(x) for x in vals.split()]))
    return maps


@pytest.mark.parametrize("case", range(3))
def test_nearest_anchor_golden(case):
    R, anchors, want = _golden_maps()[case]
    np.testing.assert_array_equal(nearest_anchor_rows(R, anchors), want)


@pytest.mark.parametrize("case", range(3))
def test_generator_anchor_sets_match_golden(case):
    R, anchors, _ = _golden_maps()[case]
    np.testing.assert_array_equal(workloads.equally_spaced_anchor_rows(R, len(anchors)), anchors)


def _rand(seed, N, d):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, d)) for _ in range(3))


@pytest.mark.parametrize("F,R,C,anchors", [(2, 6, 3, [1, 4]), (3, 16, 4, [4, 12]), (2, 9, 5, [2, 7]),
                                           (1, 5, 2, [0])])
def test_identical_rows_make_broadcast_exact(F, R, C, anchors):
    N, d = F * R * C, 8
    q, k, v = _rand(F * R + C, N, d)
    amap = nearest_anchor_rows(R, anchors)
    q3 = q.reshape(F, R, C, d)
    q3[:] = q3[:, amap]  # every spatial row repeats its anchor's queries
    q = q3.reshape(N, d)
    o, lse = anchor_head(q, k, v, F, R, C, anchors, 0.6)
    assert max_err(o, sdpa_reference(q, k, v, None, 0.6)) < 1e-12


def test_anchor_rows_are_exact_dense_attention_and_copies_are_bitwise():
    F, R, C, d = 2, 10, 4, 6
    anchors = [2, 7]
    N = F * R * C
    q, k, v = _rand(21, N, d)
    o, lse = anchor_head(q, k, v, F, R, C, anchors, 0.5)
    dense = sdpa_reference(q, k, v, None, 0.5)
    amap = nearest_anchor_rows(R, anchors)
    for f in range(F):
        for r in range(R):
            dst = slice((f * R + r) * C, (f * R + r + 1) * C)
            src = slice((f * R + amap[r]) * C, (f * R + amap[r] + 1) * C)
            np.testing.assert_array_equal(o[dst], o[src])
            np.testing.assert_array_equal(lse[dst], lse[src])
        for a in anchors:
            s = slice((f * R + a) * C, (f * R + a + 1) * C)
            assert max_err(o[s], dense[s]) < 1e-12


def test_non_anchor_queries_are_never_read():
    F, R, C, d = 2, 8, 3, 4
    anchors = [1, 5]
    N = F * R * C
    q, k, v = _rand(22, N, d)
    o1, l1 = anchor_head(q, k, v, F, R, C, anchors, 1.0)
    q2 = q.copy().reshape(F, R, C, d)
    other = [r for r in range(R) if r not in anchors]
    q2[:, other] = np.random.default_rng(5).standard_normal((F, len(other), C, d)) * 100
    o2, l2 = anchor_head(q2.reshape(N, d), k, v, F, R, C, anchors, 1.0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_distinct_query_count_is_k_rows_per_frame():
    # k anchors in a frame of R rows leave F*k*C distinct outputs (interaction
    # sparsity 1 - k/R over the query rows).
    F, R, C, d = 3, 9, 4, 5
    anchors = [1, 4, 7]
    N = F * R * C
    q, k, v = _rand(23, N, d)
    o, _ = anchor_head(q, k, v, F, R, C, anchors, 1.0)
    assert len({tuple(row) for row in o}) == F * len(anchors) * C


def test_no_cross_frame_copy():
    # Outputs of frame f depend on frame f's anchor queries only.
    F, R, C, d = 3, 6, 2, 4
    anchors = [2]
    N = F * R * C
    q, k, v = _rand(24, N, d)
    o1, _ = anchor_head(q, k, v, F, R, C, anchors, 1.0)
    q2 = q.copy()
    q2[(0 * R + 2) * C:(0 * R + 3) * C] += 1.0  # perturb frame 0's anchor row only
    o2, _ = anchor_head(q2, k, v, F, R, C, anchors, 1.0)
    fw = R * C
    assert not np.array_equal(o1[:fw], o2[:fw])
    np.testing.assert_array_equal(o1[fw:], o2[fw:])


def test_layer_dispatch_selects_paths_and_ignores_masks_of_repetitive_heads():
    cfg = workloads.get_config("tiny")
    wl = workloads.make_workload(cfg)
    q, k, v = (x.astype(np.float64) for x in (wl.q, wl.k, wl.v))
    rp, ci, _ = compile_skiplist(wl.masks)
    args = (cfg.T, cfg.L, cfg.H, cfg.B, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors, wl.scale)
    o, lse = layer_forward(q, k, v, rp, ci, *args)
    assert wl.rep_flags[0, 0].tolist() == [0, 1]
    o0, l0 = block_sparse_head(q[0], k[0], v[0], rp, ci, 0, cfg.B, wl.scale)
    o1, l1 = anchor_head(q[1], k[1], v[1], cfg.F, cfg.R, cfg.C, wl.anchors, wl.scale)
    np.testing.assert_array_equal(o[0], o0)
    np.testing.assert_array_equal(o[1], o1)
    np.testing.assert_array_equal(lse[1], l1)
    # a different mask for the repetitive head changes nothing
    masks2 = wl.masks.copy()
    masks2[0, 0, 1] = 1 - masks2[0, 0, 1]
    np.fill_diagonal(masks2[0, 0, 1], 1)
    rp2, ci2, _ = compile_skiplist(masks2)
    o_b, _ = layer_forward(q, k, v, rp2, ci2, *args)
    np.testing.assert_array_equal(o_b, o)
