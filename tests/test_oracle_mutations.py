"""The pins catch plausible oracle mistakes (CPU only).

Each case plants one mistake in the oracle (by monkeypatching a copy of its
step) and checks that at least one of the independent references rejects the
result. This is what makes the pins meaningful: an oracle that passes them
cannot carry a transposed mask, a flipped sign, a shifted block index, a
dropped tail, a wrong tie-break or a cross-frame broadcast.
"""
import numpy as np
import pytest

import oracle.attention as oatt
from oracle import anchor_head, block_sparse_head, compile_skiplist, nearest_anchor_rows
from _oracle_pins import max_err, sdpa_reference, token_mask

N, D, B = 48, 8, 8


def _case(seed=31):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    nb = N // B
    m = (rng.random((nb, nb)) < 0.4) | np.eye(nb, dtype=bool)
    m[0, nb - 1] = True
    m[nb - 1, 0] = False   # asymmetric on purpose
    return q, k, v, m.astype(np.uint8)


def _pin_masked(q, k, v, m, o):
    return max_err(o, sdpa_reference(q, k, v, token_mask(m, N, B), 0.7)) < 1e-12


def test_unmutated_passes():
    q, k, v, m = _case()
    rp, ci, _ = compile_skiplist(m.reshape(1, 1, 1, *m.shape))
    o, _ = block_sparse_head(q, k, v, rp, ci, 0, B, 0.7)
    assert _pin_masked(q, k, v, m, o)


def test_transposed_mask_is_caught():
    q, k, v, m = _case()
    rp, ci, _ = compile_skiplist(m.T.copy().reshape(1, 1, 1, *m.shape))
    o, _ = block_sparse_head(q, k, v, rp, ci, 0, B, 0.7)
    assert not _pin_masked(q, k, v, m, o)


def test_flipped_score_sign_is_caught(monkeypatch):
    orig = oatt._softmax_attention
    monkeypatch.setattr(oatt, "_softmax_attention", lambda qi, kj, vj, s: orig(qi, kj, vj, -s))
    q, k, v, m = _case()
    rp, ci, _ = compile_skiplist(m.reshape(1, 1, 1, *m.shape))
    o, _ = oatt.block_sparse_head(q, k, v, rp, ci, 0, B, 0.7)
    assert not _pin_masked(q, k, v, m, o)


def test_transposed_value_operand_is_caught(monkeypatch):
    # P V computed with the keys' rows of Q instead of V (operand mix-up).
    orig = oatt._softmax_attention
    monkeypatch.setattr(oatt, "_softmax_attention", lambda qi, kj, vj, s: orig(qi, kj, kj, s))
    q, k, v, m = _case()
    rp, ci, _ = compile_skiplist(m.reshape(1, 1, 1, *m.shape))
    o, _ = oatt.block_sparse_head(q, k, v, rp, ci, 0, B, 0.7)
    assert not _pin_masked(q, k, v, m, o)


def test_shifted_row_index_is_caught():
    q, k, v, m = _case()
    shifted = np.roll(m, 1, axis=0)  # query block r reads row r-1's list
    rp, ci, _ = compile_skiplist(shifted.reshape(1, 1, 1, *m.shape))
    o, _ = block_sparse_head(q, k, v, rp, ci, 0, B, 0.7)
    assert not _pin_masked(q, k, v, m, o)


def test_dropped_partial_tail_is_caught(monkeypatch):
    # Clipping the last key block one token short of N.
    n2, b2 = 50, 16
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((n2, D)) for _ in range(3))
    m = np.ones((4, 4), np.uint8)
    orig = oatt.block_tokens
    monkeypatch.setattr(oatt, "block_tokens", lambda b, B_, N_: orig(b, B_, N_ - 1) if b == 3 else orig(b, B_, N_))
    rp, ci, _ = compile_skiplist(m.reshape(1, 1, 1, 4, 4))
    o, _ = oatt.block_sparse_head(q, k, v, rp, ci, 0, b2, 0.7)
    assert max_err(o[:48], sdpa_reference(q, k, v, np.ones((n2, n2), bool), 0.7)[:48]) > 1e-9


def test_tie_to_larger_anchor_is_caught():
    want = [4] * 9 + [12] * 7   # golden map for R=16, anchors {4, 12}
    def wrong(R, anchors):
        out = []
        for r in range(R):
            best = None
            for a in sorted(anchors):
                if best is None or abs(r - a) <= abs(r - best):
                    best = a
            out.append(best)
        return np.array(out)
    assert nearest_anchor_rows(16, [4, 12]).tolist() == want
    assert wrong(16, [4, 12]).tolist() != want


def test_cross_frame_broadcast_is_caught(monkeypatch):
    # A broadcast that copies frame 0's anchor output into every frame.
    F, R, C, d = 3, 6, 2, 4
    anchors = [1, 4]
    n3 = F * R * C
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((n3, d)) for _ in range(3))
    amap = nearest_anchor_rows(R, anchors)
    q3 = q.reshape(F, R, C, d)
    q3[:] = q3[:, amap]
    q = q3.reshape(n3, d)
    good, _ = anchor_head(q, k, v, F, R, C, anchors, 1.0)
    assert max_err(good, sdpa_reference(q, k, v, None, 1.0)) < 1e-12
    bad = good.reshape(F, R * C, d).copy()
    bad[1:] = bad[0]
    assert max_err(bad.reshape(n3, d), sdpa_reference(q, k, v, None, 1.0)) > 1e-6
