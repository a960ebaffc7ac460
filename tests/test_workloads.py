"""Checks of the seeded input generators (CPU only)."""
import numpy as np
import pytest
import torch

import workloads


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.0078125, 1.01171875, 3.4e38, -1e-40],
                                 dtype=np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(workloads.bf16_bits(x), want)
    back = workloads.bf16_to_f32(want)
    np.testing.assert_array_equal(back, torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_shapes_and_counts():
    c = workloads.get_config("wan720")
    assert (c.N, c.nb, c.N - (c.nb - 1) * c.B) == (75600, 591, 80)
    c = workloads.get_config("wan480_sparse")
    assert (c.N, c.nb, c.N - (c.nb - 1) * c.B) == (32760, 256, 120)
    c = workloads.get_config("tiny")
    assert (c.N, c.nb) == (1024, 16)


def test_tiny_workload_is_deterministic():
    a = workloads.make_workload("tiny")
    b = workloads.make_workload("tiny")
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.masks, b.masks)
    assert a.q.dtype == np.float32 and a.q.shape == (2, 1024, 64)
    assert np.all(np.diagonal(a.masks[0, 0, 0]) == 1)
    assert a.rep_flags[0, 0].tolist() == [0, 1]
    assert a.anchors.tolist() == [4, 12]


def _block_sparsity(m):
    return 1.0 - m.mean()


def test_mask_rules_reach_their_targets():
    cfg = workloads.get_config("wan480_sparse")
    m = workloads.make_masks(cfg)
    s = 1.0 - m.astype(np.float64).mean()
    assert 0.66 < s < 0.72
    assert all(np.all(np.diagonal(m[0, 0, h]) == 1) for h in range(cfg.H))
    cfg4 = workloads.get_config("wan720")
    rep = workloads.make_rep_flags(cfg4)
    assert int(rep.sum()) == 8
    m4 = workloads.make_masks(cfg4, rep_flags=rep)
    sp = [1.0 - m4[0, 0, h].mean() for h in range(cfg4.H) if not rep[0, 0, h]]
    assert abs(np.mean(sp) - 0.68) < 0.01
    assert min(sp) > 0.39 and max(sp) < 0.91


def test_rep_flags_counts():
    assert int(workloads.make_rep_flags(workloads.get_config("wan480_dual")).sum()) == 10
    assert int(workloads.make_rep_flags(workloads.get_config("wan480_sparse")).sum()) == 0


def test_frame_distance_band_fractions_720p():
    d = workloads.block_frame_distance(75600, 128, 21, 45, 80)
    fr = [(d <= w).mean() for w in range(9)]
    np.testing.assert_allclose(fr, [0.0505, 0.1409, 0.2269, 0.3083, 0.3853, 0.4578, 0.5256, 0.5889, 0.6478],
                               atol=5e-4)


def test_dictionary_workload_small():
    cfg, masks, flags = workloads.make_dictionary_workload(0.68, 0.25, L=2, H=4)
    assert masks.shape == (1, 2, 4, 256, 256)
    assert int(flags.sum()) == 2 * 1
    s = 1.0 - masks.astype(np.float64).mean()
    assert abs(s - 0.68) < 0.01
    _, dense, _ = workloads.make_dictionary_workload(0.0, 0.0, L=1, H=2)
    assert dense.min() == 1


def test_dictionary_prefix_of_layers():
    # The benchmark's sweep summary times the first layers of each dictionary point, drawn with
    # L = 2; they must be the first two layers of the full 40-layer dictionary.
    for sp, rf in ((0.68, 0.25), (0.85, 0.10)):
        _, m40, f40 = workloads.make_dictionary_workload(sp, rf)
        _, m2, f2 = workloads.make_dictionary_workload(sp, rf, L=2)
        np.testing.assert_array_equal(m40[:, :2], m2)
        np.testing.assert_array_equal(f40[:, :2], f2)
