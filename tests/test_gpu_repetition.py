"""GPU spatial-repetition parity: row similarities within tolerance of the fp64
oracle, flags and means equal to the oracle's on identical similarity inputs.

Similarity tolerance: probabilities are formed in fp32 from exact bf16 (or
fp32) inputs with each query's fp32 log-sum-exp, and three fp32 sums over up
to C*N products are divided; the cosine's error stays around 1e-6, so 1e-5
absolute is used.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import calibrated_block_sparse_skiplist_amd as cal
from _gpu_util import exact_values, say, to_device

pytestmark = pytest.mark.gpu

TOL_SIM = 1e-5


def _sims(q, k, F, R, C, anchors, dtype, scale=None):
    H, N, d = q.shape
    sim = torch.full((H, F, R), float("nan"), dtype=torch.float32, device="cuda")
    cal.calibatt_spatial_similarity(to_device(q, dtype), to_device(k, dtype), F, R, C, anchors, sim, scale=scale)
    torch.cuda.synchronize()
    return sim.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("F,R,C,anchors,d,dtype", [
    (2, 10, 20, [2, 7], 128, "bf16"), (3, 16, 16, [4, 12], 64, "bf16"), (2, 30, 8, [3, 9, 15, 21, 27], 128, "bf16"),
    (1, 5, 150, [2], 128, "bf16"), (2, 8, 10, [1, 5], 64, "f32"), (2, 6, 5, [0], 128, "f32"),
    # rows wider than one workgroup (two passes), the 480p row width with a short last group,
    # one column per row (hundreds of rows per group, fewer keys than one stage), an odd width
    (1, 3, 300, [1], 64, "bf16"), (2, 4, 52, [1], 128, "bf16"), (2, 7, 1, [3], 64, "bf16"),
    (3, 5, 33, [0, 4], 128, "bf16"),
])
def test_row_similarity_small(F, R, C, anchors, d, dtype):
    say(f"[repetition] F={F} R={R} C={C} anchors={anchors} d={d} {dtype}")
    N = F * R * C
    q, k = workloads.make_calibration_prompts(N, d, F, R, C, 2, 1, dtype=dtype, seed=9000 + N)
    q, k = q[0], k[0]
    scale = float(np.float32(1.0 / np.sqrt(d)))
    got = _sims(q, k, F, R, C, anchors, dtype, scale)
    for h in range(2):
        want = oracle.row_similarity(exact_values(q[h], dtype), exact_values(k[h], dtype), F, R, C, anchors, scale)
        err = float(np.max(np.abs(got[h] - want)))
        say(f"  head {h}: max|d sim| = {err:.2e}, sims in [{want.min():.3f}, {want.max():.3f}]")
        assert err <= TOL_SIM, (h, err)


def test_head_subset_leaves_other_heads():
    F, R, C, d, H = 2, 6, 24, 128, 3
    N = F * R * C
    anchors = [1, 4]
    q, k = workloads.make_calibration_prompts(N, d, F, R, C, H, 1, seed=9300)
    q, k = q[0], k[0]
    scale = float(np.float32(1.0 / np.sqrt(d)))
    sim = torch.full((H, F, R), float("nan"), dtype=torch.float32, device="cuda")
    cal.calibatt_spatial_similarity(to_device(q, "bf16"), to_device(k, "bf16"), F, R, C, anchors, sim,
                                    heads=[2, 0], scale=scale)
    torch.cuda.synchronize()
    got = sim.cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(got[1]))
    for h in (0, 2):
        want = oracle.row_similarity(exact_values(q[h], "bf16"), exact_values(k[h], "bf16"), F, R, C, anchors, scale)
        assert float(np.max(np.abs(got[h] - want))) <= TOL_SIM


def test_identical_rows_give_one():
    F, R, C, d = 3, 12, 40, 128
    rng = np.random.default_rng(5)
    q = np.repeat(rng.standard_normal((2, F, 1, C, d), dtype=np.float32), R, axis=2).reshape(2, -1, d)
    k = rng.standard_normal((2, F * R * C, d), dtype=np.float32)
    got = _sims(workloads.bf16_bits(q), workloads.bf16_bits(k), F, R, C, [3, 8], "bf16")
    np.testing.assert_allclose(got, 1.0, atol=TOL_SIM)


def test_row_similarity_720p_head():
    cfg = workloads.get_config("wan720")
    say(f"[repetition] 720p head, N={cfg.N}")
    q, k = workloads.make_calibration_prompts(cfg.N, cfg.d, cfg.F, cfg.R, cfg.C, 1, 1, seed=9500)
    anchors = workloads.equally_spaced_anchor_rows(cfg.R, 5)
    got = _sims(q[0], k[0], cfg.F, cfg.R, cfg.C, anchors, "bf16")
    assert np.all((got > 0) & (got <= 1 + TOL_SIM))
    want = oracle.row_similarity(exact_values(q[0, 0], "bf16"), exact_values(k[0, 0], "bf16"), cfg.F, cfg.R, cfg.C,
                                 anchors, float(np.float32(1.0 / np.sqrt(cfg.d))), frames=[0])
    err = float(np.max(np.abs(got[0, 0] - want[0])))
    say(f"  frame 0: max|d sim| = {err:.2e}, mean sim {want[0].mean():.4f}")
    assert err <= TOL_SIM


def test_flags_and_mean_on_fixed_similarities():
    rng = np.random.default_rng(8)
    P, H, F, R = 3, 40, 21, 45
    anchors = [4, 13, 22, 31, 40]
    base = rng.uniform(0.6, 1.0, size=(1, H, 1, 1))
    sims = np.clip(base + rng.normal(0.0, 0.05, size=(P, H, F, R)), 0.0, 1.0).astype(np.float32)
    dev = torch.from_numpy(sims).cuda()
    flags = torch.full((H,), 7, dtype=torch.uint8, device="cuda")
    mean = torch.empty((H,), dtype=torch.float32, device="cuda")
    cal.calibatt_repetition_flags(dev, anchors, 0.87, flags=flags, mean=mean)
    torch.cuda.synchronize()
    want_mean = oracle.repetition_mean(sims, anchors)
    np.testing.assert_allclose(mean.cpu().numpy(), want_mean, rtol=1e-6)
    assert np.all(np.abs(want_mean - 0.87) > 1e-5)        # no decision within rounding of the threshold
    np.testing.assert_array_equal(flags.cpu().numpy(), oracle.repetition_flags(sims, anchors, 0.87))


def test_flags_hand_fixture():
    sims = np.array([[[[0.75, 1.0, 1.0, 0.5], [1.0, 1.0, 0.75, 1.0]]]], dtype=np.float32)   # [1, 1, 2, 4]
    flags = torch.empty((1,), dtype=torch.uint8, device="cuda")
    for thr, want in ((0.8, 1), (0.85, 0)):
        cal.calibatt_repetition_flags(torch.from_numpy(sims).cuda(), [1], thr, flags=flags)
        torch.cuda.synchronize()
        assert int(flags.item()) == want
    eq = np.array([[[[1.0, 1.0, 0.75, 0.875]]]], dtype=np.float32)
    cal.calibatt_repetition_flags(torch.from_numpy(eq).cuda(), [1], 0.875, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0                          # equal is not exceeding


def test_repetition_chain_agrees_with_oracle():
    F, R, C, d, H, P = 2, 10, 20, 128, 3, 3
    N = F * R * C
    anchors = [2, 7]
    q, k = workloads.make_calibration_prompts(N, d, F, R, C, H, P, seed=9900)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    sims = torch.empty((P, H, F, R), dtype=torch.float32, device="cuda")
    want = np.empty((P, H, F, R))
    for p in range(P):
        cal.calibatt_spatial_similarity(to_device(q[p], "bf16"), to_device(k[p], "bf16"), F, R, C, anchors,
                                        sims[p], scale=scale)
        for h in range(H):
            want[p, h] = oracle.row_similarity(exact_values(q[p, h], "bf16"), exact_values(k[p, h], "bf16"), F, R, C,
                                               anchors, scale)
    mean = torch.empty((H,), dtype=torch.float32, device="cuda")
    flags = torch.empty((H,), dtype=torch.uint8, device="cuda")
    cal.calibatt_repetition_flags(sims, anchors, 0.87, flags=flags, mean=mean)
    torch.cuda.synchronize()
    want_mean = oracle.repetition_mean(want, anchors)
    np.testing.assert_allclose(mean.cpu().numpy(), want_mean, atol=TOL_SIM)
    for h in range(H):
        if abs(want_mean[h] - 0.87) > 1e-4:
            assert int(flags[h].item()) == int(want_mean[h] > 0.87)
