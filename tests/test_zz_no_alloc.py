"""calibatt_block_energy_noalloc (the entry point for callers that cannot allocate device memory) against
calibatt_block_energy with a caller workspace, through the C ABI: bitwise-equal energies, and within the
energy tolerance (2e-5) of the fp64 oracle on shapes the oracle finishes quickly. Two calls in a row, the
second smaller, share the scratch; a shape with more query blocks than the scratch holds runs in several
launches and must still match."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import calibrated_block_sparse_skiplist_amd as cal
from calibrated_block_sparse_skiplist_amd import _lib
from _gpu_util import exact_values, say, to_device

pytestmark = pytest.mark.gpu

TOL_E = 2e-5


def _prompt(N, d, H, dtype, seed, geom):
    F, R, C = geom
    q, k = workloads.make_calibration_prompts(N, d, F, R, C, H, 1, dtype=dtype, seed=seed)
    return q[0], k[0]


def _both(q, k, B, dtype, heads=None):
    """Energies from the no-alloc entry point and from the workspace entry point (same inputs)."""
    H, N, d = q.shape
    nb = -(-N // B)
    qd, kd = to_device(q, dtype), to_device(k, dtype)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    e_na = torch.full((H, nb, nb), float("nan"), dtype=torch.float32, device="cuda")
    e_ws = torch.full((H, nb, nb), float("nan"), dtype=torch.float32, device="cuda")
    n_listed = H if heads is None else len(heads)
    work = torch.empty((cal.energy_work_bytes(N, B, n_listed) // 4,), dtype=torch.float32, device="cuda")
    cal.calibatt_block_energy_noalloc(qd, kd, e_na, B, heads=heads, scale=scale)
    cal.calibatt_block_energy(qd, kd, e_ws, B, heads=heads, scale=scale, work=work if dtype == "bf16" else None)
    torch.cuda.synchronize()
    return e_na.cpu().numpy(), e_ws.cpu().numpy(), scale


def _check_oracle(e, q, k, B, dtype, scale, heads):
    for h in heads:
        want = oracle.block_energy(exact_values(q[h], dtype), exact_values(k[h], dtype), B, scale)
        err = float(np.max(np.abs(e[h].astype(np.float64) - want)))
        say(f"  head {h}: max|dE| = {err:.2e}")
        assert err <= TOL_E, (h, err)


def test_two_calls_in_a_row_second_smaller():
    # first call: 3 heads, N = 1500, d = 128, B = 128
    say("[noalloc] call 1: H=3 N=1500 d=128 B=128 bf16")
    q, k = _prompt(1500, 128, 3, "bf16", 7100, (5, 10, 30))
    e_na, e_ws, scale = _both(q, k, 128, "bf16")
    assert np.array_equal(e_na.view(np.uint32), e_ws.view(np.uint32)), "call 1 differs from the workspace call"
    _check_oracle(e_na, q, k, 128, "bf16", scale, range(3))
    # second call, smaller: 2 of 2 heads, N = 500, d = 64, B = 64 (the scratch keeps call 1's contents)
    say("[noalloc] call 2: H=2 N=500 d=64 B=64 bf16")
    q2, k2 = _prompt(500, 64, 2, "bf16", 7200, (5, 10, 10))
    e_na2, e_ws2, scale2 = _both(q2, k2, 64, "bf16")
    assert np.array_equal(e_na2.view(np.uint32), e_ws2.view(np.uint32)), "call 2 differs from the workspace call"
    _check_oracle(e_na2, q2, k2, 64, "bf16", scale2, range(2))


def test_head_subset_and_fp32():
    say("[noalloc] head subset [2, 0] of 3, N=700 d=128 B=64 bf16")
    q, k = _prompt(700, 128, 3, "bf16", 7300, (7, 10, 10))
    e_na, e_ws, scale = _both(q, k, 64, "bf16", heads=[2, 0])
    assert np.array_equal(e_na[[0, 2]].view(np.uint32), e_ws[[0, 2]].view(np.uint32))
    assert np.isnan(e_na[1]).all(), "an unlisted head was written"
    _check_oracle(e_na, q, k, 64, "bf16", scale, [0, 2])
    say("[noalloc] fp32 H=2 N=300 d=64 B=64 (no workspace needed)")
    q, k = _prompt(300, 64, 2, "f32", 7400, (3, 10, 10))
    e_na, e_ws, scale = _both(q, k, 64, "f32")
    assert np.array_equal(e_na.view(np.uint32), e_ws.view(np.uint32))
    _check_oracle(e_na, q, k, 64, "f32", scale, range(2))


def test_more_query_blocks_than_the_scratch_holds():
    # Wan-720p head shape: a query block's workspace is 591 * 128 floats, so the scratch holds 887 of the
    # 2 * 591 query blocks and the call runs in two launches; the energies match the workspace call bitwise.
    N, d, B, H = 75600, 128, 128, 2
    nb = -(-N // B)
    per_item = nb * B * 4
    assert H * nb > _lib.NOALLOC_SCRATCH_BYTES // per_item
    say(f"[noalloc] H={H} N={N} d={d} B={B}: {H * nb} query blocks, {_lib.NOALLOC_SCRATCH_BYTES // per_item} per launch")
    q, k = _prompt(N, d, H, "bf16", 7500, (21, 45, 80))
    e_na, e_ws, scale = _both(q, k, B, "bf16")
    assert np.array_equal(e_na.view(np.uint32), e_ws.view(np.uint32)), "chunked launches differ"
    np.testing.assert_allclose(e_na.sum(axis=2), 1.0, atol=TOL_E)
    # sampled rows against the oracle (it evaluates query blocks one by one)
    rows = [0, 300, nb - 1]
    for h in range(H):
        want = oracle.block_energy(workloads.bf16_to_f32(q[h]), workloads.bf16_to_f32(k[h]), B, scale, blocks=rows)
        err = float(np.max(np.abs(e_na[h, rows].astype(np.float64) - want[rows])))
        say(f"  head {h} rows {rows}: max|dE| = {err:.2e}")
        assert err <= TOL_E


def test_rejects_bad_arguments_before_launch():
    q = torch.zeros((2, 256, 128), dtype=torch.bfloat16, device="cuda")
    e = torch.full((2, 2, 2), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(cal.CalibattError, match="out of range"):
        cal.calibatt_block_energy_noalloc(q, q, e, 128, heads=[0, 5])
    with pytest.raises(cal.CalibattError, match="block size"):
        cal.calibatt_block_energy_noalloc(q, q, e, 96)
    torch.cuda.synchronize()
    assert torch.isnan(e).all()
