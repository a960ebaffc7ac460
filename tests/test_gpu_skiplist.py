"""GPU skip-list compilation: bit-exact against the oracle (row_ptr, col_idx, order)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import calibrated_block_sparse_skiplist_amd as cal
from _gpu_util import say

pytestmark = pytest.mark.gpu


def _compile_and_compare(masks: np.ndarray, N: int, B: int, label: str):
    say(f"[skiplist] {label}: masks {masks.shape}")
    T, L, H, nb, _ = masks.shape
    dm = torch.from_numpy(np.ascontiguousarray(masks)).cuda()
    sl = cal.compile_skiplist(dm, N, B)
    torch.cuda.synchronize()
    rp, ci, order = oracle.compile_skiplist(masks)
    assert sl.nnz == int(rp[-1])
    np.testing.assert_array_equal(sl.row_ptr.cpu().numpy(), rp)
    np.testing.assert_array_equal(sl.col_idx.cpu().numpy()[:sl.nnz], ci)
    np.testing.assert_array_equal(sl.order.cpu().numpy(), order)
    return sl


@pytest.mark.parametrize("shape,p,seed", [
    ((1, 1, 1, 1), 1.0, 0), ((1, 1, 1, 1), 0.0, 1), ((1, 1, 2, 3), 0.5, 2), ((2, 3, 2, 7), 0.4, 3),
    ((1, 1, 3, 64), 0.3, 4), ((1, 1, 2, 65), 0.7, 5), ((1, 2, 5, 131), 0.2, 6), ((3, 1, 2, 300), 0.05, 7),
    ((1, 1, 1, 1030), 0.5, 8),
    # sparse rows: counts 0..~15, so most ranks are decided by the row index
    ((1, 1, 2, 591), 0.01, 10),
    # nb = CALIBATT_MAX_NB: 64 groups of 64 rows in the ranking
    ((1, 1, 1, 4096), 0.002, 11),
])
def test_random_masks(shape, p, seed):
    rng = np.random.default_rng(seed)
    T, L, H, nb = shape
    masks = (rng.random((T, L, H, nb, nb)) < p).astype(np.uint8)
    masks[masks == 1] = rng.integers(1, 256, size=int(masks.sum()), dtype=np.uint8)
    if nb > 2:
        masks[0, 0, 0, 1] = 0          # an empty row
        masks[0, 0, -1, -1] = 7        # a full row
    _compile_and_compare(masks, nb * 16, 16, f"random {shape} p={p}")


@pytest.mark.parametrize("offset", [1, 7, 13])
@pytest.mark.parametrize("nb", [33, 591, 1030])
def test_masks_not_16_byte_aligned(offset, nb):
    """The compile reads masks as 16-byte aligned chunks: masks starting at any byte address give the same lists."""
    rng = np.random.default_rng(offset * 1000 + nb)
    masks = (rng.random((1, 1, 2, nb, nb)) < 0.4).astype(np.uint8)
    buf = torch.zeros(masks.size + 64, dtype=torch.uint8, device="cuda")
    view = buf[offset:offset + masks.size]
    view.copy_(torch.from_numpy(masks.reshape(-1)).cuda())
    say(f"[skiplist] masks at byte offset {offset} (address % 16 = {view.data_ptr() % 16}), nb={nb}")
    sl = cal.compile_skiplist(view.view(masks.shape), nb * 16, 16)
    torch.cuda.synchronize()
    rp, ci, order = oracle.compile_skiplist(masks)
    assert sl.nnz == int(rp[-1])
    np.testing.assert_array_equal(sl.row_ptr.cpu().numpy(), rp)
    np.testing.assert_array_equal(sl.col_idx.cpu().numpy()[:sl.nnz], ci)
    np.testing.assert_array_equal(sl.order.cpu().numpy(), order)


def test_all_zero_dictionary_has_no_entries():
    masks = np.zeros((1, 2, 3, 40, 40), np.uint8)
    sl = _compile_and_compare(masks, 40 * 64, 64, "all zero")
    assert sl.nnz == 0


def test_many_segments_scan():
    # rows = 2*4*5*300 = 12000 > several scan segments of 1024 rows
    rng = np.random.default_rng(9)
    masks = (rng.random((2, 4, 5, 300, 300)) < 0.1).astype(np.uint8)
    _compile_and_compare(masks, 300 * 128 - 50, 128, "multi-segment")


@pytest.mark.parametrize("key", ["tiny", "wan480_sparse", "wan720"])
def test_config_masks(key):
    wl = workloads.make_workload(key, with_data=False)
    _compile_and_compare(wl.masks, wl.cfg.N, wl.cfg.B, key)


def test_dictionary_480p_68():
    cfg, masks, _ = workloads.make_dictionary_workload(0.68, 0.25, L=8, H=40)
    _compile_and_compare(masks, cfg.N, cfg.B, "480p dictionary, 8 layers")


def test_size_query_and_capacity_error():
    rng = np.random.default_rng(10)
    masks = (rng.random((1, 1, 2, 20, 20)) < 0.5).astype(np.uint8)
    dm = torch.from_numpy(masks).cuda()
    rp = torch.empty(2 * 20 + 1, dtype=torch.int64, device="cuda")
    nnz = cal.calibatt_compile_skiplist(dm, 1, 1, 2, 20 * 64, 64, rp, None, 0, None)
    assert nnz == int(masks.sum())
    small = torch.full((nnz - 1,), -5, dtype=torch.int32, device="cuda")
    with pytest.raises(cal.CalibattError) as ei:
        cal.calibatt_compile_skiplist(dm, 1, 1, 2, 20 * 64, 64, rp, small, small.numel(), None)
    assert ei.value.status == 2
    assert torch.all(small == -5)          # nothing written on CAPACITY
    want_rp, _, _ = oracle.compile_skiplist(masks)
    np.testing.assert_array_equal(rp.cpu().numpy(), want_rp)


def test_checked_mode_on_device_views():
    """Compiled device views validate; in checked mode a malformed record is rejected before any launch
    (the output stays untouched) and a valid one gives the same output as without checking. The
    malformed list only reorders valid key blocks, so even an unchecked launch would stay in bounds."""
    from _gpu_util import alloc_out, random_qkv, to_device
    H, N, d, B = 3, 1000, 128, 128
    nb = -(-N // B)
    rng = np.random.default_rng(41)
    masks = (rng.random((1, 2, H, nb, nb)) < 0.5).astype(np.uint8)
    for l in range(2):
        for h in range(H):
            np.fill_diagonal(masks[0, l, h], 1)
    dm = torch.from_numpy(masks).cuda()
    sl = cal.compile_skiplist(dm, N, B)
    il = cal.compile_intervals(dm, N, B)
    cal.calibatt_validate_skiplist(sl)
    cal.calibatt_validate_skiplist(sl, 0, 1)
    cal.calibatt_validate_intervals(il)
    cal.calibatt_validate_intervals(il, 0, 0)
    q, k, v = (to_device(x, "bf16") for x in random_qkv(H, N, d, "bf16", seed=42))
    o_ref, _ = alloc_out(H, N, d, "bf16")
    cal.calibatt_block_sparse_attn(q, k, v, o_ref, None, sl, 0, 1)
    # a descending pair of key blocks in a row of record (0, 1)
    rp = sl.row_ptr.cpu().numpy()
    lens = np.diff(rp)
    row = H * nb + int(np.flatnonzero(lens[H * nb:] >= 2)[0])
    bad_ci = sl.col_idx.clone()
    j = int(rp[row])
    bad_ci[j], bad_ci[j + 1] = sl.col_idx[j + 1].item(), sl.col_idx[j].item()
    bad = cal.SkipList(sl.T, sl.L, sl.H, sl.N, sl.B, sl.nb, sl.row_ptr, bad_ci, sl.order, sl.nnz)
    with pytest.raises(cal.CalibattError, match="ascending"):
        cal.calibatt_validate_skiplist(bad, 0, 1)
    cal.calibatt_validate_skiplist(bad, 0, 0)          # the other record is fine
    cal.calibatt_set_checked_mode(True)
    try:
        o, _ = alloc_out(H, N, d, "bf16")
        with pytest.raises(cal.CalibattError, match="ascending"):
            cal.calibatt_block_sparse_attn(q, k, v, o, None, bad, 0, 1)
        torch.cuda.synchronize()
        assert torch.isnan(o.float()).all(), "a rejected call wrote its output"
        o2, _ = alloc_out(H, N, d, "bf16")
        cal.calibatt_block_sparse_attn(q, k, v, o2, None, sl, 0, 1)
        torch.cuda.synchronize()
        assert torch.equal(o2.view(torch.int16), o_ref.view(torch.int16))
    finally:
        cal.calibatt_set_checked_mode(False)
