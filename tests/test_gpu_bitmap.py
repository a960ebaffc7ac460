"""GPU bitmap form of the dictionary: compile bit-exact against the oracle's packing, attention over bitmaps
bitwise equal to the index-list form (same blocks, same order, same arithmetic) and within tolerance of the
fp64 oracle, padding bits ignored by the kernels and rejected by the validator."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import calibrated_block_sparse_skiplist_amd as cal
from _gpu_util import TOL_BF16, TOL_F32, alloc_out, exact_values, host64, max_abs, random_qkv, say, to_device

pytestmark = pytest.mark.gpu


def _bits_np(bm):
    return bm.bits.cpu().numpy().view(np.uint64)


@pytest.mark.parametrize("shape,p,seed", [
    ((1, 1, 1, 1), 1.0, 0), ((1, 1, 2, 3), 0.5, 1), ((2, 3, 2, 7), 0.4, 2), ((1, 1, 3, 63), 0.3, 3),
    ((1, 1, 2, 64), 0.7, 4), ((1, 2, 2, 65), 0.2, 5), ((1, 1, 2, 591), 0.3, 6), ((1, 1, 1, 1030), 0.5, 7),
    ((1, 1, 1, 4096), 0.01, 8),
])
def test_compile_matches_oracle(shape, p, seed):
    rng = np.random.default_rng(seed)
    T, L, H, nb = shape
    masks = (rng.random((T, L, H, nb, nb)) < p).astype(np.uint8)
    masks[masks != 0] = rng.integers(1, 256, size=int((masks != 0).sum()))   # any nonzero byte keeps
    say(f"[bitmap] compile {shape} p={p}")
    bm = cal.compile_bitmap(torch.from_numpy(masks).cuda(), nb * 8, 8)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits_np(bm), oracle.compile_bitmap(masks))
    cal.calibatt_validate_bitmap(bm)


@pytest.mark.parametrize("nb,shift", [(591, 1), (591, 7), (1030, 15), (64, 9), (5, 3)])
def test_compile_unaligned_masks(nb, shift):
    """Masks that start off a 16-byte boundary (a view into a larger buffer): the kernel's chunk alignment
    moves with the base address."""
    rng = np.random.default_rng(nb + shift)
    T, L, H = 1, 2, 3
    masks = (rng.random((T, L, H, nb, nb)) < 0.4).astype(np.uint8)
    buf = torch.full((masks.size + 32,), 255, dtype=torch.uint8, device="cuda")
    view = buf[shift:shift + masks.size].view(T, L, H, nb, nb)
    view.copy_(torch.from_numpy(masks).cuda())
    assert view.data_ptr() % 16 == shift % 16
    say(f"[bitmap] compile unaligned nb={nb} shift={shift}")
    bm = cal.compile_bitmap(view, nb * 8, 8)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits_np(bm), oracle.compile_bitmap(masks))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,d,B", [(1000, 128, 128), (700, 64, 64), (1500, 64, 128), (300, 128, 64)])
@pytest.mark.parametrize("with_lse", [True, False])
def test_attention_equals_index_form(dtype, N, d, B, with_lse):
    say(f"[bitmap] attention dtype={dtype} N={N} d={d} B={B} lse={with_lse}")
    H = 3
    nb = -(-N // B)
    rng = np.random.default_rng(N + d + B)
    masks = (rng.random((1, 1, H, nb, nb)) < 0.35).astype(np.uint8)
    for h in range(H):
        np.fill_diagonal(masks[0, 0, h], 1)
    masks[0, 0, 1, nb // 2] = 0                                 # an empty row
    dm = torch.from_numpy(masks).cuda()
    sl, bm = cal.compile_skiplist(dm, N, B), cal.compile_bitmap(dm, N, B)
    q, k, v = random_qkv(H, N, d, dtype, seed=7 * N + d)
    qd, kd, vd = (to_device(x, dtype) for x in (q, k, v))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o1, l1 = alloc_out(H, N, d, dtype)
    o2, l2 = alloc_out(H, N, d, dtype)
    cal.calibatt_block_sparse_attn(qd, kd, vd, o1, l1 if with_lse else None, sl, 0, 0, scale=scale)
    cal.calibatt_block_sparse_attn_bm(qd, kd, vd, o2, l2 if with_lse else None, bm, 0, 0, scale=scale)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(o1.view(bits), o2.view(bits)), "bitmap form differs from the index-list form"
    if with_lse:
        assert torch.equal(l1, l2)
    rp, ci, _ = oracle.compile_skiplist(masks)
    og = host64(o2)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for h in range(H):
        want, _ = oracle.block_sparse_head(exact_values(q[h], dtype), exact_values(k[h], dtype),
                                           exact_values(v[h], dtype), rp, ci, h, B, scale)
        assert max_abs(og[h], want) <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dispatch_by_record(dtype):
    T, L, H, F, R, C, d, B = 2, 3, 3, 2, 8, 32, 64, 64
    N = F * R * C
    nb = -(-N // B)
    rng = np.random.default_rng(51)
    masks = (rng.random((T, L, H, nb, nb)) < 0.3).astype(np.uint8)
    flags = (rng.random((T, L, H)) < 0.4).astype(np.uint8)
    flags[0, 1] = [0, 0, 0]
    anchors = [1, 5]
    dm = torch.from_numpy(masks).cuda()
    sl, bm = cal.compile_skiplist(dm, N, B), cal.compile_bitmap(dm, N, B)
    q, k, v = random_qkv(H, N, d, dtype, seed=52)
    qd, kd, vd = (to_device(x, dtype) for x in (q, k, v))
    bits = torch.int16 if dtype == "bf16" else torch.int32
    for t in range(T):
        for l in range(L):
            say(f"[bitmap] dispatch {dtype} record t={t} l={l}")
            o1, l1 = alloc_out(H, N, d, dtype)
            o2, l2 = alloc_out(H, N, d, dtype)
            cal.calibatt_layer_dispatch(qd, kd, vd, o1, l1, sl, t, l, flags, F, R, C, anchors)
            cal.calibatt_layer_dispatch_bm(qd, kd, vd, o2, l2, bm, t, l, flags, F, R, C, anchors)
            torch.cuda.synchronize()
            assert torch.equal(o1.view(bits), o2.view(bits)) and torch.equal(l1, l2)


def test_full_wan720_layer_equals_index_form():
    # the benchmark's launch (O only) through both forms of the same masks
    wl = workloads.make_workload("wan720")
    cfg = wl.cfg
    say(f"[bitmap] {cfg.title}")
    dm = torch.from_numpy(wl.masks).cuda()
    sl, bm = cal.compile_skiplist(dm, cfg.N, cfg.B), cal.compile_bitmap(dm, cfg.N, cfg.B)
    q, k, v = (to_device(x, "bf16") for x in (wl.q, wl.k, wl.v))
    o1, _ = alloc_out(cfg.H, cfg.N, cfg.d, "bf16")
    o2, _ = alloc_out(cfg.H, cfg.N, cfg.d, "bf16")
    cal.calibatt_layer_dispatch(q, k, v, o1, None, sl, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                scale=wl.scale)
    cal.calibatt_layer_dispatch_bm(q, k, v, o2, None, bm, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                   scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    np.testing.assert_array_equal(_bits_np(bm), oracle.compile_bitmap(wl.masks))


def test_padding_bits_ignored_and_rejected():
    H, N, d, B = 2, 1000, 128, 128     # nb = 8: bits 8..63 of each row are padding
    nb = -(-N // B)
    rng = np.random.default_rng(61)
    masks = (rng.random((1, 1, H, nb, nb)) < 0.5).astype(np.uint8)
    dm = torch.from_numpy(masks).cuda()
    bm = cal.compile_bitmap(dm, N, B)
    dirty = cal.Bitmap(bm.T, bm.L, bm.H, bm.N, bm.B, bm.nb, bm.words, bm.bits.clone())
    dirty.bits[:, 0] |= torch.tensor(-256, dtype=torch.int64, device="cuda")   # every padding bit set
    with pytest.raises(cal.CalibattError, match="past nb"):
        cal.calibatt_validate_bitmap(dirty)
    q, k, v = (to_device(x, "bf16") for x in random_qkv(H, N, d, "bf16", seed=62))
    o1, _ = alloc_out(H, N, d, "bf16")
    o2, _ = alloc_out(H, N, d, "bf16")
    cal.calibatt_block_sparse_attn_bm(q, k, v, o1, None, bm, 0, 0)
    cal.calibatt_block_sparse_attn_bm(q, k, v, o2, None, dirty, 0, 0)    # the kernels drop bits past nb
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    cal.calibatt_set_checked_mode(True)
    try:
        o3, _ = alloc_out(H, N, d, "bf16")
        with pytest.raises(cal.CalibattError, match="past nb"):
            cal.calibatt_block_sparse_attn_bm(q, k, v, o3, None, dirty, 0, 0)
        torch.cuda.synchronize()
        assert torch.isnan(o3.float()).all()
    finally:
        cal.calibatt_set_checked_mode(False)
