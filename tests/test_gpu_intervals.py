"""GPU interval skip lists: compile bit-exact against the oracle, and attention
over runs bitwise equal to attention over index lists (same blocks, same order,
same arithmetic) and within tolerance of the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import oracle.skiplist as osk
import workloads
import calibrated_block_sparse_skiplist_amd as cal
from _gpu_util import (TOL_BF16, TOL_F32, TOL_LSE_BF16, TOL_LSE_F32, alloc_out, exact_values, host64, max_abs,
                       random_qkv, say, to_device)

pytestmark = pytest.mark.gpu


def _packed(iv: np.ndarray) -> np.ndarray:
    return (iv[:, 0].astype(np.int64) | (iv[:, 1].astype(np.int64) << 16)).astype(np.uint32)


def _compile_and_compare(masks: np.ndarray, N: int, B: int, label: str):
    say(f"[intervals] {label}: masks {masks.shape}")
    il = cal.compile_intervals(torch.from_numpy(np.ascontiguousarray(masks)).cuda(), N, B)
    torch.cuda.synchronize()
    iv_ptr, iv, order = osk.compile_intervals(masks)
    assert il.n_iv == int(iv_ptr[-1])
    np.testing.assert_array_equal(il.iv_ptr.cpu().numpy(), iv_ptr)
    np.testing.assert_array_equal(il.iv.cpu().numpy().view(np.uint32)[:il.n_iv], _packed(iv))
    np.testing.assert_array_equal(il.order.cpu().numpy(), order)
    return il


def _random(shape, p, seed):
    rng = np.random.default_rng(seed)
    masks = (rng.random(shape) < p).astype(np.uint8)
    masks[masks == 1] = rng.integers(1, 256, size=int(masks.sum()), dtype=np.uint8)
    return masks


@pytest.mark.parametrize("shape,p,seed", [
    ((1, 1, 1, 1, 1), 1.0, 0), ((1, 1, 1, 1, 1), 0.0, 1), ((1, 1, 2, 3, 3), 0.5, 2), ((2, 3, 2, 7, 7), 0.4, 3),
    ((1, 1, 3, 64, 64), 0.5, 4), ((1, 1, 2, 65, 65), 0.7, 5), ((1, 2, 5, 131, 131), 0.2, 6),
    ((3, 1, 2, 300, 300), 0.9, 7), ((1, 1, 1, 1030, 1030), 0.5, 8),
])
def test_random_masks(shape, p, seed):
    masks = _random(shape, p, seed)
    nb = shape[-1]
    if nb > 2:
        masks[0, 0, 0, 1] = 0                 # an empty row
        masks[0, 0, -1, -1] = 7               # a full row: one run
        masks[0, 0, 0, 2] = 0
        masks[0, 0, 0, 2, ::2] = 3            # alternating: single-block runs
    _compile_and_compare(masks, nb * 16, 16, f"random {shape} p={p}")


def test_runs_across_64_block_windows():
    # runs that start, end or continue exactly at the 64-block window edges of the kernels
    nb = 200
    masks = np.zeros((1, 1, 1, nb, nb), np.uint8)
    for r, (lo, hi) in enumerate([(0, 64), (63, 65), (64, 128), (60, 70), (127, 129), (128, 200), (0, 200),
                                  (199, 200)]):
        masks[0, 0, 0, r, lo:hi] = 1
    il = _compile_and_compare(masks, nb * 64, 64, "window edges")
    assert il.n_iv == 8


def test_runs_across_1kb_windows():
    # the compile reads a row 1 KB (1024 blocks) per wave load; runs that start, end or continue at
    # those window edges, for rows starting at several alignments (nb odd)
    nb = 2101
    masks = np.zeros((1, 1, 1, nb, nb), np.uint8)
    spans = [(1000, 1100), (1023, 1025), (1024, 2048), (0, 2101), (2047, 2049), (5, 1024), (1024, 1025),
             (2100, 2101), (0, 1), (1020, 2060)]
    for r, (lo, hi) in enumerate(spans):
        masks[0, 0, 0, r, lo:hi] = 1
    masks[0, 0, 0, len(spans), ::2] = 5       # alternating across both window edges
    il = _compile_and_compare(masks, nb * 16, 16, "1 KB window edges")
    assert il.n_iv == len(spans) + (nb + 1) // 2


@pytest.mark.parametrize("offset", [1, 7, 13])
@pytest.mark.parametrize("nb", [33, 591, 1030])
def test_masks_not_16_byte_aligned(offset, nb):
    """Masks starting at any byte address give the same runs (the compile reads 16-byte aligned chunks)."""
    rng = np.random.default_rng(offset * 1000 + nb)
    masks = (rng.random((1, 1, 2, nb, nb)) < 0.6).astype(np.uint8)
    buf = torch.zeros(masks.size + 64, dtype=torch.uint8, device="cuda")
    view = buf[offset:offset + masks.size]
    view.copy_(torch.from_numpy(masks.reshape(-1)).cuda())
    say(f"[intervals] masks at byte offset {offset} (address % 16 = {view.data_ptr() % 16}), nb={nb}")
    il = cal.compile_intervals(view.view(masks.shape), nb * 16, 16)
    torch.cuda.synchronize()
    ptr, runs, order = oracle.compile_intervals(masks)
    assert il.n_iv == int(ptr[-1])
    np.testing.assert_array_equal(il.iv_ptr.cpu().numpy(), ptr)
    got = il.iv.cpu().numpy()[:il.n_iv].astype(np.int64)
    np.testing.assert_array_equal(np.stack([got & 0xffff, got >> 16], axis=1), runs)
    np.testing.assert_array_equal(il.order.cpu().numpy(), order)


def test_many_segments_scan():
    masks = _random((2, 4, 5, 300, 300), 0.3, 9)
    _compile_and_compare(masks, 300 * 128 - 50, 128, "multi-segment")


@pytest.mark.parametrize("key", ["tiny", "wan480_sparse", "wan720"])
def test_config_masks(key):
    wl = workloads.make_workload(key, with_data=False)
    il = _compile_and_compare(wl.masks, wl.cfg.N, wl.cfg.B, key)
    rp, _, _ = oracle.compile_skiplist(wl.masks)
    say(f"[intervals] {key}: {il.n_iv} runs for {int(rp[-1])} kept blocks")


def test_size_query_and_capacity_error():
    masks = _random((1, 1, 2, 20, 20), 0.5, 10)
    dm = torch.from_numpy(masks).cuda()
    ptr = torch.empty(2 * 20 + 1, dtype=torch.int64, device="cuda")
    n_iv = cal.calibatt_compile_intervals(dm, 1, 1, 2, 20 * 64, 64, ptr, None, 0, None)
    want_ptr, _, _ = osk.compile_intervals(masks)
    assert n_iv == int(want_ptr[-1])
    np.testing.assert_array_equal(ptr.cpu().numpy(), want_ptr)
    small = torch.full((n_iv - 1,), -5, dtype=torch.int32, device="cuda")
    with pytest.raises(cal.CalibattError) as ei:
        cal.calibatt_compile_intervals(dm, 1, 1, 2, 20 * 64, 64, ptr, small, small.numel(), None)
    assert ei.value.status == 2
    assert torch.all(small == -5)          # nothing written on CAPACITY


def _tols(dtype):
    return (TOL_BF16, TOL_LSE_BF16) if dtype == "bf16" else (TOL_F32, TOL_LSE_F32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,d,B,p", [(1000, 128, 128, 0.5), (1000, 64, 128, 0.8), (700, 128, 64, 0.3),
                                     (700, 64, 64, 0.6), (77, 128, 128, 1.0), (3000, 128, 128, 0.5)])
def test_attention_over_runs(dtype, N, d, B, p):
    say(f"[intervals] attention dtype={dtype} N={N} d={d} B={B} p={p}")
    H = 3
    nb = -(-N // B)
    rng = np.random.default_rng(N + d + B)
    masks = (rng.random((1, 1, H, nb, nb)) < p)
    for h in range(H):
        np.fill_diagonal(masks[0, 0, h], True)
    if nb > 1:
        masks[0, 0, 1, nb // 2] = False       # an empty row
    masks = masks.astype(np.uint8)
    q, k, v = random_qkv(H, N, d, dtype, seed=7 * N + d)
    dq, dk, dv = (to_device(x, dtype) for x in (q, k, v))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    dm = torch.from_numpy(masks).cuda()
    il = cal.compile_intervals(dm, N, B)
    sl = cal.compile_skiplist(dm, N, B)
    o_iv, l_iv = alloc_out(H, N, d, dtype)
    o_cs, l_cs = alloc_out(H, N, d, dtype)
    cal.calibatt_block_sparse_attn_iv(dq, dk, dv, o_iv, l_iv, il, 0, 0, scale=scale)
    cal.calibatt_block_sparse_attn(dq, dk, dv, o_cs, l_cs, sl, 0, 0, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o_iv.view(torch.int16 if dtype == "bf16" else torch.int32),
                       o_cs.view(torch.int16 if dtype == "bf16" else torch.int32))
    assert torch.equal(l_iv.view(torch.int32), l_cs.view(torch.int32))
    rp, ci, _ = oracle.compile_skiplist(masks)
    tol, tol_lse = _tols(dtype)
    og, lg = host64(o_iv), l_iv.cpu().numpy()
    for h in range(H):
        want_o, want_l = oracle.block_sparse_head(exact_values(q[h], dtype), exact_values(k[h], dtype),
                                                  exact_values(v[h], dtype), rp, ci, h, B, scale)
        assert max_abs(og[h], want_o) <= tol, (h, max_abs(og[h], want_o))
        assert max_abs(lg[h], want_l) <= tol_lse


@pytest.mark.parametrize("key", ["wan480_dual", "wan720"])
def test_layer_dispatch_over_runs_matches_index_lists(key):
    say(f"[intervals] layer dispatch {key}")
    wl = workloads.make_workload(key)
    cfg = wl.cfg
    dq, dk, dv = (to_device(x, "bf16") for x in (wl.q, wl.k, wl.v))
    dm = torch.from_numpy(wl.masks).cuda()
    il = cal.compile_intervals(dm, cfg.N, cfg.B)
    sl = cal.compile_skiplist(dm, cfg.N, cfg.B)
    o_iv, l_iv = alloc_out(cfg.H, cfg.N, cfg.d, "bf16")
    o_cs, l_cs = alloc_out(cfg.H, cfg.N, cfg.d, "bf16")
    cal.calibatt_layer_dispatch_iv(dq, dk, dv, o_iv, l_iv, il, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                   scale=wl.scale)
    cal.calibatt_layer_dispatch(dq, dk, dv, o_cs, l_cs, sl, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(o_iv.view(torch.int16), o_cs.view(torch.int16))
    assert torch.equal(l_iv.view(torch.int32), l_cs.view(torch.int32))
    # sampled oracle check of two query blocks of the first block-sparse head
    h = int(np.flatnonzero(wl.rep_flags[0, 0] == 0)[0])
    rp, ci, _ = oracle.compile_skiplist(wl.masks)
    blocks = [0, cfg.nb - 1]
    want_o, _ = oracle.block_sparse_head(exact_values(wl.q[h], "bf16"), exact_values(wl.k[h], "bf16"),
                                         exact_values(wl.v[h], "bf16"), rp, ci, h, cfg.B, wl.scale, blocks=blocks)
    og = host64(o_iv[h])
    for b in blocks:
        lo, hi = b * cfg.B, min((b + 1) * cfg.B, cfg.N)
        assert max_abs(og[lo:hi], want_o[lo:hi]) <= TOL_BF16


@pytest.mark.parametrize("B,d", [(128, 128), (64, 64)])
def test_maximum_size_lists(B, d):
    """nb = CALIBATT_MAX_NB = 4096 blocks: a full row (the longest list the kernels stage), an alternating
    row (the most runs, nb/2), first-and-last blocks, and an empty head; both list forms."""
    nb = 4096                                   # CALIBATT_MAX_NB
    N = nb * B - B // 2                         # ragged last block
    H = 2
    say(f"[max size] nb={nb} N={N} B={B} d={d}")
    masks = np.zeros((1, 1, H, nb, nb), np.uint8)
    masks[0, 0, 0, 0, :] = 1                    # every key block
    masks[0, 0, 0, 1, ::2] = 1                  # 2048 single-block runs
    masks[0, 0, 0, nb - 1, [0, nb - 1]] = 1     # first and last block (ragged)
    # head 1: every list empty
    q, k, v = random_qkv(H, N, d, "bf16", seed=nb + B)
    dq, dk, dv = (to_device(x, "bf16") for x in (q, k, v))
    dm = torch.from_numpy(masks).cuda()
    sl = cal.compile_skiplist(dm, N, B)
    il = cal.compile_intervals(dm, N, B)
    o, lse = alloc_out(H, N, d, "bf16")
    o_iv, lse_iv = alloc_out(H, N, d, "bf16")
    scale = float(np.float32(1.0 / np.sqrt(d)))
    cal.calibatt_block_sparse_attn(dq, dk, dv, o, lse, sl, 0, 0, scale=scale)
    cal.calibatt_block_sparse_attn_iv(dq, dk, dv, o_iv, lse_iv, il, 0, 0, scale=scale)
    torch.cuda.synchronize()
    assert il.n_iv == 1 + nb // 2 + 2
    assert torch.equal(o.view(torch.int16), o_iv.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse_iv.view(torch.int32))
    rp, ci, _ = oracle.compile_skiplist(masks)
    blocks = [0, 1, nb - 1]
    want_o, want_l = oracle.block_sparse_head(exact_values(q[0], "bf16"), exact_values(k[0], "bf16"),
                                              exact_values(v[0], "bf16"), rp, ci, 0, B, scale, blocks=blocks)
    og, lg = host64(o[0]), lse[0].cpu().numpy()
    for b in blocks:
        lo, hi = b * B, min((b + 1) * B, N)
        assert max_abs(og[lo:hi], want_o[lo:hi]) <= TOL_BF16, b
        assert max_abs(lg[lo:hi], want_l[lo:hi]) <= TOL_LSE_BF16, b
    # the empty head: O = 0 and lse = -inf everywhere
    assert torch.all(o[1] == 0)
    assert torch.all(torch.isneginf(lse[1]))
