"""A full denoising-run dictionary resident on the GPU: T = 50 timesteps x
L = 40 layers x H = 40 heads at the 480p shape (5.2 GB of masks, about 2e9 kept
blocks, so list offsets pass 2^31). The three forms (index lists, runs,
bitmaps) are compiled in one call each; sampled records are bit-exact against
the oracle's compile of the same mask records, and layer calls at the first, a
middle and the last (t, l) agree with the oracle on sampled query blocks and
anchor frames, bitwise equal across the forms."""
import numpy as np
import pytest
import torch

import oracle
import oracle.skiplist as osk
import workloads
import calibrated_block_sparse_skiplist_amd as cal
from _gpu_util import TOL_BF16, exact_values, host64, say, to_device

pytestmark = pytest.mark.gpu

T, L, H = 50, 40, 40


@pytest.fixture(scope="module")
def dictionary():
    say(f"[dictionary] generating {T}x{L}x{H} masks at 480p on the GPU")
    cfg, masks, flags = workloads.make_step_dictionary("wan480_sparse", T, L, H, "cuda")
    sl = cal.compile_skiplist(masks, cfg.N, cfg.B)
    il = cal.compile_intervals(masks, cfg.N, cfg.B)
    bm = cal.compile_bitmap(masks, cfg.N, cfg.B)
    torch.cuda.synchronize()
    say(f"[dictionary] kept blocks {sl.nnz}, runs {il.n_iv}, bitmap words {bm.bits.numel()}")
    yield cfg, masks, flags, sl, il, bm
    del masks, sl, il, bm
    torch.cuda.empty_cache()


def _records():
    rng = np.random.default_rng(12)
    recs = [(0, 0, 0), (T - 1, L - 1, H - 1), (25, 17, 3)]
    recs += [tuple(int(x) for x in (rng.integers(T), rng.integers(L), rng.integers(H))) for _ in range(12)]
    return recs


def test_kept_count_matches_masks(dictionary):
    cfg, masks, flags, sl, il, bm = dictionary
    assert sl.nnz == int(torch.count_nonzero(masks).item())
    assert sl.nnz > 2 ** 31                          # offsets beyond 32 bits are exercised
    assert int(sl.row_ptr[-1].item()) == sl.nnz and int(il.iv_ptr[-1].item()) == il.n_iv


@pytest.mark.parametrize("rec", _records())
def test_sampled_records_bit_exact(dictionary, rec):
    cfg, masks, flags, sl, il, bm = dictionary
    t, l, h = rec
    nb = cfg.nb
    m = masks[t, l, h].cpu().numpy()[None, None, None]
    rid = (t * L + l) * H + h
    rp, ci, order = oracle.compile_skiplist(m)
    base = int(sl.row_ptr[rid * nb].item())
    got_rp = sl.row_ptr[rid * nb:(rid + 1) * nb + 1].cpu().numpy() - base
    np.testing.assert_array_equal(got_rp, rp)
    np.testing.assert_array_equal(sl.col_idx[base:base + int(rp[-1])].cpu().numpy(), ci)
    np.testing.assert_array_equal(sl.order[rid * nb:(rid + 1) * nb].cpu().numpy(), order)
    ip, iv, _ = osk.compile_intervals(m)
    ibase = int(il.iv_ptr[rid * nb].item())
    np.testing.assert_array_equal(il.iv_ptr[rid * nb:(rid + 1) * nb + 1].cpu().numpy() - ibase, ip)
    packed = (iv[:, 0].astype(np.int64) | (iv[:, 1].astype(np.int64) << 16)).astype(np.uint32)
    np.testing.assert_array_equal(il.iv[ibase:ibase + int(ip[-1])].cpu().numpy().view(np.uint32), packed)
    np.testing.assert_array_equal(bm.bits[rid * nb:(rid + 1) * nb].cpu().numpy().view(np.uint64),
                                  oracle.compile_bitmap(m))


@pytest.mark.parametrize("tl", [(0, 0), (25, 17), (T - 1, L - 1)])
def test_layer_calls_across_the_run(dictionary, tl):
    cfg, masks, flags, sl, il, bm = dictionary
    t, l = tl
    say(f"[dictionary] layer call t={t} l={l}")
    wl = workloads.make_workload("wan480_dual")
    dq, dk, dv = (to_device(x, "bf16") for x in (wl.q, wl.k, wl.v))
    o = torch.full((cfg.H, cfg.N, cfg.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    o_iv = torch.full_like(o, float("nan"))
    o_bm = torch.full_like(o, float("nan"))
    anchors = wl.anchors
    cal.calibatt_layer_dispatch(dq, dk, dv, o, None, sl, t, l, flags, cfg.F, cfg.R, cfg.C, anchors, scale=wl.scale)
    cal.calibatt_layer_dispatch_iv(dq, dk, dv, o_iv, None, il, t, l, flags, cfg.F, cfg.R, cfg.C, anchors,
                                   scale=wl.scale)
    cal.calibatt_layer_dispatch_bm(dq, dk, dv, o_bm, None, bm, t, l, flags, cfg.F, cfg.R, cfg.C, anchors,
                                   scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_iv.view(torch.int16))
    assert torch.equal(o.view(torch.int16), o_bm.view(torch.int16))
    sparse = [h for h in range(H) if not flags[t, l, h]]
    rep = [h for h in range(H) if flags[t, l, h]]
    h = sparse[len(sparse) // 2]
    m = masks[t, l, h].cpu().numpy()[None, None, None]
    rp, ci, _ = oracle.compile_skiplist(m)
    blocks = [0, cfg.nb // 2, cfg.nb - 1]
    want, _ = oracle.block_sparse_head(exact_values(wl.q[h], "bf16"), exact_values(wl.k[h], "bf16"),
                                       exact_values(wl.v[h], "bf16"), rp, ci, 0, cfg.B, wl.scale, blocks=blocks)
    og = host64(o[h])
    for b in blocks:
        lo, hi = b * cfg.B, min((b + 1) * cfg.B, cfg.N)
        assert float(np.max(np.abs(og[lo:hi] - want[lo:hi]))) <= TOL_BF16
    hr = rep[0]
    want_a, _ = oracle.anchor_head(exact_values(wl.q[hr], "bf16"), exact_values(wl.k[hr], "bf16"),
                                   exact_values(wl.v[hr], "bf16"), cfg.F, cfg.R, cfg.C, anchors, wl.scale, frames=[t % cfg.F])
    f = t % cfg.F
    lo, hi = f * cfg.R * cfg.C, (f + 1) * cfg.R * cfg.C
    assert float(np.max(np.abs(host64(o[hr])[lo:hi] - want_a[lo:hi]))) <= TOL_BF16
