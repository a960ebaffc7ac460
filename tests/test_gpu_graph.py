"""The layer path captured in a HIP graph (torch.cuda.CUDAGraph over the library's stream launches):
the dispatch issues only kernel launches (no allocation, no memset, no host sync), and the bitmap
compile has no host sync either, so compile + dispatch can be captured once and replayed per layer.
Every replay is checked bitwise against the eager result, with eager work and synchronisations between
the replays; one test changes the masks in place between replays, so the replay recompiles from device
data."""
import numpy as np
import pytest
import torch

import workloads
import calibrated_block_sparse_skiplist_amd as cal
from _gpu_util import say

pytestmark = pytest.mark.gpu


def _inputs(key):
    wl = workloads.make_workload(key)
    cfg = wl.cfg
    up = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return wl, cfg, up(wl.q), up(wl.k), up(wl.v), torch.from_numpy(wl.masks).cuda()


def _bits16(t):
    return t.view(torch.int16)


def test_layer_dispatch_replays_bitwise():
    wl, cfg, q, k, v, masks = _inputs("wan480_dual")
    say(f"[graph] dispatch capture: {cfg.title}")
    sl = cal.compile_skiplist(masks, cfg.N, cfg.B)
    ref = torch.empty_like(q)
    cal.calibatt_layer_dispatch(q, k, v, ref, None, sl, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                scale=wl.scale)
    torch.cuda.synchronize()
    o = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cal.calibatt_layer_dispatch(q, k, v, o, None, sl, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                    scale=wl.scale)
    other = torch.empty_like(q)
    for r in range(3):
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits16(o), _bits16(ref)), f"replay {r}"
        # eager work between the replays, on the same stream
        cal.calibatt_layer_dispatch(q, k, v, other, None, sl, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C,
                                    wl.anchors, scale=wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(_bits16(other), _bits16(ref))


def test_bitmap_compile_and_dispatch_replay_on_new_masks():
    wl, cfg, q, k, v, masks = _inputs("wan480_sparse")
    say(f"[graph] bitmap compile + dispatch capture: {cfg.title}")
    bm = cal.compile_bitmap(masks, cfg.N, cfg.B)
    o = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cal.calibatt_compile_bitmap(masks, 1, 1, cfg.H, cfg.N, cfg.B, bm.bits)
        cal.calibatt_layer_dispatch_bm(q, k, v, o, None, bm, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C,
                                       wl.anchors, scale=wl.scale)
    rng = np.random.default_rng(91)
    original = masks.clone()
    for r in range(3):
        if r > 0:
            # new masks in place (eager): drop a random third of the kept blocks, keep the diagonal
            drop = torch.from_numpy(rng.random(tuple(masks.shape)) < 0.33).cuda()
            eye = torch.eye(cfg.nb, dtype=torch.bool, device="cuda")
            masks.copy_(torch.where(drop & ~eye, torch.zeros_like(original), original))
        torch.cuda.synchronize()
        sl = cal.compile_skiplist(masks, cfg.N, cfg.B)
        ref = torch.empty_like(q)
        cal.calibatt_layer_dispatch(q, k, v, ref, None, sl, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                    scale=wl.scale)
        torch.cuda.synchronize()
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits16(o), _bits16(ref)), f"replay {r}"
