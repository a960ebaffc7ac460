"""How the attention kernels walk a query block's key blocks, at the edges: rows listing one, two or
three blocks, runs of one block, runs that end on the last block, the last block (nb - 1) at odd and at
even list positions, and rows whose blocks are all far apart or all adjacent. The three list forms must
give bitwise-equal output (same blocks, same order, same arithmetic) and O within tolerance of the
oracle."""
import numpy as np
import pytest
import torch

import oracle
import calibrated_block_sparse_skiplist_amd as cal
from _gpu_util import TOL_BF16, TOL_F32, alloc_out, exact_values, host64, max_abs, random_qkv, say, to_device

pytestmark = pytest.mark.gpu


def _edge_masks(nb, H, seed):
    rng = np.random.default_rng(seed)
    m = np.zeros((1, 1, H, nb, nb), dtype=np.uint8)
    rows = [
        [0],                                   # one block
        [nb - 1],                              # only the last block
        [0, nb - 1],                           # two runs of one, the last block at position 1
        [1, 2, nb - 1],                        # last block at position 2
        [nb - 3, nb - 2, nb - 1],              # one run ending on the last block
        list(range(0, nb, 2)),                 # every other block: runs of one
        list(range(nb)),                       # everything: one run
        list(range(1, nb, 3)),                 # far apart
        [],                                    # empty
    ]
    for h in range(H):
        for r in range(nb):
            pick = rows[(r + h) % len(rows)]
            if not pick:
                continue
            if (r + h) % 5 == 0:               # and some random rows
                pick = sorted(set(rng.choice(nb, size=rng.integers(1, nb + 1), replace=False).tolist()))
            m[0, 0, h, r, pick] = 1
    return m


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,d,B", [(1000, 128, 128), (700, 64, 64), (1500, 128, 128), (1300, 64, 128)])
def test_three_forms_walk_the_same_blocks(dtype, N, d, B):
    nb = -(-N // B)
    H = 3
    say(f"[walk] dtype={dtype} N={N} d={d} B={B} nb={nb}")
    masks = _edge_masks(nb, H, seed=N + d)
    dm = torch.from_numpy(masks).cuda()
    sl, il, bm = cal.compile_skiplist(dm, N, B), cal.compile_intervals(dm, N, B), cal.compile_bitmap(dm, N, B)
    q, k, v = random_qkv(H, N, d, dtype, seed=3 * N + d)
    qd, kd, vd = (to_device(x, dtype) for x in (q, k, v))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    outs = []
    for call, lst in ((cal.calibatt_block_sparse_attn, sl), (cal.calibatt_block_sparse_attn_iv, il),
                      (cal.calibatt_block_sparse_attn_bm, bm)):
        o, _ = alloc_out(H, N, d, dtype)
        call(qd, kd, vd, o, None, lst, 0, 0, scale=scale)
        outs.append(o)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(outs[0].view(bits), outs[1].view(bits)), "run form differs from the index form"
    assert torch.equal(outs[0].view(bits), outs[2].view(bits)), "bitmap form differs from the index form"
    rp, ci, _ = oracle.compile_skiplist(masks)
    og = host64(outs[0])
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for h in range(H):
        want, _ = oracle.block_sparse_head(exact_values(q[h], dtype), exact_values(k[h], dtype),
                                           exact_values(v[h], dtype), rp, ci, h, B, scale)
        assert max_abs(og[h], want) <= tol
