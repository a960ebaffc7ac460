"""Benchmark of the CalibAtt layer hot path on one MI355X.

One step = one pass of the whole hot path over one synthetic layer held in HBM:
skip-list compilation of the layer's block masks (calibatt_compile_skiplist)
followed by the per-head dual-path layer-call (calibatt_layer_dispatch: one
attention launch covering block-sparse and anchor-row heads, then the anchor
broadcast). W untimed warmup steps, then K timed steps bracketed by
torch.cuda.synchronize(). The same layer is also timed through the interval
form of the skip list (calibatt_compile_intervals + calibatt_layer_dispatch_iv),
reported under "intervals".

Default workload: a Wan-720p-shaped layer (H=40, N=75600 = 21x45x80 tokens,
d=128, 128x128 blocks, bf16), 32 block-sparse heads at 68% mean sparsity
(40-90% per head) and 8 repetitive heads with 5 anchor rows of 45.

Printed: one JSON line with the metric (retained-block TFLOP/s), ms per step,
the roofline of the dominant kernel (the attention kernel, timed per launch
with HIP events on its stream), the same kernel run dense over all heads, and
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0
ATTN_KERNEL = "attn_bf16_kernel"
# Sources the bf16 attention kernel is compiled from (its own file and the headers it includes).
# the kernel and its launch (api.hip fixes the grid's mapping to XCDs, which moves the counters too)
ATTN_SOURCES = [os.path.join(ROOT, "calibrated_block_sparse_skiplist_amd", "csrc", f)
                for f in ("attn_bf16.hip", "gfx950_device.h", "internal.h", "api.hip")]


def attn_source_sha() -> str:
    """sha256 over the attention kernel's sources, in order: the key that ties a counter profile to a build."""
    h = hashlib.sha256()
    for path in ATTN_SOURCES:
        h.update(open(path, "rb").read())
    return h.hexdigest()


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--protocol-reps", type=int, default=30,
                    help="layer calls timed one by one, warm and cache-flushed (0: skip)")
    ap.add_argument("--config", default="wan720",
                    choices=["tiny", "wan480_sparse", "wan480_dual", "wan720"])
    ap.add_argument("--dense-reps", type=int, default=3, help="launches of the dense comparator")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="time budget of each CPU oracle worker (the baseline's bounded sample)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates HBM byte counters)")
    ap.add_argument("--dictionary-sweep", action="store_true",
                    help="480p 40x40 dictionary: compile time and per-layer time over sparsity x "
                         "repetitive fraction (one JSON line per point)")
    ap.add_argument("--sweep-layers", type=int, default=4, help="layers timed per sweep point")
    ap.add_argument("--calibration", action="store_true",
                    help="offline calibration at the Wan-720p shape: block energies of one prompt (all 40 heads), "
                         "top-tau selection, keep frequency (one JSON line)")
    ap.add_argument("--prompts", type=int, default=3, help="calibration prompts timed")
    ap.add_argument("--dictionary-run", action="store_true",
                    help="a whole denoising run's dictionary at the Wan-720p shape (50 timesteps x 40 layers x "
                         "40 heads) resident on the GPU: compile both list forms, account memory, and stream "
                         "layer calls through sampled timesteps (one JSON line)")
    ap.add_argument("--run-steps", default="0,25,49", help="timesteps whose 40 layer calls are timed")
    ap.add_argument("--profile", choices=["layer", "sweep"],
                    help="a short fixed workload for rocprofv3 passes (no timing printed): 'layer' = the 720p "
                         "skip-list compile x3, layer-call x3 (O only) and the same kernel dense over 8 heads x3; "
                         "'sweep' = layer 0 of the 480p dictionary at sparsity 0, 0.68 and 0.85, x3 each")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="skip the 480p layers and the sweep summary in the default run")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work (what the method must compute; exp and softmax not counted)
# ---------------------------------------------------------------------------
def block_sizes(N, B):
    nb = -(-N // B)
    s = np.full(nb, B, dtype=np.int64)
    s[-1] = N - (nb - 1) * B
    return s


def sparse_head_flops(mask: np.ndarray, N: int, B: int, d: int) -> float:
    """4 d sum over kept (r, c) of |I_r| |J_c|  (QK^T and PV, 2 FLOP per MAC)."""
    s = block_sizes(N, B)
    return float(4 * d * (s[:, None] * s[None, :] * (mask != 0)).sum())


def anchor_head_flops(F, k, C, N, d) -> float:
    return float(4 * d * F * k * C * N)


def layer_work(wl):
    cfg = wl.cfg
    flags = wl.rep_flags[0, 0]
    sparse = [h for h in range(cfg.H) if not flags[h]]
    rep = [h for h in range(cfg.H) if flags[h]]
    f_sparse = sum(sparse_head_flops(wl.masks[0, 0, h], cfg.N, cfg.B, cfg.d) for h in sparse)
    f_anchor = len(rep) * anchor_head_flops(cfg.F, len(wl.anchors), cfg.C, cfg.N, cfg.d)
    s = block_sizes(cfg.N, cfg.B)
    tok = s[:, None] * s[None, :]
    token_sp = [1.0 - float((tok * (wl.masks[0, 0, h] != 0)).sum()) / cfg.N ** 2 for h in sparse]
    block_sp = [1.0 - float(wl.masks[0, 0, h].mean()) for h in sparse]
    anchor_sp = 1.0 - len(wl.anchors) / cfg.R
    layer_sp = (sum(token_sp) + anchor_sp * len(rep)) / cfg.H
    dense = cfg.H * 4.0 * cfg.d * cfg.N * cfg.N
    return dict(sparse_heads=sparse, rep_heads=rep, flops_sparse=f_sparse, flops_anchor=f_anchor,
                flops=f_sparse + f_anchor, flops_dense=dense,
                token_sparsity_sparse_heads=float(np.mean(token_sp)) if token_sp else None,
                block_sparsity_sparse_heads=float(np.mean(block_sp)) if block_sp else None,
                anchor_query_sparsity=anchor_sp if rep else None, layer_interaction_sparsity=layer_sp)


# ---------------------------------------------------------------------------
# CPU oracle baseline: a process pool over a stated subset of heads
# ---------------------------------------------------------------------------
CPU_POOL_CAP = 16     # host cores that go with one GPU on the measurement boxes


def _oracle_worker(job):
    """One pool worker: evaluates oracle units (a query block of a block-sparse head, or one frame of
    an anchor head) from its share until its time budget is spent, with BLAS on one thread.
    Returns (FLOP done, seconds busy, units done)."""
    tmp, meta, units, budget = job
    from threadpoolctl import threadpool_limits
    import oracle
    q = np.load(os.path.join(tmp, "q.npy"), mmap_mode="r")
    k = np.load(os.path.join(tmp, "k.npy"), mmap_mode="r")
    v = np.load(os.path.join(tmp, "v.npy"), mmap_mode="r")
    rp = np.load(os.path.join(tmp, "rp.npy"))
    ci = np.load(os.path.join(tmp, "ci.npy"))
    N, d, B = meta["N"], meta["d"], meta["B"]
    sizes = block_sizes(N, B)
    flop, done = 0.0, 0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        for kind, slot, idx in units:
            if time.perf_counter() - t0 >= budget:
                break
            if kind == "anchor":
                oracle.anchor_head(q[slot], k[slot], v[slot], meta["F"], meta["R"], meta["C"], meta["anchors"],
                                   meta["scale"], frames=[idx])
                flop += 4.0 * d * len(meta["anchors"]) * meta["C"] * N
            else:
                oracle.block_sparse_head(q[slot], k[slot], v[slot], rp, ci, slot, B, meta["scale"], blocks=[idx])
                row = slot * len(sizes) + idx
                flop += 4.0 * d * sizes[idx] * float(sizes[ci[rp[row]:rp[row + 1]]].sum())
            done += 1
        busy = time.perf_counter() - t0
    return flop, busy, done


def cpu_baseline(wl, budget_s: float, flops_layer: float):
    """The fp64 oracle on the host cores: a process pool (one worker per core, up to the cores that go
    with one GPU; BLAS on one thread per worker) over a subset of the layer's heads, 4 block-sparse heads
    and 1 anchor head. Each worker takes a shuffled share of the subset's units (query blocks of the
    sparse heads, frames of the anchor head) and runs them until `budget_s` of its own time is spent.
    The rate is the sum of the workers' FLOP/s (they run concurrently); the full layer's oracle time is
    extrapolated from it by algorithmic FLOP."""
    import multiprocessing as mp
    import shutil
    import tempfile
    import oracle
    import workloads
    cfg = wl.cfg
    cores_visible = len(os.sched_getaffinity(0))
    workers = max(1, min(cores_visible, CPU_POOL_CAP))
    flags = wl.rep_flags[0, 0]
    sparse = [h for h in range(cfg.H) if not flags[h]]
    rep = [h for h in range(cfg.H) if flags[h]]
    rng = np.random.default_rng(123)
    sub_sparse = sorted(int(h) for h in rng.choice(sparse, size=min(4, len(sparse)), replace=False))
    sub_rep = [int(rep[0])] if rep else []
    heads = sub_sparse + sub_rep
    as_f = workloads.bf16_to_f32 if cfg.dtype == "bf16" else (lambda x: np.asarray(x, np.float32))
    tmp = tempfile.mkdtemp(prefix="calibatt_oracle_")
    try:
        # the subset's exact input values in fp64 (the oracle's precision), shared by the workers
        for name, arr in (("q", wl.q), ("k", wl.k), ("v", wl.v)):
            np.save(os.path.join(tmp, f"{name}.npy"), np.stack([as_f(arr[h]).astype(np.float64) for h in heads]))
        # lists of the subset's sparse heads (records renumbered to the subset's slots)
        sub_masks = wl.masks[:, :, sub_sparse] if sub_sparse else wl.masks[:, :, :0]
        rp, ci, _ = oracle.compile_skiplist(sub_masks)
        np.save(os.path.join(tmp, "rp.npy"), rp)
        np.save(os.path.join(tmp, "ci.npy"), ci)
        units = [("sparse", i, r) for i in range(len(sub_sparse)) for r in range(cfg.nb)]
        units += [("anchor", len(sub_sparse) + i, f) for i in range(len(sub_rep)) for f in range(cfg.F)]
        order = rng.permutation(len(units))
        units = [units[i] for i in order]
        meta = {"N": cfg.N, "d": cfg.d, "B": cfg.B, "F": cfg.F, "R": cfg.R, "C": cfg.C,
                "anchors": [int(a) for a in wl.anchors], "scale": wl.scale}
        jobs = [(tmp, meta, units[w::workers], budget_s) for w in range(workers)]
        with mp.get_context("spawn").Pool(workers) as pool:
            res = pool.map(_oracle_worker, jobs)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    flop = sum(r[0] for r in res)
    rate = sum(r[0] / r[1] for r in res if r[1] > 0)
    done = sum(r[2] for r in res)
    busy = max(r[1] for r in res)
    n_sp = sum(1 for u in units if u[0] == "sparse")
    value = rate / 1e12 if rate > 0 else None
    return {"value": value, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"fp64 numpy oracle, process pool of {workers} workers (BLAS 1 thread each) over heads "
                      f"{sub_sparse} (block-sparse) and {sub_rep} (anchor) of the same layer: {done} of "
                      f"{len(units)} units ({n_sp} query blocks, {len(units) - n_sp} anchor frames), "
                      f"{flop / 1e12:.3f} TFLOP, in at most {busy:.1f} s per worker (budget {budget_s:.0f} s); "
                      f"the full layer extrapolated by algorithmic FLOP",
            "seconds_busy_max": round(busy, 2), "units_done": done, "units_total": len(units),
            "cores_visible": cores_visible, "blas_threads_per_worker": 1,
            "subset_heads": {"block_sparse": sub_sparse, "anchor": sub_rep},
            "extrapolated": True,
            "layer_seconds_extrapolated": round(flops_layer / rate, 1) if rate > 0 else None,
            "tflop_done": round(flop / 1e12, 4)}


def pmc_traffic(kernel_sha: str):
    """L2 <-> fabric bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by a 1 GiB copy; the MALL and HBM
    together, an upper bound on HBM bytes) from the committed counter summary, if it matches this kernel
    source."""
    path = os.path.join(ROOT, "profiles", "attn_wan720_hbm_counters.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256", "")[:16] != kernel_sha[:16]:
        return None
    try:
        return float(vals["fabric_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def dictionary_sweep(args):
    """Full-step mask dictionary at the 480p shape (40 layers x 40 heads): skip-list compile time
    and per-layer attention time across sparsity {0, 50, 68, 85}% x repetitive fraction {0, 10, 25}%."""
    import torch
    import workloads
    import calibrated_block_sparse_skiplist_amd as cal
    base = workloads.get_config("wan480_dual")
    q, k, v = workloads.make_qkv(base)
    dev = torch.device("cuda")
    qd, kd, vd = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) for x in (q, k, v))
    o = torch.empty_like(qd)
    anchors = workloads.equally_spaced_anchor_rows(base.R, base.n_anchor)
    scale = float(np.float32(1.0 / np.sqrt(base.d)))
    stream = torch.cuda.current_stream()
    for sp in (0.0, 0.5, 0.68, 0.85):
        for rf in (0.0, 0.10, 0.25):
            cfg, masks, flags = workloads.make_dictionary_workload(sp, rf)
            dm = torch.from_numpy(masks).to(dev)
            sl = cal.compile_skiplist(dm, cfg.N, cfg.B)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            reps = 3
            for _ in range(reps):
                cal.calibatt_compile_skiplist(dm, 1, cfg.L, cfg.H, cfg.N, cfg.B, sl.row_ptr, sl.col_idx,
                                              sl.col_idx.numel(), sl.order, stream)
            torch.cuda.synchronize()
            compile_ms = (time.perf_counter() - t0) * 1e3 / reps
            mask_bytes = masks.size
            out_bytes = 4 * sl.nnz + 8 * (masks.shape[1] * masks.shape[2] * cfg.nb + 1) + 4 * masks.shape[1] * masks.shape[2] * cfg.nb
            il = cal.compile_intervals(dm, cfg.N, cfg.B)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                cal.calibatt_compile_intervals(dm, 1, cfg.L, cfg.H, cfg.N, cfg.B, il.iv_ptr, il.iv, il.iv.numel(),
                                               il.order, stream)
            torch.cuda.synchronize()
            compile_iv_ms = (time.perf_counter() - t0) * 1e3 / reps
            rows = masks.shape[1] * masks.shape[2] * cfg.nb
            n_iv = il.n_iv
            del il
            # the compile oracle (plain numpy scan, one host core) on the same whole dictionary, once
            # per sparsity point
            oracle_compile_s = None
            if rf == 0.0 and not args.no_cpu_baseline:
                import oracle
                t0 = time.perf_counter()
                oracle.compile_skiplist(masks)
                oracle_compile_s = round(time.perf_counter() - t0, 3)
            layer_ms, flops = [], 0.0
            for l in range(min(args.sweep_layers, cfg.L)):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                for _ in range(2):
                    cal.calibatt_layer_dispatch(qd, kd, vd, o, None, sl, 0, l, flags, cfg.F, cfg.R, cfg.C, anchors,
                                                scale=scale, stream=stream)
                a.record(stream)
                for _ in range(5):
                    cal.calibatt_layer_dispatch(qd, kd, vd, o, None, sl, 0, l, flags, cfg.F, cfg.R, cfg.C, anchors,
                                                scale=scale, stream=stream)
                b.record(stream)
                torch.cuda.synchronize()
                layer_ms.append(a.elapsed_time(b) / 5)
                f = 0.0
                for h in range(cfg.H):
                    if flags[0, l, h]:
                        f += anchor_head_flops(cfg.F, len(anchors), cfg.C, cfg.N, cfg.d)
                    else:
                        f += sparse_head_flops(masks[0, l, h], cfg.N, cfg.B, cfg.d)
                flops += f / layer_ms[-1] / 1e9
            print(json.dumps({"sweep": "wan480_dictionary", "sparsity_target": sp, "repetitive_fraction": rf,
                              "layers": cfg.L, "heads": cfg.H, "nnz": sl.nnz,
                              "block_sparsity": round(1.0 - float(masks.astype(np.float64).mean()), 4),
                              "compile_with_order_ms": round(compile_ms, 3),
                              "compile_oracle_s_1core": oracle_compile_s,
                              "compile_GBps": round((2 * mask_bytes + out_bytes) / compile_ms / 1e6, 1),
                              "runs": n_iv, "compile_intervals_ms": round(compile_iv_ms, 3),
                              "list_MB_index_form": round((8 * (rows + 1) + 4 * sl.nnz) / 1e6, 2),
                              "list_MB_interval_form": round((8 * (rows + 1) + 4 * n_iv) / 1e6, 2),
                              "layer_ms_mean": round(float(np.mean(layer_ms)), 3),
                              "layer_ms": [round(x, 3) for x in layer_ms],
                              "tflops_mean": round(flops / len(layer_ms), 1)}), flush=True)
            del dm, sl


def calibration_bench(args):
    """Offline calibration of one layer at the Wan-720p shape: per prompt, block energies of all 40 heads
    (calibatt_block_energy, one pass with a workspace for all heads; the two-pass form without one is
    timed once beside it) and their top-tau selection accumulated into keep counts
    (calibatt_select_blocks); then the keep-frequency mask (calibatt_keep_frequency). The
    spatial-repetition branch: per prompt, row similarities of all heads in one pass
    (calibatt_spatial_similarity), then the flags (calibatt_repetition_flags)."""
    import torch
    import workloads
    import calibrated_block_sparse_skiplist_amd as cal
    cfg = workloads.get_config("wan720")
    H, N, d, B, nb = cfg.H, cfg.N, cfg.d, cfg.B, cfg.nb
    tau, rho = 0.9, 0.5
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    # one prompt's synthetic Q, K in HBM (the timed work does not depend on the values)
    q, k = workloads.make_calibration_prompts(N, d, cfg.F, cfg.R, cfg.C, H, 1, seed=8000)
    qd = torch.from_numpy(q[0].view(np.int16)).view(torch.bfloat16).to(dev)
    kd = torch.from_numpy(k[0].view(np.int16)).view(torch.bfloat16).to(dev)
    del q, k
    energy = torch.empty((H, nb, nb), dtype=torch.float32, device=dev)
    counts = torch.zeros((H, nb, nb), dtype=torch.int32, device=dev)
    mask = torch.empty((H, nb, nb), dtype=torch.uint8, device=dev)
    # two-pass form (no workspace), timed once
    cal.calibatt_block_energy(qd, kd, energy, B, stream=stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    cal.calibatt_block_energy(qd, kd, energy, B, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    two_pass_ms = a.elapsed_time(b)
    # one-pass form: the workspace of every head (nb*nb*B floats each)
    work = torch.empty((cal.energy_work_bytes(N, B, H) // 4,), dtype=torch.float32, device=dev)
    cal.calibatt_block_energy(qd, kd, energy, B, work=work, stream=stream)
    torch.cuda.synchronize()
    e_ms, s_ms = [], []
    for _ in range(args.prompts):
        a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record(stream)
        b.record(stream)
        cal.calibatt_set_kernel_events(a.cuda_event, b.cuda_event)
        cal.calibatt_block_energy(qd, kd, energy, B, work=work, stream=stream)
        cal.calibatt_select_blocks(energy, tau, counts=counts, stream=stream)
        c.record(stream)
        torch.cuda.synchronize()
        e_ms.append(a.elapsed_time(b))
        s_ms.append(b.elapsed_time(c))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    cal.calibatt_keep_frequency(counts, args.prompts, rho, mask, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    keep_ms = a.elapsed_time(b)
    # spatial-repetition branch: per prompt, row similarities of all heads; then the flags
    anchors = workloads.equally_spaced_anchor_rows(cfg.R, cfg.n_anchor)
    sims = torch.empty((args.prompts, H, cfg.F, cfg.R), dtype=torch.float32, device=dev)
    cal.calibatt_spatial_similarity(qd, kd, cfg.F, cfg.R, cfg.C, anchors, sims[0], stream=stream)
    torch.cuda.synchronize()
    sim_ms, simk_ms = [], []
    for p in range(args.prompts):
        a, b, c, e = (torch.cuda.Event(enable_timing=True) for _ in range(4))
        a.record(stream)
        b.record(stream)
        c.record(stream)
        cal.calibatt_set_kernel_events(b.cuda_event, c.cuda_event)
        cal.calibatt_spatial_similarity(qd, kd, cfg.F, cfg.R, cfg.C, anchors, sims[p], stream=stream)
        e.record(stream)
        torch.cuda.synchronize()
        sim_ms.append(a.elapsed_time(e))
        simk_ms.append(b.elapsed_time(c))
    flags = torch.empty((H,), dtype=torch.uint8, device=dev)
    mean = torch.empty((H,), dtype=torch.float32, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    cal.calibatt_repetition_flags(sims, anchors, 0.87, flags=flags, mean=mean, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    flags_ms = a.elapsed_time(b)
    sim_flop = 2.0 * d * N * (2 * cfg.C * (cfg.R - len(anchors)) * cfg.F) * H    # row and anchor scores per pair

    energy_ms = float(np.mean(e_ms))
    qk_flop = 2.0 * d * N * N * H                  # one QK^T product over all heads (computed once)
    work_gb = work.numel() * 4 / 1e9
    del work
    row_sums = energy.sum(dim=2)
    print(json.dumps({
        "mode": "calibration", "workload": "wan720 shape: H=40, N=75600, d=128, 128x128 blocks, bf16",
        "prompts": args.prompts, "tau": tau, "rho": rho,
        "energy_ms_per_prompt": round(energy_ms, 3),
        "energy_tflops": round(qk_flop / (energy_ms * 1e-3) / 1e12, 1),
        "energy_frac_of_bf16_peak": round(qk_flop / (energy_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "energy_workspace_gb": round(work_gb, 2),
        "energy_two_pass_ms": round(two_pass_ms, 3),
        "select_ms_per_prompt": round(float(np.mean(s_ms)), 3),
        "select_rows": H * nb, "nb": nb, "keep_frequency_ms": round(keep_ms, 3),
        "kept_fraction_final_mask": round(float(mask.float().mean().item()), 4),
        "energy_row_sum_max_dev": float((row_sums - 1.0).abs().max().item()),
        "similarity_ms_per_prompt": round(float(np.mean(sim_ms)), 3),
        "similarity_kernel_ms": round(float(np.mean(simk_ms)), 3),
        "similarity_kernel_tflops": round(sim_flop / (float(np.mean(simk_ms)) * 1e-3) / 1e12, 1),
        "repetition_flags_ms": round(flags_ms, 3),
        "mean_row_similarity": [round(float(x), 4) for x in mean.cpu().numpy()[:4]],
    }), flush=True)


def dictionary_run(args):
    """Wan-720p denoising-run dictionary (T=50, L=40, H=40): 27.9 GB of block masks generated on the GPU,
    compiled into index lists, runs and bitmaps in one call each; memory of each form; then every layer
    call of the chosen timesteps (record (t, l) selected from the resident dictionary), through the runs
    and through the bitmaps."""
    import torch
    import workloads
    import calibrated_block_sparse_skiplist_amd as cal
    T, L, H = 50, 40, 40
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    cfg, masks, flags = workloads.make_step_dictionary("wan720", T, L, H, dev)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0
    nb = cfg.nb
    rows = T * L * H * nb
    mask_bytes = masks.numel()
    kept = int(torch.count_nonzero(masks).item())

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        a = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - a) * 1e3 / reps

    il = cal.compile_intervals(masks, cfg.N, cfg.B)
    iv_ms = timed(lambda: cal.calibatt_compile_intervals(masks, T, L, H, cfg.N, cfg.B, il.iv_ptr, il.iv,
                                                         il.iv.numel(), il.order, stream))
    sl = cal.compile_skiplist(masks, cfg.N, cfg.B)
    csr_ms = timed(lambda: cal.calibatt_compile_skiplist(masks, T, L, H, cfg.N, cfg.B, sl.row_ptr, sl.col_idx,
                                                         sl.col_idx.numel(), sl.order, stream))
    bm = cal.compile_bitmap(masks, cfg.N, cfg.B)
    bm_ms = timed(lambda: cal.calibatt_compile_bitmap(masks, T, L, H, cfg.N, cfg.B, bm.bits, stream))
    n_iv, nnz = il.n_iv, sl.nnz
    # block sizes for the work of each record
    sizes = torch.from_numpy(block_sizes(cfg.N, cfg.B)).to(dev, torch.float64)
    tok = sizes[:, None] * sizes[None, :]
    del sl
    torch.cuda.empty_cache()

    import workloads as W
    q, k, v = W.make_qkv(cfg)
    qd, kd, vd = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) for x in (q, k, v))
    del q, k, v
    o = torch.empty_like(qd)
    anchors = W.equally_spaced_anchor_rows(cfg.R, cfg.n_anchor)
    scale = float(np.float32(1.0 / np.sqrt(cfg.d)))
    per_step = []
    bm_bytes = bm.bits.numel() * 8
    for t in [int(x) for x in args.run_steps.split(",")]:
        cal.calibatt_layer_dispatch_iv(qd, kd, vd, o, None, il, t, 0, flags, cfg.F, cfg.R, cfg.C, anchors,
                                       scale=scale, stream=stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for l in range(L):
            cal.calibatt_layer_dispatch_iv(qd, kd, vd, o, None, il, t, l, flags, cfg.F, cfg.R, cfg.C, anchors,
                                           scale=scale, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        flop = 0.0
        for l in range(L):
            sp = torch.from_numpy(flags[t, l] == 0).to(dev)
            flop += float(4 * cfg.d * (tok[None] * masks[t, l][sp].to(torch.float64)).sum().item())
            flop += float((~sp).sum().item()) * anchor_head_flops(cfg.F, len(anchors), cfg.C, cfg.N, cfg.d)
        # the same 40 layer calls through the bitmap form
        a.record(stream)
        for l in range(L):
            cal.calibatt_layer_dispatch_bm(qd, kd, vd, o, None, bm, t, l, flags, cfg.F, cfg.R, cfg.C, anchors,
                                           scale=scale, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms_bm = a.elapsed_time(b)
        per_step.append({"t": t, "layers": L, "ms_total": round(ms, 2), "ms_per_layer": round(ms / L, 3),
                         "ms_per_layer_bitmap_form": round(ms_bm / L, 3),
                         "kept_fraction": round(float(masks[t].float().mean().item()), 4),
                         "tflops": round(flop / (ms * 1e-3) / 1e12, 1)})
    print(json.dumps({
        "mode": "dictionary_run", "workload": "wan720 shape, 50 timesteps x 40 layers x 40 heads",
        "mask_generation_s": round(gen_s, 2), "records": T * L * H, "rows": rows, "nb": nb,
        "kept_blocks": kept, "kept_fraction": round(kept / mask_bytes, 4), "runs": n_iv,
        "bytes": {"masks": mask_bytes, "index_form": 8 * (rows + 1) + 4 * nnz + 4 * rows,
                  "interval_form": 8 * (rows + 1) + 4 * n_iv + 4 * rows,
                  "interval_form_runs_only": 4 * n_iv, "bitmap_form": bm_bytes},
        "compile_ms": {"index_form": round(csr_ms, 2), "interval_form": round(iv_ms, 2),
                       "bitmap_form": round(bm_ms, 2)},
        "compile_GBps_masks_read_twice": round(2 * mask_bytes / (iv_ms * 1e-3) / 1e9, 1),
        "layer_calls": per_step}), flush=True)


def measure_layer_config(key: str, reps: int = 10, dense_reps: int = 2):
    """A further layer configuration, timed the way the headline is (layer-call = calibatt_layer_dispatch
    with O only; the attention kernel alone via HIP events on its stream; the same kernel dense over all
    heads). Returns a small dict for the bench line."""
    import torch
    import workloads
    import calibrated_block_sparse_skiplist_amd as cal
    wl = workloads.make_workload(key)
    cfg = wl.cfg
    work = layer_work(wl)
    dev = torch.device("cuda")
    q, k, v = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) for x in (wl.q, wl.k, wl.v))
    o = torch.empty_like(q)
    sl = cal.compile_skiplist(torch.from_numpy(wl.masks).to(dev), cfg.N, cfg.B)
    stream = torch.cuda.current_stream()

    def call(ev=None):
        if ev is not None:
            cal.calibatt_set_kernel_events(ev[0].cuda_event, ev[1].cuda_event)
        cal.calibatt_layer_dispatch(q, k, v, o, None, sl, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                    scale=wl.scale, stream=stream)
    for _ in range(2):
        call()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for ev in evs:
        call(ev)
    e1.record(stream)
    torch.cuda.synchronize()
    layer_ms = e0.elapsed_time(e1) / reps
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    ones = torch.ones((1, 1, cfg.H, cfg.nb, cfg.nb), dtype=torch.uint8, device=dev)
    sld = cal.compile_skiplist(ones, cfg.N, cfg.B)
    cal.calibatt_block_sparse_attn(q, k, v, o, None, sld, 0, 0, scale=wl.scale, stream=stream)
    e0.record(stream)
    for _ in range(dense_reps):
        cal.calibatt_block_sparse_attn(q, k, v, o, None, sld, 0, 0, scale=wl.scale, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    dense_ms = e0.elapsed_time(e1) / dense_reps
    tf = work["flops"] / (layer_ms * 1e-3) / 1e12
    return {"workload": f"{cfg.key}: {cfg.title}", "sparse_heads": len(work["sparse_heads"]),
            "repetitive_heads": len(work["rep_heads"]),
            "token_sparsity_sparse_heads": round(work["token_sparsity_sparse_heads"], 4),
            "retained_tflop": round(work["flops"] / 1e12, 3), "layer_call_ms": round(layer_ms, 3),
            "attn_kernel_ms": round(kern_ms, 3), "tflops": round(tf, 1),
            "pct_of_bf16_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
            "kernel_tflops": round(work["flops"] / (kern_ms * 1e-3) / 1e12, 1),
            "dense_same_kernel_ms": round(dense_ms, 3), "speedup_vs_dense": round(dense_ms / layer_ms, 3)}


def sweep_summary(layers: int = 2, reps: int = 5):
    """The 480p dictionary sweep (sparsity 0/50/68/85 % x repetitive fraction 0/10/25 %), cut to its
    first `layers` layers (the same masks and flags as the first layers of the 40-layer dictionary):
    per point the compile of those layers' masks and the mean layer-call (each layer timed over
    `reps` back-to-back calls after two warm-up calls)."""
    import torch
    import workloads
    import calibrated_block_sparse_skiplist_amd as cal
    base = workloads.get_config("wan480_dual")
    q, k, v = workloads.make_qkv(base)
    dev = torch.device("cuda")
    qd, kd, vd = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) for x in (q, k, v))
    del q, k, v
    o = torch.empty_like(qd)
    anchors = workloads.equally_spaced_anchor_rows(base.R, base.n_anchor)
    scale = float(np.float32(1.0 / np.sqrt(base.d)))
    stream = torch.cuda.current_stream()
    points = []
    for sp in (0.0, 0.5, 0.68, 0.85):
        for rf in (0.0, 0.10, 0.25):
            cfg, masks, flags = workloads.make_dictionary_workload(sp, rf, L=layers)
            dm = torch.from_numpy(masks).to(dev)
            sl = cal.compile_skiplist(dm, cfg.N, cfg.B)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            cal.calibatt_compile_skiplist(dm, 1, cfg.L, cfg.H, cfg.N, cfg.B, sl.row_ptr, sl.col_idx,
                                          sl.col_idx.numel(), None, stream)
            torch.cuda.synchronize()
            compile_ms = (time.perf_counter() - t0) * 1e3
            ms, fl = [], []
            for l in range(cfg.L):
                # two warm-up calls, then `reps` back to back (a single call timed right after a new
                # dictionary point reads several hundred microseconds long: cold caches and clocks)
                for _ in range(2):
                    cal.calibatt_layer_dispatch(qd, kd, vd, o, None, sl, 0, l, flags, cfg.F, cfg.R, cfg.C, anchors,
                                                scale=scale, stream=stream)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(reps):
                    cal.calibatt_layer_dispatch(qd, kd, vd, o, None, sl, 0, l, flags, cfg.F, cfg.R, cfg.C, anchors,
                                                scale=scale, stream=stream)
                b.record(stream)
                torch.cuda.synchronize()
                ms.append(a.elapsed_time(b) / reps)
                f = sum(anchor_head_flops(cfg.F, len(anchors), cfg.C, cfg.N, cfg.d) if flags[0, l, h]
                        else sparse_head_flops(masks[0, l, h], cfg.N, cfg.B, cfg.d) for h in range(cfg.H))
                fl.append(f)
            lm = float(np.mean(ms))
            points.append({"sparsity": sp, "repetitive_fraction": rf,
                           "block_sparsity": round(1.0 - float(masks.astype(np.float64).mean()), 4),
                           "compile_ms": round(compile_ms, 3), "layer_call_ms": round(lm, 3),
                           "tflops": round(float(np.mean(fl)) / (lm * 1e-3) / 1e12, 1)})
            del dm, sl
    dense = {p["repetitive_fraction"]: p["layer_call_ms"] for p in points if p["sparsity"] == 0.0}
    for p in points:
        p["speedup_vs_dense"] = round(dense[0.0] / p["layer_call_ms"], 3)
    return {"workload": f"480p dictionary, 40 heads, first {layers} layers per point "
                        "(speedups against the 0 %-sparsity, 0 %-repetitive point)", "points": points}


def profile_workload(kind: str):
    """Fixed kernel sequences for counter passes (launches told apart by kernel name, grid and order)."""
    import torch
    import workloads
    import calibrated_block_sparse_skiplist_amd as cal
    dev = torch.device("cuda")
    if kind == "layer":
        wl = workloads.make_workload("wan720")
        cfg = wl.cfg
        q, k, v = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) for x in (wl.q, wl.k, wl.v))
        o = torch.empty_like(q)
        masks = torch.from_numpy(wl.masks).to(dev)
        sl = cal.compile_skiplist(masks, cfg.N, cfg.B)
        sld = cal.compile_skiplist(torch.ones((1, 1, cfg.H, cfg.nb, cfg.nb), dtype=torch.uint8, device=dev),
                                   cfg.N, cfg.B)
        torch.cuda.synchronize()
        for _ in range(3):
            cal.calibatt_compile_skiplist(masks, 1, 1, cfg.H, cfg.N, cfg.B, sl.row_ptr, sl.col_idx,
                                          sl.col_idx.numel(), None)
        bm = cal.compile_bitmap(masks, cfg.N, cfg.B)
        for _ in range(3):
            cal.calibatt_compile_bitmap(masks, 1, 1, cfg.H, cfg.N, cfg.B, bm.bits)
        for _ in range(3):
            cal.calibatt_layer_dispatch(q, k, v, o, None, sl, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                        scale=wl.scale)
        torch.cuda.synchronize()
        for _ in range(3):
            cal.calibatt_block_sparse_attn(q, k, v, o, None, sld, 0, 0, heads=list(range(8)), scale=wl.scale)
    else:
        base = workloads.get_config("wan480_dual")
        q, k, v = workloads.make_qkv(base)
        qd, kd, vd = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) for x in (q, k, v))
        o = torch.empty_like(qd)
        scale = float(np.float32(1.0 / np.sqrt(base.d)))
        lists = []
        for sp in (0.0, 0.68, 0.85):
            cfg, masks, _ = workloads.make_dictionary_workload(sp, 0.0, L=1)
            lists.append(cal.compile_skiplist(torch.from_numpy(masks).to(dev), cfg.N, cfg.B))
        torch.cuda.synchronize()
        for sl in lists:
            for _ in range(3):
                cal.calibatt_block_sparse_attn(qd, kd, vd, o, None, sl, 0, 0, scale=scale)
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    print(json.dumps({"profile": kind, "done": True}), flush=True)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(a layer shards by head with no communication: each GPU would run this single-GPU workload on its share "
              "of the heads)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.profile:
        profile_workload(args.profile)
        return
    if args.dictionary_sweep:
        dictionary_sweep(args)
        return
    if args.calibration:
        calibration_bench(args)
        return
    if args.dictionary_run:
        dictionary_run(args)
        return
    if args.copy_calib:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": src.numel() * 4}))
        return

    import workloads
    import calibrated_block_sparse_skiplist_amd as cal

    t0 = time.time()
    wl = workloads.make_workload(args.config)
    cfg = wl.cfg
    work = layer_work(wl)
    print(f"[bench] {cfg.title}: generated in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    dev = torch.device("cuda")
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def up(x):
        if cfg.dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    q, k, v = up(wl.q), up(wl.k), up(wl.v)
    o = torch.empty_like(q)
    lse = torch.empty((cfg.H, cfg.N), dtype=torch.float32, device=dev)
    masks = torch.from_numpy(wl.masks).to(dev)
    sl = cal.compile_skiplist(masks, cfg.N, cfg.B)
    T, L, H, nb = 1, 1, cfg.H, cfg.nb
    stream = torch.cuda.current_stream()

    def step(ev_pair=None):
        # (the heaviest-first order is a compile output for callers that schedule by cost; the attention
        # kernel visits query blocks in block order and does not read it, so the step does not compute it)
        cal.calibatt_compile_skiplist(masks, T, L, H, cfg.N, cfg.B, sl.row_ptr, sl.col_idx, sl.col_idx.numel(),
                                      None, stream)
        if ev_pair is not None:
            cal.calibatt_set_kernel_events(ev_pair[0].cuda_event, ev_pair[1].cuda_event)
        cal.calibatt_layer_dispatch(q, k, v, o, None, sl, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                    scale=wl.scale, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:          # create the underlying HIP events
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    kernel_ms = [a.elapsed_time(b) for a, b in evs]
    attn_ms = float(np.mean(kernel_ms))

    # layer-call alone (no compile), for reference
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    reps = max(3, args.steps // 2)
    for _ in range(reps):
        cal.calibatt_layer_dispatch(q, k, v, o, None, sl, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                    scale=wl.scale, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    layer_ms = e0.elapsed_time(e1) / reps
    # the same layer-call also writing the optional log-sum-exp (an extra fp32 row sum in the kernel)
    e0.record(stream)
    for _ in range(reps):
        cal.calibatt_layer_dispatch(q, k, v, o, lse, sl, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                    scale=wl.scale, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    layer_lse_ms = e0.elapsed_time(e1) / reps

    # layer-call timing protocol: 5 warm-ups, then R calls timed one by one with HIP events, back to
    # back (warm) and with 1 GiB written before each call (cold: more than the 256 MB MALL); the
    # median and the minimum of each
    protocol = None
    if args.protocol_reps > 0:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)

        def dispatch():
            cal.calibatt_layer_dispatch(q, k, v, o, None, sl, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                        scale=wl.scale, stream=stream)

        def timed(cold):
            pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(args.protocol_reps)]
            for _ in range(5):
                dispatch()
            for a, b in pairs:
                if cold:
                    flush.fill_(1.0)
                a.record(stream)
                dispatch()
                b.record(stream)
            torch.cuda.synchronize()
            return [a.elapsed_time(b) for a, b in pairs]

        warm, cold = timed(False), timed(True)
        protocol = {"reps": args.protocol_reps, "warmups": 5, "flush_bytes": flush.numel() * 4,
                    "warm_median_ms": round(float(np.median(warm)), 3), "warm_min_ms": round(float(np.min(warm)), 3),
                    "cold_median_ms": round(float(np.median(cold)), 3), "cold_min_ms": round(float(np.min(cold)), 3)}
        del flush
    # compile alone: the lists (as in the step), and the lists with the heaviest-first order
    t_c = time.perf_counter()
    for _ in range(5):
        cal.calibatt_compile_skiplist(masks, T, L, H, cfg.N, cfg.B, sl.row_ptr, sl.col_idx, sl.col_idx.numel(),
                                      None, stream)
    torch.cuda.synchronize()
    compile_ms = (time.perf_counter() - t_c) * 1e3 / 5
    t_c = time.perf_counter()
    for _ in range(5):
        cal.calibatt_compile_skiplist(masks, T, L, H, cfg.N, cfg.B, sl.row_ptr, sl.col_idx, sl.col_idx.numel(),
                                      sl.order, stream)
    torch.cuda.synchronize()
    compile_order_ms = (time.perf_counter() - t_c) * 1e3 / 5

    # the same layer through the interval form of the skip list
    il = cal.compile_intervals(masks, cfg.N, cfg.B)
    t_c = time.perf_counter()
    for _ in range(5):
        cal.calibatt_compile_intervals(masks, T, L, H, cfg.N, cfg.B, il.iv_ptr, il.iv, il.iv.numel(), il.order,
                                       stream)
    torch.cuda.synchronize()
    compile_iv_ms = (time.perf_counter() - t_c) * 1e3 / 5
    cal.calibatt_layer_dispatch_iv(q, k, v, o, None, il, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                   scale=wl.scale, stream=stream)
    e0.record(stream)
    for _ in range(reps):
        cal.calibatt_layer_dispatch_iv(q, k, v, o, None, il, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                       scale=wl.scale, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    layer_iv_ms = e0.elapsed_time(e1) / reps
    rows = T * L * H * nb
    intervals = {"runs": il.n_iv, "kept_blocks": sl.nnz, "compile_ms": round(compile_iv_ms, 3),
                 "layer_call_ms": round(layer_iv_ms, 3),
                 "list_bytes_index_form": 8 * (rows + 1) + 4 * sl.nnz,
                 "list_bytes_interval_form": 8 * (rows + 1) + 4 * il.n_iv}
    del il

    # the same layer through the bitmap form (one bit per key block)
    bm = cal.compile_bitmap(masks, cfg.N, cfg.B)
    t_c = time.perf_counter()
    for _ in range(5):
        cal.calibatt_compile_bitmap(masks, T, L, H, cfg.N, cfg.B, bm.bits, stream)
    torch.cuda.synchronize()
    compile_bm_ms = (time.perf_counter() - t_c) * 1e3 / 5
    cal.calibatt_layer_dispatch_bm(q, k, v, o, None, bm, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                   scale=wl.scale, stream=stream)
    e0.record(stream)
    for _ in range(reps):
        cal.calibatt_layer_dispatch_bm(q, k, v, o, None, bm, 0, 0, wl.rep_flags, cfg.F, cfg.R, cfg.C, wl.anchors,
                                       scale=wl.scale, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    bitmap = {"words_per_row": bm.bits.shape[1], "compile_ms": round(compile_bm_ms, 3),
              "layer_call_ms": round(e0.elapsed_time(e1) / reps, 3), "bytes": bm.bits.numel() * 8}
    del bm

    dense_ms = None
    if not args.no_dense:
        ones = torch.ones((1, 1, H, nb, nb), dtype=torch.uint8, device=dev)
        sld = cal.compile_skiplist(ones, cfg.N, cfg.B)
        od = torch.empty_like(q)
        cal.calibatt_block_sparse_attn(q, k, v, od, None, sld, 0, 0, scale=wl.scale, stream=stream)
        torch.cuda.synchronize()
        d_ms = []
        for _ in range(args.dense_reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            b.record(stream)
            cal.calibatt_set_kernel_events(a.cuda_event, b.cuda_event)
            cal.calibatt_block_sparse_attn(q, k, v, od, None, sld, 0, 0, scale=wl.scale, stream=stream)
            torch.cuda.synchronize()
            d_ms.append(a.elapsed_time(b))
        dense_ms = float(np.mean(d_ms))
        del od, sld, ones

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds, work["flops"])

    # the other layer configurations and the sweep, measured in the same run (after the headline)
    extra = None
    if not args.no_extra_configs and args.config == "wan720":
        del q, k, v, o, lse, masks, sl
        torch.cuda.empty_cache()
        extra = {"configs": [measure_layer_config(key) for key in ("wan480_sparse", "wan480_dual")],
                 "sweep_480p": sweep_summary()}

    flops = work["flops"]
    achieved = flops / (attn_ms * 1e-3) / 1e12
    traffic = pmc_traffic(attn_source_sha())
    value = flops / (ms_per_step * 1e-3) / 1e12
    res = {
        "metric": "ms per attention layer-call + retained-block TFLOP/s (% of bf16 MFMA peak)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.key}: {cfg.title}", "H": cfg.H, "N": cfg.N, "d": cfg.d, "B": cfg.B,
                   "frames_rows_cols": [cfg.F, cfg.R, cfg.C], "sparse_heads": len(work["sparse_heads"]),
                   "repetitive_heads": len(work["rep_heads"]), "anchor_rows": [int(a) for a in wl.anchors],
                   "step": "calibatt_compile_skiplist (lists, no order) + calibatt_layer_dispatch (O; lse timed "
                           "separately)"},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "layer_call_ms": round(layer_ms, 3),
        "compile_ms": round(compile_ms, 3),
        "compile_with_order_ms": round(compile_order_ms, 3),
        "attn_kernel_ms": round(attn_ms, 3),
        "retained_tflop_per_layer": round(flops / 1e12, 3),
        "tflop_sparse_heads": round(work["flops_sparse"] / 1e12, 3),
        "tflop_anchor_heads": round(work["flops_anchor"] / 1e12, 3),
        "dense_same_kernel_ms": round(dense_ms, 3) if dense_ms else None,
        "dense_tflops": round(work["flops_dense"] / (dense_ms * 1e-3) / 1e12, 1) if dense_ms else None,
        "speedup_vs_dense": round(dense_ms / layer_ms, 3) if dense_ms else None,
        "layer_call_with_lse_ms": round(layer_lse_ms, 3),
        "layer_call_protocol": protocol,
        "intervals": intervals,
        "bitmap": bitmap,
        "sparsity": {"token_sparse_heads": work["token_sparsity_sparse_heads"],
                     "block_sparse_heads": work["block_sparsity_sparse_heads"],
                     "anchor_query": work["anchor_query_sparsity"],
                     "layer_interactions": work["layer_interaction_sparsity"]},
        "roofline": {"kernel": ATTN_KERNEL, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "traffic_kind": "L2<->fabric bytes per launch (MALL and HBM together; FETCH_SIZE + WRITE_SIZE "
                                     "scaled by a 1 GiB copy)",
                     "flop_per_launch": flops, "launch_ms": round(attn_ms, 3)},
        "cpu_baseline": cpu,
        "other_workloads": extra,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
