"""Seeded synthetic workloads for the CalibAtt layer hot path.

This module is shared by the tests, the benchmark and the smoke check. It only
*draws inputs*: attention activations with video-transformer shapes, block
masks with spatiotemporal locality, repetition flags and anchor-row lists. It
holds none of the method's arithmetic (no skip-list encoding, no attention, no
anchor assignment): the CPU oracle and the HIP library each implement those on
their own, and both consume exactly the arrays produced here.

The shapes stand in for the Wan 2.1 14B video transformer that the pages
measure on (papernotes.org notes on "Accelerating Text-to-Video Generation with
Calibrated Sparse Attention", Main Results, Tables 1 and 2): 40 heads of width
128, 21 latent frames of 30x52 (480p) or 45x80 (720p) tokens, and 128x128
FlashAttention blocks (same notes, Key Design 1). No model weights or prompts
are involved; every value is drawn from a seeded PCG64 stream.

Token order inside a layer is frame-major, then spatial row, then column:
token n = (f * R + r) * C + c.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "LayerConfig", "CONFIGS", "get_config", "bf16_bits", "bf16_to_f32",
    "make_qkv", "block_frame_distance", "make_masks", "make_rep_flags",
    "equally_spaced_anchor_rows", "Workload", "make_workload",
    "make_dictionary_workload", "make_calibration_prompts", "make_step_dictionary",
]


# ---------------------------------------------------------------------------
# bf16 helpers (input preparation only)
# ---------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the raw 16-bit patterns as uint16. Inputs are finite by
    construction (normal samples plus a bounded bias), so no NaN handling.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Configurations
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class LayerConfig:
    """One synthetic attention layer (or a dictionary of layers).

    H heads, F frames of R spatial rows by C columns (N = F*R*C tokens),
    head width d, square blocks of B tokens, dtype "bf16" or "f32".
    """
    key: str
    title: str
    H: int
    F: int
    R: int
    C: int
    d: int
    B: int
    dtype: str
    n_rep: int                 # repetitive heads per layer
    n_anchor: int              # anchor rows per frame for repetitive heads
    mask_rule: str             # "tiny" | "band" | "target"
    k_bias: bool               # add the smooth spatiotemporal bias to K
    L: int = 1
    T: int = 1
    seed_base: int = 0         # data seed = 1000 + base, masks 2000 + base, rep 3000 + base
    sparsity_targets: tuple = ()  # "target" rule only (per-sparse-head targets drawn from these)
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def N(self) -> int:
        return self.F * self.R * self.C

    @property
    def nb(self) -> int:
        return -(-self.N // self.B)


CONFIGS = {
    "tiny": LayerConfig(
        key="tiny", title="tiny fp32 layer, H=2, 4x16x16 tokens, d=64, 64x64 blocks",
        H=2, F=4, R=16, C=16, d=64, B=64, dtype="f32", n_rep=1, n_anchor=2,
        mask_rule="tiny", k_bias=False, seed_base=1),
    "wan480_sparse": LayerConfig(
        key="wan480_sparse", title="Wan-480p-shaped layer, all 40 heads block-sparse",
        H=40, F=21, R=30, C=52, d=128, B=128, dtype="bf16", n_rep=0, n_anchor=5,
        mask_rule="band", k_bias=True, seed_base=2),
    "wan480_dual": LayerConfig(
        key="wan480_dual", title="Wan-480p-shaped layer, 10 of 40 heads repetitive",
        H=40, F=21, R=30, C=52, d=128, B=128, dtype="bf16", n_rep=10, n_anchor=5,
        mask_rule="band", k_bias=True, seed_base=3),
    "wan720": LayerConfig(
        key="wan720", title="Wan-720p-shaped layer, 32 block-sparse heads at 68% mean sparsity + 8 anchor heads",
        H=40, F=21, R=45, C=80, d=128, B=128, dtype="bf16", n_rep=8, n_anchor=5,
        mask_rule="target", k_bias=True, seed_base=4),
}


def get_config(key: str) -> LayerConfig:
    return CONFIGS[key]


# ---------------------------------------------------------------------------
# Activations
# ---------------------------------------------------------------------------
def _k_bias(H, F, R, C, d, rng):
    """Smooth spatiotemporal bias, one wave pattern per head and a phase per channel.

    bias[h, n, j] = 0.5 * cos(theta_h(n) + phi[h, j]) with
    theta_h(f, r, c) = 2*pi*(alpha_h f/F + beta_h r/R + gamma_h c/C).
    Evaluated as cos(a)cos(b) - sin(a)sin(b) so it costs two outer products.
    """
    f = np.arange(F, dtype=np.float64)[:, None, None] / F
    r = np.arange(R, dtype=np.float64)[None, :, None] / R
    c = np.arange(C, dtype=np.float64)[None, None, :] / C
    abc = rng.integers(1, 4, size=(H, 3))
    phi = rng.uniform(0.0, 2.0 * np.pi, size=(H, d))
    out = np.empty((H, F * R * C, d), dtype=np.float32)
    for h in range(H):
        theta = (2.0 * np.pi * (abc[h, 0] * f + abc[h, 1] * r + abc[h, 2] * c)).reshape(-1)
        ca, sa = np.cos(theta), np.sin(theta)
        cb, sb = np.cos(phi[h]), np.sin(phi[h])
        out[h] = (0.5 * (np.outer(ca, cb) - np.outer(sa, sb))).astype(np.float32)
    return out


def make_qkv(cfg: LayerConfig, seed: int | None = None, heads: int | None = None):
    """Q, K, V of shape [H, N, d].

    bf16 configs return uint16 bit patterns (the exact inputs both sides
    consume); the f32 config returns float32 arrays. Values are standard
    normal samples; K gets the smooth bias when the config asks for it.
    """
    H = cfg.H if heads is None else heads
    rng = np.random.Generator(np.random.PCG64(1000 + cfg.seed_base if seed is None else seed))
    shape = (H, cfg.N, cfg.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if cfg.k_bias:
        k += _k_bias(H, cfg.F, cfg.R, cfg.C, cfg.d, rng)
    if cfg.dtype == "bf16":
        return bf16_bits(q), bf16_bits(k), bf16_bits(v)
    return q, k, v


# ---------------------------------------------------------------------------
# Masks (workload structure: temporal locality plus random far blocks)
# ---------------------------------------------------------------------------
def block_frame_distance(N: int, B: int, F: int, R: int, C: int) -> np.ndarray:
    """Temporal distance in frames between query block r and key block c.

    Each block spans frames [first // (R*C), last // (R*C)] of the tokens it
    covers; the distance is the gap between the two spans (0 if they overlap).
    """
    nb = -(-N // B)
    first = np.arange(nb, dtype=np.int64) * B
    last = np.minimum(first + B, N) - 1
    lo, hi = first // (R * C), last // (R * C)
    return np.maximum(0, np.maximum(lo[None, :] - hi[:, None], lo[:, None] - hi[None, :]))


def _largest_band(dist: np.ndarray, keep_fraction: float) -> int:
    w = 0
    while w + 1 <= int(dist.max()) and (dist <= w + 1).mean() <= keep_fraction:
        w += 1
    return w


def _exact_count_mask(dist, w, keep_fraction, rng):
    nb = dist.shape[0]
    band = dist <= w
    want = int(round(keep_fraction * nb * nb)) - int(band.sum())
    m = band.copy()
    if want > 0:
        far = np.flatnonzero(~band.reshape(-1))
        pick = rng.choice(far, size=min(want, far.size), replace=False)
        m.reshape(-1)[pick] = True
    return m


def make_masks(cfg: LayerConfig, seed: int | None = None, rep_flags=None) -> np.ndarray:
    """uint8 masks [T, L, H, nb, nb] (nonzero = compute this block pair)."""
    rng = np.random.Generator(np.random.PCG64(2000 + cfg.seed_base if seed is None else seed))
    nb, H = cfg.nb, cfg.H
    out = np.zeros((cfg.T, cfg.L, H, nb, nb), dtype=np.uint8)
    eye = np.eye(nb, dtype=bool)
    if cfg.mask_rule == "tiny":
        for h in range(H):
            m = eye | (rng.random((nb, nb)) < 0.35)
            out[0, 0, h] = m
        return out
    dist = block_frame_distance(cfg.N, cfg.B, cfg.F, cfg.R, cfg.C)
    if cfg.mask_rule == "band":
        for h in range(H):
            w = 1 + (h % 4)
            m = (dist <= w) | eye | (rng.random((nb, nb)) < 0.05)
            out[0, 0, h] = m
        return out
    if cfg.mask_rule == "target":
        # Per-head sparsity targets 0.40 + 0.50 * u**0.786 on a permuted uniform
        # grid over the block-sparse heads (mean 0.68, range about 0.42-0.89).
        if rep_flags is None:
            rep_flags = make_rep_flags(cfg)
        sparse = [h for h in range(H) if not rep_flags[0, 0, h]]
        perm = rng.permutation(len(sparse))
        target = np.full(H, 0.68)
        for i, h in enumerate(sparse):
            u = (perm[i] + 0.5) / len(sparse)
            target[h] = 0.40 + 0.50 * u ** 0.786
        for h in range(H):
            keep = 1.0 - target[h]
            w = _largest_band(dist, keep)
            out[0, 0, h] = _exact_count_mask(dist, w, keep, rng) | eye
        return out
    raise ValueError(cfg.mask_rule)


def make_rep_flags(cfg: LayerConfig, seed: int | None = None) -> np.ndarray:
    """uint8 [T, L, H]: 1 marks a head that takes the anchor-row path."""
    rng = np.random.Generator(np.random.PCG64(3000 + cfg.seed_base if seed is None else seed))
    flags = np.zeros((cfg.T, cfg.L, cfg.H), dtype=np.uint8)
    for t in range(cfg.T):
        for l in range(cfg.L):
            if cfg.mask_rule == "tiny":
                flags[t, l, 1:1 + cfg.n_rep] = 1      # head 0 sparse, head 1 repetitive
            elif cfg.n_rep:
                flags[t, l, rng.choice(cfg.H, size=cfg.n_rep, replace=False)] = 1
    return flags


def equally_spaced_anchor_rows(R: int, k: int) -> np.ndarray:
    """k equally spaced spatial rows: the centres of k equal segments of R rows.

    floor((2i+1) * R / (2k)) for i < k: rows {4, 12} of 16, {3, 9, 15, 21, 27}
    of 30 and {4, 13, 22, 31, 40} of 45.
    """
    i = np.arange(k, dtype=np.int64)
    return ((2 * i + 1) * R // (2 * k)).astype(np.int32)


@dataclass
class Workload:
    cfg: LayerConfig
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    masks: np.ndarray          # uint8 [T, L, H, nb, nb]
    rep_flags: np.ndarray      # uint8 [T, L, H]
    anchors: np.ndarray        # int32 [k]
    scale: float               # float32-representable softmax scale 1/sqrt(d)


def make_workload(key_or_cfg, with_data: bool = True) -> Workload:
    cfg = get_config(key_or_cfg) if isinstance(key_or_cfg, str) else key_or_cfg
    rep = make_rep_flags(cfg)
    masks = make_masks(cfg, rep_flags=rep)
    q = k = v = None
    if with_data:
        q, k, v = make_qkv(cfg)
    return Workload(cfg, q, k, v, masks, rep, equally_spaced_anchor_rows(cfg.R, cfg.n_anchor),
                    float(np.float32(1.0 / np.sqrt(cfg.d))))


def make_dictionary_workload(sparsity: float, rep_fraction: float, L: int = 40,
                             H: int = 40, seed_base: int = 5) -> tuple[LayerConfig, np.ndarray, np.ndarray]:
    """Full-step dictionary at the 480p shape: masks [1, L, H, nb, nb] and flags [1, L, H].

    Each (layer, head) draws a band width uniformly from [0, w*] where w* is the
    widest band within the sparsity target, then fills far blocks to the exact
    kept count. Sparsity 0 gives all-ones masks.
    """
    cfg = LayerConfig(
        key=f"wan480_dict_s{int(round(sparsity * 100))}_r{int(round(rep_fraction * 100))}",
        title=f"Wan-480p dictionary, {L} layers x {H} heads, sparsity {sparsity:.2f}, repetitive {rep_fraction:.2f}",
        H=H, F=21, R=30, C=52, d=128, B=128, dtype="bf16",
        n_rep=int(round(rep_fraction * H)), n_anchor=5, mask_rule="dict", k_bias=True,
        L=L, seed_base=seed_base)
    rng = np.random.Generator(np.random.PCG64(2000 + seed_base + int(round(1000 * sparsity))))
    nb = cfg.nb
    masks = np.zeros((1, L, H, nb, nb), dtype=np.uint8)
    if sparsity <= 0.0:
        masks[:] = 1
    else:
        dist = block_frame_distance(cfg.N, cfg.B, cfg.F, cfg.R, cfg.C)
        keep = 1.0 - sparsity
        wmax = _largest_band(dist, keep)
        eye = np.eye(nb, dtype=bool)
        for l in range(L):
            for h in range(H):
                w = int(rng.integers(0, wmax + 1))
                masks[0, l, h] = _exact_count_mask(dist, w, keep, rng) | eye
    rrng = np.random.Generator(np.random.PCG64(3000 + seed_base + int(round(100 * rep_fraction))))
    flags = np.zeros((1, L, H), dtype=np.uint8)
    for l in range(L):
        if cfg.n_rep:
            flags[0, l, rrng.choice(H, size=cfg.n_rep, replace=False)] = 1
    return cfg, masks, flags


# ---------------------------------------------------------------------------
# Calibration prompts (inputs of the offline block-energy calibration)
# ---------------------------------------------------------------------------
def make_calibration_prompts(N: int, d: int, F: int, R: int, C: int, H: int, n_prompts: int,
                             dtype: str = "bf16", seed: int = 4000, strength: float = 1.3):
    """Q and K [P, H, N, d] of P synthetic calibration prompts.

    Each prompt draws its own standard-normal Q and K noise; every prompt adds
    the same position code (per head: random frequencies along frame, row and
    column, as cos/sin pairs scaled by `strength`) to both Q and K. The code
    makes q_i . k_j large for nearby positions, so attention concentrates near
    the query as it does in video transformers, and the pattern is stable
    across prompts while the details are not. bf16 configs return uint16 bit
    patterns, fp32 configs float32 arrays.
    """
    if F * R * C != N:
        raise ValueError("N must equal F*R*C")
    code_rng = np.random.Generator(np.random.PCG64(seed))
    n = np.arange(N)
    pos = np.stack([n // (R * C), (n // C) % R, n % C]).astype(np.float64)     # [3, N]
    extent = np.array([F, R, C], dtype=np.float64)
    code = np.empty((H, N, d), dtype=np.float32)
    for h in range(H):
        axis = code_rng.integers(0, 3, size=d // 2)
        freq = code_rng.uniform(0.2, 3.0, size=d // 2) * 2.0 * np.pi / extent[axis] * code_rng.integers(1, 4, size=d // 2)
        ang = pos[axis] * freq[:, None]                                       # [d/2, N]
        code[h, :, 0::2] = (strength * np.cos(ang)).T
        code[h, :, 1::2] = (strength * np.sin(ang)).T
    qs, ks = [], []
    for p in range(n_prompts):
        rng = np.random.Generator(np.random.PCG64(seed + 1 + p))
        q = rng.standard_normal((H, N, d), dtype=np.float32) + code
        k = rng.standard_normal((H, N, d), dtype=np.float32) + code
        if dtype == "bf16":
            q, k = bf16_bits(q), bf16_bits(k)
        qs.append(q)
        ks.append(k)
    return np.stack(qs), np.stack(ks)


# ---------------------------------------------------------------------------
# Full denoising-run dictionary (all timesteps), generated on the GPU
# ---------------------------------------------------------------------------
def step_keep_fraction(T: int, L: int, H: int, seed: int = 6000) -> np.ndarray:
    """Target kept-block fraction per (t, l, h): denser at early (noisy) steps.

    0.55 at t = 0 falling linearly to 0.25 at the last step, times a per-(l, h)
    factor in [0.7, 1.3], clipped to [0.05, 0.95].
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    base = 0.55 - 0.30 * np.arange(T) / max(T - 1, 1)
    jitter = rng.uniform(0.7, 1.3, size=(1, L, H))
    return np.clip(base[:, None, None] * jitter, 0.05, 0.95)


def make_step_dictionary(key: str, T: int, L: int, H: int, device, seed: int = 6000):
    """Masks [T, L, H, nb, nb] (uint8 torch tensor on `device`) and flags [T, L, H] (numpy uint8).

    Per (t, l, h) with keep fraction k: blocks within a frame distance of
    round(0.4 * k * F) are kept (temporal band), every other block with
    probability 0.3 * k (far blocks), and the diagonal always; the realized
    kept fraction comes out close to k. The random draws
    come from a seeded torch generator on `device`, one (t, l) slice at a
    time. 20% of the heads of every (t, l) are flagged repetitive.
    """
    import torch
    cfg = get_config(key)
    nb = cfg.nb
    dist = torch.from_numpy(block_frame_distance(cfg.N, cfg.B, cfg.F, cfg.R, cfg.C)).to(device)
    eye = torch.eye(nb, dtype=torch.bool, device=device)
    keep = step_keep_fraction(T, L, H, seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    masks = torch.empty((T, L, H, nb, nb), dtype=torch.uint8, device=device)
    for t in range(T):
        for l in range(L):
            k = torch.from_numpy(keep[t, l]).to(device=device, dtype=torch.float32)
            band = torch.round(0.4 * k * cfg.F).to(torch.int64)
            u = torch.rand((H, nb, nb), generator=gen, device=device)
            m = (dist[None] <= band[:, None, None]) | (u < (0.3 * k)[:, None, None]) | eye[None]
            masks[t, l] = m.to(torch.uint8)
    frng = np.random.Generator(np.random.PCG64(seed + 1))
    flags = np.zeros((T, L, H), dtype=np.uint8)
    n_rep = max(1, H // 5)
    for t in range(T):
        for l in range(L):
            flags[t, l, frng.choice(H, size=n_rep, replace=False)] = 1
    return cfg, masks, flags
