"""ctypes binding of libcalibatt.so (the C ABI in include/calibatt.h).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels. torch supplies device buffers (``tensor.data_ptr()``) and the
stream handle; nothing here computes attention or skip lists. There is no
fallback: if the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# CALIBATT_LIB selects another build of the same library (the host-sanitized
# one, for CPU runs of the host logic); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("CALIBATT_LIB") or os.path.join(_HERE, "libcalibatt.so")

OK, ERR_INVALID_ARG, ERR_CAPACITY, ERR_HIP, ERR_UNSUPPORTED = 0, 1, 2, 3, 4
BF16, F32 = 0, 1
MAX_HEADS, MAX_ANCHORS, MAX_NB = 256, 64, 4096

EXPORTED = (
    "calibatt_compile_skiplist", "calibatt_block_sparse_attn", "calibatt_anchor_attn",
    "calibatt_layer_dispatch", "calibatt_compile_intervals", "calibatt_block_sparse_attn_iv",
    "calibatt_layer_dispatch_iv", "calibatt_block_energy", "calibatt_select_blocks", "calibatt_keep_frequency",
    "calibatt_spatial_similarity", "calibatt_repetition_flags",
    "calibatt_last_error", "calibatt_set_kernel_events", "calibatt_version",
    "calibatt_validate_skiplist", "calibatt_validate_intervals", "calibatt_set_checked_mode",
    "calibatt_block_energy_noalloc",
    "calibatt_compile_bitmap", "calibatt_block_sparse_attn_bm", "calibatt_layer_dispatch_bm",
    "calibatt_validate_bitmap",
)
NOALLOC_SCRATCH_BYTES = 256 << 20


class CalibattError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"calibatt status {status}: {message}")
        self.status = status


class SkipListView(ctypes.Structure):
    """Mirror of calibatt_skiplist_t."""
    _fields_ = [("T", ctypes.c_int32), ("L", ctypes.c_int32), ("H", ctypes.c_int32),
                ("N", ctypes.c_int32), ("B", ctypes.c_int32), ("nb", ctypes.c_int32),
                ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p), ("order", ctypes.c_void_p)]


class IntervalListView(ctypes.Structure):
    """Mirror of calibatt_intervals_t."""
    _fields_ = [("T", ctypes.c_int32), ("L", ctypes.c_int32), ("H", ctypes.c_int32),
                ("N", ctypes.c_int32), ("B", ctypes.c_int32), ("nb", ctypes.c_int32),
                ("iv_ptr", ctypes.c_void_p), ("iv", ctypes.c_void_p), ("order", ctypes.c_void_p)]


class BitmapView(ctypes.Structure):
    """Mirror of calibatt_bitmap_t."""
    _fields_ = [("T", ctypes.c_int32), ("L", ctypes.c_int32), ("H", ctypes.c_int32),
                ("N", ctypes.c_int32), ("B", ctypes.c_int32), ("nb", ctypes.c_int32), ("words", ctypes.c_int32),
                ("bits", ctypes.c_void_p)]


def _load():
    # torch ships its own HIP runtime (same soname as /opt/rocm's). Loading it
    # first makes the library bind to that runtime, so device pointers and
    # streams coming from torch are valid in the library's HIP calls.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "or python -m calibrated_block_sparse_skiplist_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.calibatt_compile_skiplist.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, i64, vp,
                                              ctypes.POINTER(i64), vp]
    lib.calibatt_compile_skiplist.restype = i32
    lib.calibatt_block_sparse_attn.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                               ctypes.POINTER(SkipListView), i32, i32, vp, i32, vp]
    lib.calibatt_block_sparse_attn.restype = i32
    lib.calibatt_anchor_attn.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                         i32, i32, i32, vp, i32, vp, i32, vp]
    lib.calibatt_anchor_attn.restype = i32
    lib.calibatt_layer_dispatch.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                            ctypes.POINTER(SkipListView), i32, i32, vp,
                                            i32, i32, i32, vp, i32, vp]
    lib.calibatt_layer_dispatch.restype = i32
    lib.calibatt_compile_intervals.argtypes = lib.calibatt_compile_skiplist.argtypes
    lib.calibatt_compile_intervals.restype = i32
    lib.calibatt_block_sparse_attn_iv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                                  ctypes.POINTER(IntervalListView), i32, i32, vp, i32, vp]
    lib.calibatt_block_sparse_attn_iv.restype = i32
    lib.calibatt_layer_dispatch_iv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                               ctypes.POINTER(IntervalListView), i32, i32, vp,
                                               i32, i32, i32, vp, i32, vp]
    lib.calibatt_layer_dispatch_iv.restype = i32
    lib.calibatt_block_energy.argtypes = [vp, vp, i32, i32, i32, i32, f32, i32, vp, vp, i32, vp, i64, vp]
    lib.calibatt_block_energy.restype = i32
    lib.calibatt_select_blocks.argtypes = [vp, i64, i32, f32, vp, vp, vp]
    lib.calibatt_select_blocks.restype = i32
    lib.calibatt_keep_frequency.argtypes = [vp, i64, i32, f32, vp, vp]
    lib.calibatt_keep_frequency.restype = i32
    lib.calibatt_spatial_similarity.argtypes = [vp, vp, i32, i32, i32, i32, f32, i32, i32, i32, vp, i32, vp, vp,
                                                i32, vp]
    lib.calibatt_spatial_similarity.restype = i32
    lib.calibatt_repetition_flags.argtypes = [vp, i32, i32, i32, i32, vp, i32, f32, vp, vp, vp]
    lib.calibatt_repetition_flags.restype = i32
    lib.calibatt_last_error.argtypes = []
    lib.calibatt_last_error.restype = ctypes.c_char_p
    lib.calibatt_set_kernel_events.argtypes = [vp, vp]
    lib.calibatt_set_kernel_events.restype = None
    lib.calibatt_version.argtypes = []
    lib.calibatt_version.restype = i32
    lib.calibatt_validate_skiplist.argtypes = [ctypes.POINTER(SkipListView), i32, i32, i32, vp]
    lib.calibatt_validate_skiplist.restype = i32
    lib.calibatt_validate_intervals.argtypes = [ctypes.POINTER(IntervalListView), i32, i32, i32, vp]
    lib.calibatt_validate_intervals.restype = i32
    lib.calibatt_set_checked_mode.argtypes = [i32]
    lib.calibatt_set_checked_mode.restype = None
    lib.calibatt_block_energy_noalloc.argtypes = [vp, vp, i32, i32, i32, i32, f32, i32, vp, vp, i32, vp]
    lib.calibatt_block_energy_noalloc.restype = i32
    lib.calibatt_compile_bitmap.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp]
    lib.calibatt_compile_bitmap.restype = i32
    lib.calibatt_block_sparse_attn_bm.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                                  ctypes.POINTER(BitmapView), i32, i32, vp, i32, vp]
    lib.calibatt_block_sparse_attn_bm.restype = i32
    lib.calibatt_layer_dispatch_bm.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                               ctypes.POINTER(BitmapView), i32, i32, vp,
                                               i32, i32, i32, vp, i32, vp]
    lib.calibatt_layer_dispatch_bm.restype = i32
    lib.calibatt_validate_bitmap.argtypes = [ctypes.POINTER(BitmapView), i32, i32, i32, vp]
    lib.calibatt_validate_bitmap.restype = i32
    return lib


lib = _load()


def last_error() -> str:
    return lib.calibatt_last_error().decode()


def _check(status: int) -> None:
    if status != OK:
        raise CalibattError(status, last_error())


def _ptr(t) -> int | None:
    """Device address of a torch tensor (None for None)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _host_i32(values):
    if values is None:
        return None, 0
    arr = np.ascontiguousarray(np.asarray(values, dtype=np.int32))
    return arr, len(arr)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"unsupported dtype {t.dtype}")


@dataclass
class SkipList:
    """A compiled dictionary held in device tensors (row_ptr, col_idx, order)."""
    T: int
    L: int
    H: int
    N: int
    B: int
    nb: int
    row_ptr: object
    col_idx: object
    order: object
    nnz: int

    def view(self) -> SkipListView:
        return SkipListView(self.T, self.L, self.H, self.N, self.B, self.nb,
                            _ptr(self.row_ptr), _ptr(self.col_idx),
                            _ptr(self.order) if self.order is not None else None)


def calibatt_compile_skiplist(masks, T, L, H, N, B, row_ptr, col_idx, col_capacity, order, stream=None) -> int:
    """Raw call: device tensors in, returns nnz (raises on error, CAPACITY included)."""
    nnz = ctypes.c_int64(-1)
    st = lib.calibatt_compile_skiplist(_ptr(masks), T, L, H, N, B, _ptr(row_ptr), _ptr(col_idx),
                                       int(col_capacity), _ptr(order), ctypes.byref(nnz), _stream(stream))
    if st == ERR_CAPACITY:
        raise CalibattError(st, last_error() + f" (nnz={nnz.value})")
    _check(st)
    return nnz.value


def compile_skiplist(masks, N: int, B: int, with_order: bool = True, stream=None) -> SkipList:
    """Compile uint8 device masks [T, L, H, nb, nb] into a SkipList (allocates with torch)."""
    import torch
    T, L, H, nb, nb2 = masks.shape
    if nb != nb2 or nb != -(-N // B):
        raise ValueError("masks must be [T, L, H, nb, nb] with nb = ceil(N/B)")
    dev = masks.device
    rows = T * L * H * nb
    row_ptr = torch.empty(rows + 1, dtype=torch.int64, device=dev)
    nnz = calibatt_compile_skiplist(masks, T, L, H, N, B, row_ptr, None, 0, None, stream)
    col_idx = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
    order = torch.empty(rows, dtype=torch.int32, device=dev) if with_order else None
    calibatt_compile_skiplist(masks, T, L, H, N, B, row_ptr, col_idx, col_idx.numel(), order, stream)
    return SkipList(T, L, H, N, B, nb, row_ptr, col_idx, order, nnz)


@dataclass
class IntervalList:
    """A compiled dictionary in interval form held in device tensors (iv_ptr, iv, order)."""
    T: int
    L: int
    H: int
    N: int
    B: int
    nb: int
    iv_ptr: object
    iv: object
    order: object
    n_iv: int

    def view(self) -> IntervalListView:
        return IntervalListView(self.T, self.L, self.H, self.N, self.B, self.nb,
                                _ptr(self.iv_ptr), _ptr(self.iv),
                                _ptr(self.order) if self.order is not None else None)


def calibatt_compile_intervals(masks, T, L, H, N, B, iv_ptr, iv, iv_capacity, order, stream=None) -> int:
    """Raw call: device tensors in, returns the run count (raises on error, CAPACITY included)."""
    n_iv = ctypes.c_int64(-1)
    st = lib.calibatt_compile_intervals(_ptr(masks), T, L, H, N, B, _ptr(iv_ptr), _ptr(iv),
                                        int(iv_capacity), _ptr(order), ctypes.byref(n_iv), _stream(stream))
    if st == ERR_CAPACITY:
        raise CalibattError(st, last_error() + f" (n_iv={n_iv.value})")
    _check(st)
    return n_iv.value


def compile_intervals(masks, N: int, B: int, with_order: bool = True, stream=None) -> IntervalList:
    """Compile uint8 device masks [T, L, H, nb, nb] into an IntervalList (allocates with torch).

    iv holds the packed runs as int32 tensor storage (bit pattern lo | hi << 16).
    """
    import torch
    T, L, H, nb, nb2 = masks.shape
    if nb != nb2 or nb != -(-N // B):
        raise ValueError("masks must be [T, L, H, nb, nb] with nb = ceil(N/B)")
    dev = masks.device
    rows = T * L * H * nb
    iv_ptr = torch.empty(rows + 1, dtype=torch.int64, device=dev)
    n_iv = calibatt_compile_intervals(masks, T, L, H, N, B, iv_ptr, None, 0, None, stream)
    iv = torch.empty(max(n_iv, 1), dtype=torch.int32, device=dev)
    order = torch.empty(rows, dtype=torch.int32, device=dev) if with_order else None
    calibatt_compile_intervals(masks, T, L, H, N, B, iv_ptr, iv, iv.numel(), order, stream)
    return IntervalList(T, L, H, N, B, nb, iv_ptr, iv, order, n_iv)


@dataclass
class Bitmap:
    """A compiled dictionary in bitmap form held in a device tensor (bits: int64 storage of the uint64 words)."""
    T: int
    L: int
    H: int
    N: int
    B: int
    nb: int
    words: int
    bits: object

    def view(self) -> BitmapView:
        return BitmapView(self.T, self.L, self.H, self.N, self.B, self.nb, self.words, _ptr(self.bits))


def calibatt_compile_bitmap(masks, T, L, H, N, B, bits, stream=None) -> None:
    """Raw call: device masks in, bits (device tensor of T*L*H*nb*ceil(nb/64) 64-bit words) written."""
    _check(lib.calibatt_compile_bitmap(_ptr(masks), T, L, H, N, B, _ptr(bits), _stream(stream)))


def compile_bitmap(masks, N: int, B: int, stream=None) -> Bitmap:
    """Compile uint8 device masks [T, L, H, nb, nb] into a Bitmap (allocates with torch)."""
    import torch
    T, L, H, nb, nb2 = masks.shape
    if nb != nb2 or nb != -(-N // B):
        raise ValueError("masks must be [T, L, H, nb, nb] with nb = ceil(N/B)")
    words = -(-nb // 64)
    bits = torch.empty((T * L * H * nb, words), dtype=torch.int64, device=masks.device)
    calibatt_compile_bitmap(masks, T, L, H, N, B, bits, stream)
    return Bitmap(T, L, H, N, B, nb, words, bits)


def calibatt_block_sparse_attn_bm(q, k, v, o, lse, bm: Bitmap, t: int, l: int, heads=None,
                                  scale: float | None = None, stream=None) -> None:
    H, N, d = q.shape
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else scale
    harr, nh = _host_i32(heads)
    view = bm.view()
    _check(lib.calibatt_block_sparse_attn_bm(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), H, N, d,
                                             _dtype_code(q), scale, ctypes.byref(view), t, l,
                                             harr.ctypes.data if harr is not None else None, nh,
                                             _stream(stream)))


def calibatt_layer_dispatch_bm(q, k, v, o, lse, bm: Bitmap, t: int, l: int, rep_flags, F: int, R: int,
                               C: int, anchor_rows, scale: float | None = None, stream=None) -> None:
    H, N, d = q.shape
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else scale
    flags = np.ascontiguousarray(np.asarray(rep_flags, dtype=np.uint8))
    if flags.shape != (bm.T, bm.L, bm.H):
        raise ValueError("rep_flags must be [T, L, H] of the dictionary")
    aarr, ka = _host_i32(anchor_rows)
    view = bm.view()
    _check(lib.calibatt_layer_dispatch_bm(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), H, N, d,
                                          _dtype_code(q), scale, ctypes.byref(view), t, l,
                                          flags.ctypes.data, F, R, C, aarr.ctypes.data, ka, _stream(stream)))


def calibatt_validate_bitmap(bm: Bitmap, t: int = -1, l: int = -1, stream=None) -> None:
    """Checked mode for a Bitmap (device tensor)."""
    view = bm.view()
    _check(lib.calibatt_validate_bitmap(ctypes.byref(view), t, l, 0, _stream(stream)))


def calibatt_block_sparse_attn(q, k, v, o, lse, sl: SkipList, t: int, l: int, heads=None,
                               scale: float | None = None, stream=None) -> None:
    H, N, d = q.shape
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else scale
    harr, nh = _host_i32(heads)
    view = sl.view()
    _check(lib.calibatt_block_sparse_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), H, N, d,
                                          _dtype_code(q), scale, ctypes.byref(view), t, l,
                                          harr.ctypes.data if harr is not None else None, nh,
                                          _stream(stream)))


def calibatt_block_sparse_attn_iv(q, k, v, o, lse, il: IntervalList, t: int, l: int, heads=None,
                                  scale: float | None = None, stream=None) -> None:
    H, N, d = q.shape
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else scale
    harr, nh = _host_i32(heads)
    view = il.view()
    _check(lib.calibatt_block_sparse_attn_iv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), H, N, d,
                                             _dtype_code(q), scale, ctypes.byref(view), t, l,
                                             harr.ctypes.data if harr is not None else None, nh,
                                             _stream(stream)))


def calibatt_anchor_attn(q, k, v, o, lse, F: int, R: int, C: int, anchor_rows, heads=None,
                         scale: float | None = None, stream=None) -> None:
    H, N, d = q.shape
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else scale
    aarr, ka = _host_i32(anchor_rows)
    harr, nh = _host_i32(heads)
    _check(lib.calibatt_anchor_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), H, N, d,
                                    _dtype_code(q), scale, F, R, C, aarr.ctypes.data, ka,
                                    harr.ctypes.data if harr is not None else None, nh, _stream(stream)))


def calibatt_layer_dispatch(q, k, v, o, lse, sl: SkipList, t: int, l: int, rep_flags, F: int, R: int,
                            C: int, anchor_rows, scale: float | None = None, stream=None) -> None:
    H, N, d = q.shape
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else scale
    flags = np.ascontiguousarray(np.asarray(rep_flags, dtype=np.uint8))
    if flags.shape != (sl.T, sl.L, sl.H):
        raise ValueError("rep_flags must be [T, L, H] of the dictionary")
    aarr, ka = _host_i32(anchor_rows)
    view = sl.view()
    _check(lib.calibatt_layer_dispatch(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), H, N, d,
                                       _dtype_code(q), scale, ctypes.byref(view), t, l,
                                       flags.ctypes.data, F, R, C, aarr.ctypes.data, ka, _stream(stream)))


def calibatt_layer_dispatch_iv(q, k, v, o, lse, il: IntervalList, t: int, l: int, rep_flags, F: int, R: int,
                               C: int, anchor_rows, scale: float | None = None, stream=None) -> None:
    H, N, d = q.shape
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else scale
    flags = np.ascontiguousarray(np.asarray(rep_flags, dtype=np.uint8))
    if flags.shape != (il.T, il.L, il.H):
        raise ValueError("rep_flags must be [T, L, H] of the dictionary")
    aarr, ka = _host_i32(anchor_rows)
    view = il.view()
    _check(lib.calibatt_layer_dispatch_iv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), H, N, d,
                                          _dtype_code(q), scale, ctypes.byref(view), t, l,
                                          flags.ctypes.data, F, R, C, aarr.ctypes.data, ka, _stream(stream)))


def energy_work_bytes(N: int, B: int, heads: int = 1) -> int:
    """Workspace bytes for a one-pass calibatt_block_energy launch of `heads` heads."""
    nb = -(-N // B)
    return nb * nb * B * 4 * heads


def calibatt_block_energy(q, k, energy, B: int, heads=None, scale: float | None = None, work=None,
                          stream=None) -> None:
    """Block energies [H, nb, nb] (float32 device tensor) of one prompt's q, k [H, N, d].

    work: optional device tensor used as the one-pass workspace (its whole storage).
    """
    H, N, d = q.shape
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else scale
    harr, nh = _host_i32(heads)
    wbytes = 0 if work is None else work.numel() * work.element_size()
    _check(lib.calibatt_block_energy(_ptr(q), _ptr(k), H, N, d, _dtype_code(q), scale, B, _ptr(energy),
                                     harr.ctypes.data if harr is not None else None, nh, _ptr(work), wbytes,
                                     _stream(stream)))


def calibatt_block_energy_noalloc(q, k, energy, B: int, heads=None, scale: float | None = None,
                                  stream=None) -> None:
    """calibatt_block_energy for callers that cannot allocate: the workspace is the library's own
    per-GPU scratch (calls overlapping on one GPU race)."""
    H, N, d = q.shape
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else scale
    harr, nh = _host_i32(heads)
    _check(lib.calibatt_block_energy_noalloc(_ptr(q), _ptr(k), H, N, d, _dtype_code(q), scale, B, _ptr(energy),
                                             harr.ctypes.data if harr is not None else None, nh, _stream(stream)))


def calibatt_select_blocks(energy, tau: float, mask=None, counts=None, stream=None) -> None:
    """Top-tau selection over the last axis of a float32 energy tensor; writes mask and/or adds to counts."""
    nb = energy.shape[-1]
    rows = energy.numel() // nb
    _check(lib.calibatt_select_blocks(_ptr(energy), rows, nb, float(tau), _ptr(mask), _ptr(counts),
                                      _stream(stream)))


def calibatt_keep_frequency(counts, n_prompts: int, rho: float, mask, stream=None) -> None:
    """mask = counts / n_prompts >= rho (elementwise, exact)."""
    _check(lib.calibatt_keep_frequency(_ptr(counts), counts.numel(), n_prompts, float(rho), _ptr(mask),
                                       _stream(stream)))


def calibatt_spatial_similarity(q, k, F: int, R: int, C: int, anchor_rows, row_sim, heads=None,
                                scale: float | None = None, stream=None) -> None:
    """Row similarities [H, F, R] (float32 device tensor) of one prompt."""
    H, N, d = q.shape
    scale = float(np.float32(1.0 / np.sqrt(d))) if scale is None else scale
    aarr, ka = _host_i32(anchor_rows)
    harr, nh = _host_i32(heads)
    _check(lib.calibatt_spatial_similarity(_ptr(q), _ptr(k), H, N, d, _dtype_code(q), scale, F, R, C,
                                           aarr.ctypes.data, ka, _ptr(row_sim),
                                           harr.ctypes.data if harr is not None else None, nh, _stream(stream)))


def calibatt_repetition_flags(row_sim, anchor_rows, threshold: float, flags=None, mean=None, stream=None) -> None:
    """row_sim: float32 device tensor [P, H, F, R]; writes flags (uint8 [H]) and/or mean (float32 [H])."""
    P, H, F, R = row_sim.shape
    aarr, ka = _host_i32(anchor_rows)
    _check(lib.calibatt_repetition_flags(_ptr(row_sim), P, H, F, R, aarr.ctypes.data, ka, float(threshold),
                                         _ptr(flags), _ptr(mean), _stream(stream)))


def calibatt_set_kernel_events(begin, end) -> None:
    """begin/end: raw hipEvent_t handles (ints) or None."""
    lib.calibatt_set_kernel_events(begin, end)


def calibatt_version() -> int:
    return lib.calibatt_version()


def calibatt_validate_skiplist(sl: SkipList, t: int = -1, l: int = -1, stream=None) -> None:
    """Checked mode: validate a SkipList (device tensors) for record (t, l), or all of it (t = l = -1).
    Raises CalibattError on a malformed view."""
    view = sl.view()
    _check(lib.calibatt_validate_skiplist(ctypes.byref(view), t, l, 0, _stream(stream)))


def calibatt_validate_intervals(il: IntervalList, t: int = -1, l: int = -1, stream=None) -> None:
    """Checked mode for an IntervalList (device tensors)."""
    view = il.view()
    _check(lib.calibatt_validate_intervals(ctypes.byref(view), t, l, 0, _stream(stream)))


def calibatt_set_checked_mode(enabled: bool) -> None:
    """When enabled (this thread), the attention calls validate their record's lists before launching."""
    lib.calibatt_set_checked_mode(1 if enabled else 0)
