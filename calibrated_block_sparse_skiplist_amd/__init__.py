"""CalibAtt inference hot path on MI355X (gfx950): the Python face of libcalibatt.so.

The names follow the C ABI in include/calibatt.h:

* ``calibatt_compile_skiplist`` / ``compile_skiplist`` -- block masks -> CSR skip lists on the GPU
* ``calibatt_compile_intervals`` / ``compile_intervals`` -- block masks -> runs of kept key blocks
* ``calibatt_compile_bitmap`` / ``compile_bitmap`` -- block masks -> one bit per key block
* ``calibatt_block_sparse_attn`` (``_iv``, ``_bm``) -- block-sparse attention over listed key blocks
* ``calibatt_anchor_attn`` -- anchor-row attention plus broadcast
* ``calibatt_layer_dispatch`` (``_iv``, ``_bm``) -- one layer-call, per-head choice of path
* ``calibatt_block_energy`` / ``calibatt_select_blocks`` / ``calibatt_keep_frequency`` -- offline
  calibration: block energies of a prompt, its top-tau selection, cross-prompt keep frequency
* ``calibatt_spatial_similarity`` / ``calibatt_repetition_flags`` -- offline calibration: spatial-row
  similarity to the nearest anchor row, and the per-head repetition flags
* ``calibatt_validate_skiplist`` / ``calibatt_validate_intervals`` / ``calibatt_set_checked_mode`` --
  checked mode: host-side validation of a list view before it reaches the kernels
* ``calibatt_block_energy_noalloc`` -- block energies for callers that cannot allocate device memory

All computation happens in the library's HIP kernels; this package only
marshals arguments. Importing it fails if the library has not been built.
"""
from ._lib import (BF16, F32, CalibattError, IntervalList, IntervalListView, SkipList, SkipListView,
                   calibatt_anchor_attn, calibatt_block_energy, calibatt_block_sparse_attn,
                   calibatt_block_sparse_attn_iv, calibatt_keep_frequency, calibatt_select_blocks,
                   calibatt_compile_intervals, calibatt_compile_skiplist, calibatt_layer_dispatch,
                   calibatt_layer_dispatch_iv, calibatt_repetition_flags, calibatt_set_kernel_events,
                   calibatt_spatial_similarity, calibatt_version,
                   calibatt_validate_skiplist, calibatt_validate_intervals, calibatt_set_checked_mode,
                   calibatt_block_energy_noalloc,
                   Bitmap, BitmapView, calibatt_compile_bitmap, calibatt_block_sparse_attn_bm,
                   calibatt_layer_dispatch_bm, calibatt_validate_bitmap, compile_bitmap,
                   compile_intervals, compile_skiplist, energy_work_bytes, last_error)

__all__ = ["BF16", "F32", "CalibattError", "IntervalList", "IntervalListView", "SkipList", "SkipListView",
           "calibatt_anchor_attn", "calibatt_block_energy", "calibatt_block_sparse_attn",
           "calibatt_block_sparse_attn_iv", "calibatt_keep_frequency", "calibatt_select_blocks",
           "calibatt_compile_intervals", "calibatt_compile_skiplist", "calibatt_layer_dispatch",
           "calibatt_layer_dispatch_iv", "calibatt_repetition_flags", "calibatt_set_kernel_events",
           "calibatt_spatial_similarity", "calibatt_version",
           "calibatt_validate_skiplist", "calibatt_validate_intervals", "calibatt_set_checked_mode",
           "calibatt_block_energy_noalloc",
           "Bitmap", "BitmapView", "calibatt_compile_bitmap", "calibatt_block_sparse_attn_bm",
           "calibatt_layer_dispatch_bm", "calibatt_validate_bitmap", "compile_bitmap",
           "compile_intervals", "compile_skiplist", "energy_work_bytes", "last_error"]
