"""Skip-list compilation oracle. TEST INFRASTRUCTURE ONLY (see package docstring).

[Notes] Key Design 4 ("Precompiled dual-path execution"): each binary block
mask of a (timestep, layer, head) record is turned into a read-only list, for
every query block, of the key blocks to compute; the lists live on the GPU
before generation. [Notes] Overall Architecture: the dictionaries are indexed
by timestep, layer and head.

Readings applied here (the pages leave them open):

* Mask layout: uint8 [T, L, H, nb, nb], entry [t, l, h, r, c] nonzero means
  "compute query block r against key block c".
* Encoding: CSR. Rows are flattened as ((t*L + l)*H + h)*nb + r. row_ptr has
  one more entry than there are rows, starts at 0 and counts kept blocks;
  col_idx lists each row's kept key blocks in ascending order. (The pages
  describe contiguous key-block intervals; an ascending index list names the
  same set of blocks.)
* order: for each record, the query blocks sorted by descending kept count,
  ties by ascending block index (heaviest first, for load balancing).
* Bitmap form: the same selection as nb bits per row (bit c of the row set
  iff key block c is kept), in W = ceil(nb/64) 64-bit words per row, key
  block c in bit c % 64 of word c // 64; the bits past nb are zero.
"""
from __future__ import annotations

import numpy as np


def compile_skiplist(masks: np.ndarray):
    """Return (row_ptr int64 [rows+1], col_idx int32 [nnz], order int32 [rows]).

    rows = T*L*H*nb. The definition, step by step:
    1. flatten the masks to one row per (record, query block);
    2. count each row's nonzero entries; row_ptr is the running sum of counts;
    3. col_idx concatenates, row after row, the column indices of the nonzero
       entries in ascending order (row-major enumeration of the nonzeros);
    4. within each record, order lists query blocks by (-count, index).
    """
    masks = np.asarray(masks)
    if masks.ndim != 5 or masks.shape[3] != masks.shape[4]:
        raise ValueError("masks must be [T, L, H, nb, nb]")
    T, L, H, nb, _ = masks.shape
    rows = masks.reshape(T * L * H * nb, nb) != 0

    counts = rows.sum(axis=1).astype(np.int64)
    row_ptr = np.zeros(rows.shape[0] + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)

    _, cols = np.nonzero(rows)          # row-major: rows in order, columns ascending
    col_idx = cols.astype(np.int32)

    order = np.empty(rows.shape[0], dtype=np.int32)
    for rec in range(T * L * H):
        cnt = counts[rec * nb:(rec + 1) * nb]
        ranked = sorted(range(nb), key=lambda r: (-int(cnt[r]), r))
        order[rec * nb:(rec + 1) * nb] = ranked
    return row_ptr, col_idx, order


def skiplist_to_dense(row_ptr: np.ndarray, col_idx: np.ndarray, T: int, L: int, H: int,
                      nb: int) -> np.ndarray:
    """Inverse of the encoding: rebuild the uint8 [T, L, H, nb, nb] keep mask."""
    out = np.zeros((T * L * H * nb, nb), dtype=np.uint8)
    for row in range(T * L * H * nb):
        out[row, col_idx[row_ptr[row]:row_ptr[row + 1]]] = 1
    return out.reshape(T, L, H, nb, nb)


def compile_intervals(masks: np.ndarray):
    """Interval form of the skip list: (iv_ptr int64 [rows+1], iv int32 [n_iv, 2], order int32 [rows]).

    [Notes] Key Design 4 and Highlights: each binary mask becomes a read-only
    list of contiguous key-block intervals per query block. Reading: one
    interval per maximal run of kept key blocks, as the half-open pair
    [lo, hi) (blocks lo .. hi-1 kept, lo-1 and hi not kept or outside the
    row), runs in ascending order. Maximal runs make the encoding unique.
    iv_ptr is the running sum of the per-row run counts. order is the same
    heaviest-first order as the index-list form, by kept-block count.

    Written from the definition of a run: walk each row once, open a run at a
    kept block whose left neighbour is not kept, close it after a kept block
    whose right neighbour is not kept.
    """
    masks = np.asarray(masks)
    if masks.ndim != 5 or masks.shape[3] != masks.shape[4]:
        raise ValueError("masks must be [T, L, H, nb, nb]")
    T, L, H, nb, _ = masks.shape
    rows = masks.reshape(T * L * H * nb, nb) != 0

    runs = []
    iv_ptr = np.zeros(rows.shape[0] + 1, dtype=np.int64)
    for row in range(rows.shape[0]):
        keep = rows[row]
        lo = None
        for c in range(nb):
            if keep[c] and (c == 0 or not keep[c - 1]):
                lo = c
            if keep[c] and (c == nb - 1 or not keep[c + 1]):
                runs.append((lo, c + 1))
        iv_ptr[row + 1] = len(runs)
    iv = np.array(runs, dtype=np.int32).reshape(-1, 2)

    counts = rows.sum(axis=1)
    order = np.empty(rows.shape[0], dtype=np.int32)
    for rec in range(T * L * H):
        cnt = counts[rec * nb:(rec + 1) * nb]
        order[rec * nb:(rec + 1) * nb] = sorted(range(nb), key=lambda r: (-int(cnt[r]), r))
    return iv_ptr, iv, order


def intervals_to_dense(iv_ptr: np.ndarray, iv: np.ndarray, T: int, L: int, H: int, nb: int) -> np.ndarray:
    """Inverse of the interval encoding: rebuild the uint8 [T, L, H, nb, nb] keep mask."""
    out = np.zeros((T * L * H * nb, nb), dtype=np.uint8)
    for row in range(T * L * H * nb):
        for lo, hi in iv[iv_ptr[row]:iv_ptr[row + 1]]:
            out[row, lo:hi] = 1
    return out.reshape(T, L, H, nb, nb)


def compile_bitmap(masks: np.ndarray) -> np.ndarray:
    """Bitmap form of the skip list: uint64 [rows, W], W = ceil(nb / 64).

    The selection of each row ([Notes] Key Design 4: per query block, the key
    blocks to compute) as one bit per key block: bit (c % 64) of word (c // 64)
    is 1 exactly when mask[row][c] != 0; bits at positions >= nb stay 0. Rows
    are flattened as in compile_skiplist. Written from that definition: start
    from all-zero words and set the bit of every kept block, column by column.
    """
    masks = np.asarray(masks)
    if masks.ndim != 5 or masks.shape[3] != masks.shape[4]:
        raise ValueError("masks must be [T, L, H, nb, nb]")
    T, L, H, nb, _ = masks.shape
    rows = masks.reshape(T * L * H * nb, nb) != 0
    words = (nb + 63) // 64
    bits = np.zeros((rows.shape[0], words), dtype=np.uint64)
    for c in range(nb):
        bits[:, c // 64] |= rows[:, c].astype(np.uint64) << np.uint64(c % 64)
    return bits


def bitmap_to_dense(bits: np.ndarray, T: int, L: int, H: int, nb: int) -> np.ndarray:
    """Inverse of the bitmap encoding: rebuild the uint8 [T, L, H, nb, nb] keep mask."""
    bits = np.asarray(bits, dtype=np.uint64)
    out = np.zeros((T * L * H * nb, nb), dtype=np.uint8)
    for c in range(nb):
        out[:, c] = ((bits[:, c // 64] >> np.uint64(c % 64)) & np.uint64(1)).astype(np.uint8)
    return out.reshape(T, L, H, nb, nb)
