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
