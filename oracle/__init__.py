"""CPU oracle for the CalibAtt layer hot path. TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check (``__graft_entry__.smoke``) and the CPU-baseline
leg of ``bench.py`` may import or run anything in this package. The product
path (the HIP library ``libcalibatt.so`` and its Python binding) never imports,
calls or links it, and the two share no code: no helpers, no constants, no
pre- or post-processing. Both consume the same seeded inputs from the
``workloads`` module, which holds none of the method's arithmetic.

What is computed, and where it is stated
----------------------------------------
Citations name the web page and the section on it:

* [Notes] papernotes.org notes on "Accelerating Text-to-Video Generation with
  Calibrated Sparse Attention" (ECCV 2026 notes).
* [Abstract] the arXiv abstract of the same paper (2603.05503), as shown on
  the mlsanity.com paper index page.

``skiplist.compile_skiplist``
    Each calibrated binary block mask becomes, for every query block, the list
    of key blocks to compute ([Notes] Key Design 4, "Precompiled dual-path
    execution"; Highlights). The lists are indexed by timestep, layer and head
    ([Notes] Overall Architecture). Encoding read here: CSR, ascending key
    blocks, plus a per-record heaviest-first order of query blocks.

``skiplist.compile_intervals``
    The same selection in the pages' own encoding, contiguous key-block
    intervals per query block ([Notes] Key Design 4; Highlights): one
    half-open [lo, hi) pair per maximal run of kept key blocks.

``skiplist.compile_bitmap``
    The same selection packed as one bit per key block (ceil(nb/64) 64-bit
    words per query block, bit c % 64 of word c // 64), for dictionaries held
    in the least memory.

``attention.block_sparse_head``
    Retained connections are computed from the current input's Q, K and V and
    unselected ones are skipped ([Notes] Overall Architecture; [Abstract]).
    That is exactly softmax attention restricted to the kept key blocks of each
    query block, written out in fp64 from its definition.

``attention.anchor_head``
    Repetitive heads compute attention only for a few anchor spatial rows per
    frame, against all keys and values, and broadcast each anchor's output to
    its nearest spatial rows in the same frame ([Notes] Key Design 3, "Spatial
    repetition detection"; Key Design 4; A Worked Example).

``attention.layer_forward``
    The record for (timestep, layer, head) selects the path per head: the
    repetition flag chooses anchor rows, otherwise the block-sparse path; the
    two paths are alternatives ([Notes] Key Design 4).

Pins
----
Every function above is pinned by ``tests/test_oracle_*.py`` against results
fixed by the pages or by mathematics, independent of this code: brute-force
enumeration of skip lists, hand-derived fixtures under ``tests/golden/``,
PyTorch's scaled-dot-product attention (fp64, CPU) with an explicit token mask,
scipy's logsumexp, closed forms (Q = 0, constant V), exact zeros outside kept
blocks, row sums of one, and the identical-rows property of the anchor rule.
There are no printed attention values on the pages, so beyond these pins the
attention outputs have no external worked example; no function here is
"parity unpinned".

``calibration.block_energy`` / ``select_blocks`` / ``keep_counts`` / ``keep_frequency_mask``
    The offline calibration that produces the masks: block energies of the
    post-softmax attention (Eq. 5, [Notes] Key Design 1), the shortest
    descending prefix reaching the energy threshold per query block (same
    section), and the cross-prompt keep frequency thresholded at rho
    (Eq. 8-9, [Notes] Key Design 2; A Worked Example).

``repetition.row_similarity`` / ``repetition_mean`` / ``repetition_flags``
    The spatial-repetition branch of calibration ([Notes] Key Design 3): the
    cosine similarity of each spatial row's flattened attention with its
    nearest anchor row's, averaged over frames, rows and prompts, and the
    head flagged when the mean exceeds the threshold.

Readings of points the pages leave open are listed in the module docstrings
where they are applied (empty rows, partial last block, anchor ties, token
order, broadcast unit).
"""
from .skiplist import (bitmap_to_dense, compile_bitmap, compile_intervals, compile_skiplist, intervals_to_dense,
                       skiplist_to_dense)
from .attention import (block_sparse_head, anchor_head, nearest_anchor_rows,
                        layer_forward, block_tokens)
from .calibration import block_energy, keep_counts, keep_frequency_mask, select_blocks
from .repetition import repetition_flags, repetition_mean, row_similarity

__all__ = ["bitmap_to_dense", "compile_bitmap", "compile_intervals", "compile_skiplist", "intervals_to_dense", "skiplist_to_dense", "block_sparse_head", "anchor_head",
           "nearest_anchor_rows", "layer_forward", "block_tokens", "block_energy", "keep_counts",
           "keep_frequency_mask", "select_blocks", "repetition_flags", "repetition_mean", "row_similarity"]
