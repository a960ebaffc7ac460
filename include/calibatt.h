/*
 * calibatt.h -- C ABI of libcalibatt.so, the MI355X (gfx950) inference hot path
 * of calibrated block-sparse attention (CalibAtt) for one transformer layer.
 *
 * What the method computes (web pages this library follows):
 *  [Notes]    papernotes.org notes on "Accelerating Text-to-Video Generation with
 *             Calibrated Sparse Attention" (ECCV 2026 notes).
 *  [Abstract] the paper's arXiv abstract (2603.05503) on its mlsanity.com page.
 *
 * Offline calibration produces, per (timestep, layer, head), a binary mask over
 * 128x128 FlashAttention blocks and a spatial-repetition flag ([Notes] Overall
 * Architecture). Each mask becomes a read-only skip list, per query block, of
 * the key blocks to compute, resident on the GPU ([Notes] Key Design 4). At
 * inference the record selected by (t, l, h) drives one of two alternative
 * paths per head: block-sparse attention over the listed blocks for
 * non-repetitive heads, or anchor-row attention plus broadcast to the
 * neighbouring spatial rows for repetitive heads ([Notes] Key Designs 3 and 4).
 *
 * Conventions shared by every entry point
 *  - All array pointers are device pointers (hipMalloc / torch CUDA tensors)
 *    unless marked "host". The caller owns every buffer; the library never
 *    frees caller memory and keeps no state between calls beyond three
 *    thread-local items: the last error message, a pending
 *    calibatt_set_kernel_events pair and the checked-mode switch.
 *  - Tensors Q, K, V, O are [H][N][d], contiguous, row-major. Token order is
 *    n = (f*R + r)*C + c: frame f, spatial row r, column c.
 *  - Blocks: query/key block b covers tokens [b*B, min((b+1)*B, N));
 *    nb = ceil(N / B). A partial last block has fewer tokens, nothing is padded.
 *  - lse (optional, may be NULL) is float32 [H][N], natural-log units:
 *    lse_i = log sum_j exp(scale * q_i . k_j) over the keys row i attends to.
 *  - Supported: d in {64, 128}; B in {64, 128}; dtype bf16 (the performance
 *    path, fp32 accumulation and softmax) or fp32 (a correctness path with
 *    fp32 arithmetic throughout). scale must be finite and > 0.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). The
 *    attention calls are asynchronous: they only enqueue kernels on `stream`
 *    (no allocation, memset or host synchronisation), so they can be captured
 *    into a HIP graph and replayed; so can calibatt_compile_bitmap. The index
 *    and run compiles read a count back (a host sync) and checked mode reads
 *    the lists back: neither can be captured.
 *  - Errors: arguments are checked on the host before anything is enqueued.
 *    A bad argument returns CALIBATT_ERR_INVALID_ARG and touches no output; a
 *    failed HIP call returns CALIBATT_ERR_HIP. calibatt_last_error() then
 *    describes the failure. Faults inside kernels surface at the caller's next
 *    synchronisation of `stream`. The library is reentrant across threads;
 *    the error message is thread-local.
 */
#ifndef CALIBATT_H
#define CALIBATT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CALIBATT_OK = 0,
  CALIBATT_ERR_INVALID_ARG = 1,
  CALIBATT_ERR_CAPACITY = 2,
  CALIBATT_ERR_HIP = 3,
  CALIBATT_ERR_UNSUPPORTED = 4
} calibatt_status_t;

/* Element type of Q, K, V and O. A plain 32-bit integer (an enum's size and
 * range are not fixed across C and C++): a value other than the two below is
 * rejected with CALIBATT_ERR_INVALID_ARG. */
typedef int32_t calibatt_dtype_t;
enum { CALIBATT_BF16 = 0, CALIBATT_F32 = 1 };

/* Limits of one call. */
#define CALIBATT_MAX_HEADS 256    /* heads taking part in one attention call */
#define CALIBATT_MAX_ANCHORS 64   /* anchor rows per frame */
#define CALIBATT_MAX_NB 4096      /* blocks per sequence (N <= 4096 * B) */

/*
 * A compiled skip-list dictionary (a POD view of caller-owned device arrays,
 * as produced by calibatt_compile_skiplist).
 *   T, L, H : timesteps, layers and heads the dictionary covers
 *   N, B, nb: tokens, block size, blocks per sequence (nb = ceil(N/B))
 *   row_ptr : int64 [T*L*H*nb + 1]; record (t, l, h) has id (t*L + l)*H + h
 *             and its query block r is row id*nb + r.
 *   col_idx : int32 [row_ptr[T*L*H*nb]], each row's key blocks, ascending.
 *   order   : int32 [T*L*H*nb] or NULL; per record, query blocks by
 *             descending kept count (ties by index), for callers that
 *             schedule work by cost. The attention calls do not read it: they
 *             visit query blocks in block order, where neighbours share key
 *             blocks in cache (heaviest-first measured no faster).
 */
typedef struct {
  int32_t T, L, H, N, B, nb;
  const int64_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* order;
} calibatt_skiplist_t;

/*
 * Compile binary block masks into skip lists ([Notes] Key Design 4: each mask
 * becomes, per query block, the read-only list of key blocks to compute, kept
 * on the GPU; Overall Architecture: indexed by timestep, layer and head).
 *
 *   masks     uint8 [T][L][H][nb][nb], device; entry [t][l][h][r][c] != 0
 *             means "compute query block r against key block c".
 *   T, L, H   >= 1; N >= 1 tokens; B >= 1 block size; nb = ceil(N/B) <= CALIBATT_MAX_NB.
 *   row_ptr   int64 [T*L*H*nb + 1], device, written (row_ptr[0] = 0).
 *   col_idx   int32 [col_capacity], device, written; may be NULL to query the
 *             size only (then only row_ptr and *nnz_out are written).
 *   order     int32 [T*L*H*nb], device, written; may be NULL.
 *   nnz_out   host; receives the number of kept blocks (always, when OK or CAPACITY).
 * Returns CALIBATT_ERR_CAPACITY when col_capacity < nnz (col_idx and order are
 * then not written). The two compile calls are the only ones that synchronise
 * `stream` (to read the count back); they run offline, before generation.
 */
calibatt_status_t calibatt_compile_skiplist(const uint8_t* masks, int32_t T, int32_t L, int32_t H,
                                            int32_t N, int32_t B, int64_t* row_ptr, int32_t* col_idx,
                                            int64_t col_capacity, int32_t* order, int64_t* nnz_out,
                                            void* stream);

/*
 * Block-sparse attention for selected heads of one layer-call ([Notes]
 * Overall Architecture and Key Design 4; [Abstract]: retained connections are
 * computed densely from the current Q, K, V, unselected ones are skipped).
 * For every listed head h and query block r of record (t, l, h):
 *   O[h][I_r] = softmax(scale * Q[h][I_r] K[h][J]^T) V[h][J],
 * J = union of the key blocks in row r's list. An empty list gives O = 0 and
 * lse = -inf. Only rows of the listed heads are written.
 *   q, k, v   [H][N][d] (bf16 or fp32 per dtype), device, read-only.
 *   o         [H][N][d], device, written for the listed heads.
 *   lse       float [H][N], device, or NULL.
 *   sl        host pointer to a skip-list view with sl->H == H, sl->N == N,
 *             sl->B in {64, 128}, 0 <= t < sl->T, 0 <= l < sl->L.
 *   heads     host int32 [n_heads], distinct head indices in [0, H), or NULL
 *             for all H heads (then n_heads is ignored).
 */
calibatt_status_t calibatt_block_sparse_attn(const void* q, const void* k, const void* v, void* o,
                                             float* lse, int32_t H, int32_t N, int32_t d,
                                             calibatt_dtype_t dtype, float scale,
                                             const calibatt_skiplist_t* sl, int32_t t, int32_t l,
                                             const int32_t* heads, int32_t n_heads, void* stream);

/*
 * Anchor-row attention with broadcast for selected (repetitive) heads
 * ([Notes] Key Design 3: only anchor rows compute attention, against all keys
 * and values; each anchor's output is broadcast to its nearest spatial rows
 * within the frame; k anchors reduce a frame's queries from R*C to k*C).
 *   N must equal F*R*C. anchor_rows: host int32 [k], strictly ascending, in
 *   [0, R); 1 <= k <= min(R, CALIBATT_MAX_ANCHORS). Each row r copies the
 *   anchor a minimising |r - a| (ties to the smaller a), column by column, in
 *   the same frame; lse is copied the same way. Tiling is internal (128
 *   queries and keys per tile for bf16, 64 for fp32); the result does not
 *   depend on it.
 *   heads: host int32 [n_heads] or NULL for all heads.
 */
calibatt_status_t calibatt_anchor_attn(const void* q, const void* k, const void* v, void* o,
                                       float* lse, int32_t H, int32_t N, int32_t d,
                                       calibatt_dtype_t dtype, float scale,
                                       int32_t F, int32_t R, int32_t C, const int32_t* anchor_rows,
                                       int32_t k_anchors, const int32_t* heads, int32_t n_heads,
                                       void* stream);

/*
 * One attention layer-call with per-head dual-path dispatch ([Notes] Key
 * Design 4: the current timestep, layer and head select the record; the
 * repetition flag chooses anchor-row attention, otherwise block-sparse
 * attention; the paths are alternatives). rep_flags is host uint8 [T][L][H]
 * with T, L, H taken from *sl. Every head of O (and lse) is written. All work
 * is enqueued on `stream` without synchronising.
 */
calibatt_status_t calibatt_layer_dispatch(const void* q, const void* k, const void* v, void* o,
                                          float* lse, int32_t H, int32_t N, int32_t d,
                                          calibatt_dtype_t dtype, float scale,
                                          const calibatt_skiplist_t* sl, int32_t t, int32_t l,
                                          const uint8_t* rep_flags, int32_t F, int32_t R, int32_t C,
                                          const int32_t* anchor_rows, int32_t k_anchors, void* stream);

/*
 * The interval form of a compiled dictionary: the notes' own encoding, a
 * read-only list of contiguous key-block intervals per query block ([Notes]
 * Key Design 4; Highlights). One entry per maximal run of kept key blocks,
 * packed into 32 bits as two 16-bit halves (nb <= CALIBATT_MAX_NB < 2^16):
 * lo | hi << 16 names blocks lo .. hi-1, all kept; block lo-1 and block hi
 * are not kept (or lie outside the row). Runs of a row are ascending. A view
 * of caller-owned device arrays, as produced by calibatt_compile_intervals.
 *   T, L, H, N, B, nb: as in calibatt_skiplist_t.
 *   iv_ptr : int64 [T*L*H*nb + 1]; row id*nb + r owns runs iv_ptr[row] .. iv_ptr[row+1]-1.
 *   iv     : uint32 [iv_ptr[T*L*H*nb]] packed runs.
 *   order  : int32 [T*L*H*nb] or NULL; the same heaviest-first order as the
 *            index-list form (by kept-block count), likewise not read by the
 *            attention calls.
 */
typedef struct {
  int32_t T, L, H, N, B, nb;
  const int64_t* iv_ptr;
  const uint32_t* iv;
  const int32_t* order;
} calibatt_intervals_t;

/*
 * Compile binary block masks into the interval form (same masks, T, L, H, N,
 * B, order, stream and error rules as calibatt_compile_skiplist).
 *   iv_ptr    int64 [T*L*H*nb + 1], device, written (iv_ptr[0] = 0).
 *   iv        uint32 [iv_capacity], device, written; NULL to query the size only.
 *   n_iv_out  host; receives the number of runs (always, when OK or CAPACITY).
 * Returns CALIBATT_ERR_CAPACITY when iv_capacity < runs (iv and order are then
 * not written). Synchronises `stream` once to read the run count back.
 */
calibatt_status_t calibatt_compile_intervals(const uint8_t* masks, int32_t T, int32_t L, int32_t H,
                                             int32_t N, int32_t B, int64_t* iv_ptr, uint32_t* iv,
                                             int64_t iv_capacity, int32_t* order, int64_t* n_iv_out,
                                             void* stream);

/*
 * calibatt_block_sparse_attn over a dictionary in interval form: the kernels
 * walk each query block's runs directly. Same arguments, rules and results as
 * calibatt_block_sparse_attn (the key blocks, their order and the arithmetic
 * are the same, so the outputs are bitwise equal), with `il` in place of `sl`.
 */
calibatt_status_t calibatt_block_sparse_attn_iv(const void* q, const void* k, const void* v, void* o,
                                                float* lse, int32_t H, int32_t N, int32_t d,
                                                calibatt_dtype_t dtype, float scale,
                                                const calibatt_intervals_t* il, int32_t t, int32_t l,
                                                const int32_t* heads, int32_t n_heads, void* stream);

/*
 * calibatt_layer_dispatch over a dictionary in interval form (rep_flags is
 * [T][L][H] with T, L, H taken from *il). Bitwise equal to the index-list call.
 */
calibatt_status_t calibatt_layer_dispatch_iv(const void* q, const void* k, const void* v, void* o,
                                             float* lse, int32_t H, int32_t N, int32_t d,
                                             calibatt_dtype_t dtype, float scale,
                                             const calibatt_intervals_t* il, int32_t t, int32_t l,
                                             const uint8_t* rep_flags, int32_t F, int32_t R, int32_t C,
                                             const int32_t* anchor_rows, int32_t k_anchors, void* stream);

/*
 * The bitmap form of a compiled dictionary: the same selection as the lists,
 * one bit per key block ([Notes] Key Design 4: per query block, the key blocks
 * to compute), for dictionaries held in the least memory ([Notes] Limitations:
 * the masks of a whole Wan-720p run take tens of GB in the pages' own form).
 * Row r = ((t*L + l)*H + h)*nb + q of record (t, l, h), query block q, holds
 * `words` = ceil(nb/64) uint64 words; key block c is bit (c % 64) of word
 * (c / 64) (value 2^(c % 64)); bits past nb are zero. Fixed size per record:
 * no row pointers, and its compile needs no count read-back. A view of
 * caller-owned device memory, as produced by calibatt_compile_bitmap.
 *   T, L, H, N, B, nb: as in calibatt_skiplist_t.
 *   words : ceil(nb / 64).
 *   bits  : uint64 [T*L*H*nb][words], device, 8-byte aligned (a view that is
 *           not is rejected with CALIBATT_ERR_INVALID_ARG).
 */
typedef struct {
  int32_t T, L, H, N, B, nb, words;
  const uint64_t* bits;
} calibatt_bitmap_t;

/*
 * Compile binary block masks into the bitmap form (same masks, T, L, H, N, B
 * rules as calibatt_compile_skiplist).
 *   bits   uint64 [T*L*H*nb][ceil(nb/64)], device, 8-byte aligned, written.
 * Asynchronous: the size is known in advance, so nothing is read back.
 */
calibatt_status_t calibatt_compile_bitmap(const uint8_t* masks, int32_t T, int32_t L, int32_t H, int32_t N,
                                          int32_t B, uint64_t* bits, void* stream);

/*
 * calibatt_block_sparse_attn over a dictionary in bitmap form: each query
 * block's set bits are expanded, ascending, into the kernels' key-block list,
 * so the blocks, their order and the arithmetic are those of the index-list
 * form and the outputs are bitwise equal to calibatt_block_sparse_attn's.
 * Bits past nb are ignored. Same arguments and rules, with `bm` in place of `sl`.
 */
calibatt_status_t calibatt_block_sparse_attn_bm(const void* q, const void* k, const void* v, void* o,
                                                float* lse, int32_t H, int32_t N, int32_t d,
                                                calibatt_dtype_t dtype, float scale,
                                                const calibatt_bitmap_t* bm, int32_t t, int32_t l,
                                                const int32_t* heads, int32_t n_heads, void* stream);

/*
 * calibatt_layer_dispatch over a dictionary in bitmap form (rep_flags is
 * [T][L][H] with T, L, H taken from *bm). Bitwise equal to the index-list call.
 */
calibatt_status_t calibatt_layer_dispatch_bm(const void* q, const void* k, const void* v, void* o,
                                             float* lse, int32_t H, int32_t N, int32_t d,
                                             calibatt_dtype_t dtype, float scale,
                                             const calibatt_bitmap_t* bm, int32_t t, int32_t l,
                                             const uint8_t* rep_flags, int32_t F, int32_t R, int32_t C,
                                             const int32_t* anchor_rows, int32_t k_anchors, void* stream);

/*
 * ---- Checked mode (for list views the caller built or loaded itself) ----
 *
 * The attention calls trust a view's contents: the compile calls produce
 * valid lists ([Notes] Key Design 4: the lists are compiled once, offline, and
 * read-only at inference), and a malformed view makes the kernels read outside
 * the key blocks or their list staging. These calls check a view on the host.
 *
 * calibatt_validate_skiplist / calibatt_validate_intervals: validate the rows
 * of record (t, l), all H heads of it, or of the whole dictionary when
 * t = l = -1:
 *   - row pointers non-decreasing (row_ptr[0] = 0 for the whole dictionary);
 *   - index lists: entries strictly ascending inside [0, nb);
 *   - runs: lo < hi <= nb, strictly ascending with a gap of at least one
 *     block between neighbours (maximal runs, at most ceil(nb/2) per row);
 *   - order (when not NULL): a permutation of [0, nb) per record.
 * host_arrays = 0: the view's arrays are device memory; they are copied to
 * host memory on `stream`, which is synchronised. host_arrays != 0: they are
 * host memory and no HIP call is made (stream ignored).
 * Returns CALIBATT_OK, or CALIBATT_ERR_INVALID_ARG with the first offending
 * row named in calibatt_last_error() (CALIBATT_ERR_HIP if a copy fails).
 */
calibatt_status_t calibatt_validate_skiplist(const calibatt_skiplist_t* sl, int32_t t, int32_t l,
                                             int32_t host_arrays, void* stream);
calibatt_status_t calibatt_validate_intervals(const calibatt_intervals_t* il, int32_t t, int32_t l,
                                              int32_t host_arrays, void* stream);
/* Bitmaps: words == ceil(nb/64), and the bits past nb are zero. */
calibatt_status_t calibatt_validate_bitmap(const calibatt_bitmap_t* bm, int32_t t, int32_t l,
                                           int32_t host_arrays, void* stream);

/*
 * Checked mode for this thread: when enabled, calibatt_block_sparse_attn(_iv,
 * _bm) and calibatt_layer_dispatch(_iv, _bm) validate the record (t, l) they are given,
 * as calibatt_validate_* does (copying its lists to host memory and
 * synchronising `stream`), before anything is enqueued; a malformed record
 * returns CALIBATT_ERR_INVALID_ARG and no kernel runs. Off by default (the
 * calls then stay fully asynchronous).
 */
void calibatt_set_checked_mode(int32_t enabled);

/*
 * ---- Offline calibration (produces the masks compiled above) ----
 *
 * Block energies of one calibration prompt ([Notes] Key Design 1, Eq. 5; Key
 * Design 4: accumulated without materialising the attention matrix). For each
 * listed head h, query block r and key block c:
 *   E[h][r][c] = (1/|I_r|) * sum_{i in I_r} sum_{j in J_c} P[i][j],
 *   P = softmax over all N keys of scale * Q[h][i] . K[h][j].
 * The average is over the block's actual query count |I_r| (B for every full
 * block), so each row of E sums to one, also for a partial last block.
 *   q, k      [H][N][d] (bf16 or fp32), device, read-only.
 *   B         64 or 128 (query and key block size); nb = ceil(N/B) <= CALIBATT_MAX_NB.
 *   energy    float [H][nb][nb], device; rows of the listed heads are written.
 *   heads     host int32 [n_heads] or NULL for all heads.
 *   work      optional device workspace (16-byte aligned, caller-owned,
 *             overwritten), work_bytes its size. NULL: every score is computed
 *             twice (a pass for each query's log-sum-exp, then the sums).
 *             Given (bf16 inputs): one pass; each query leaves one float per
 *             key block in the workspace (nb*nb*B floats per head, 179 MB for
 *             a head of N = 75,600 at B = 128), and the listed heads run in
 *             launches of as many heads as it holds. work_bytes below one
 *             head's share is an error. fp32 inputs ignore it.
 * Asynchronous. calibatt_set_kernel_events times all of its launches.
 */
calibatt_status_t calibatt_block_energy(const void* q, const void* k, int32_t H, int32_t N, int32_t d,
                                        calibatt_dtype_t dtype, float scale, int32_t B, float* energy,
                                        const int32_t* heads, int32_t n_heads, float* work, int64_t work_bytes,
                                        void* stream);

/*
 * calibatt_block_energy for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving or calibration loops, harnesses that
 * forbid hipMalloc): the same energies, bitwise equal to calibatt_block_energy
 * with a workspace, with the one-pass workspace taken from a scratch array the
 * library holds on each GPU (CALIBATT_NOALLOC_SCRATCH_BYTES = 256 MiB, held from
 * the first call on a device until the process ends). The listed heads' query
 * blocks run in launches of as many as the scratch holds (nb*B floats each:
 * 887 query blocks per launch at N = 75,600, B = 128; every supported shape
 * fits at least one). No device memory is allocated or freed, and no host heap
 * is used. Arguments and results as calibatt_block_energy (fp32 inputs take the
 * two-pass fp32 kernel, which needs no workspace). `stream` must belong to the
 * current device. Calls that overlap on one GPU (other streams or threads)
 * share its scratch and race: serialise them. Returns CALIBATT_ERR_CAPACITY if
 * one query block's workspace exceeds the scratch (not reachable with
 * nb <= CALIBATT_MAX_NB).
 */
#define CALIBATT_NOALLOC_SCRATCH_BYTES (256ull << 20)
calibatt_status_t calibatt_block_energy_noalloc(const void* q, const void* k, int32_t H, int32_t N, int32_t d,
                                                calibatt_dtype_t dtype, float scale, int32_t B, float* energy,
                                                const int32_t* heads, int32_t n_heads, void* stream);

/*
 * Per-prompt selection ([Notes] Key Design 1): for every row of `energy`
 * (rows x nb, device, finite and >= 0), sort the energies in descending order
 * (ties to the lower key block) and keep the shortest prefix whose cumulative
 * mass reaches tau (>=). The cumulative mass is summed exactly in 2^-48 fixed
 * point: each energy counts floor(E * 2^48) units against ceil(tau * 2^48), so
 * the decision does not depend on summation order. A row that never reaches
 * tau keeps every block. 0 <= tau <= 1.
 *   mask      uint8 [rows][nb], device, written (1 = keep), or NULL.
 *   counts    int32 [rows][nb], device, or NULL: incremented by the mask
 *             (accumulates the selections of the calibration prompts).
 * At least one of mask and counts must be non-NULL. Asynchronous.
 */
calibatt_status_t calibatt_select_blocks(const float* energy, int64_t rows, int32_t nb, float tau,
                                         uint8_t* mask, int32_t* counts, void* stream);

/*
 * Cross-prompt aggregation ([Notes] Key Design 2, Eq. 8-9; A Worked Example:
 * 64 prompts at rho = 0.5 keep blocks selected at least 32 times):
 *   mask[i] = (counts[i] / n_prompts >= rho), evaluated exactly as
 *   counts[i] >= ceil(rho * n_prompts).
 *   counts    int32 [n], device (from calibatt_select_blocks over the prompts).
 *   mask      uint8 [n], device, written; e.g. the [T][L][H][nb][nb] slice of
 *             a dictionary for calibatt_compile_skiplist / _intervals.
 * n_prompts >= 1, 0 <= rho <= 1. Asynchronous.
 */
calibatt_status_t calibatt_keep_frequency(const int32_t* counts, int64_t n, int32_t n_prompts, float rho,
                                          uint8_t* mask, void* stream);

/*
 * Spatial-repetition detection, per prompt ([Notes] Key Design 3: the
 * attention of each spatial row, flattened, is compared by cosine similarity
 * with that of its nearest anchor row within the frame). For every listed
 * head h, frame f and spatial row r with nearest anchor a (ties to the smaller
 * anchor row):
 *   row_sim[h][f][r] = <P_r, P_a> / (|P_r| |P_a|),
 *   <P_r, P_a> = sum_{c < C} sum_{j < N} P[(f*R + r)*C + c][j] * P[(f*R + a)*C + c][j],
 * P = softmax over all N keys of scale * Q[h][i] . K[h][j]; anchor rows get 1.
 * One pass over the keys: each query's softmax normaliser is accumulated with
 * the sums, so no workspace is needed.
 *   q, k        [H][N][d] (bf16 or fp32), device, read-only; N = F*R*C.
 *   anchor_rows host int32 [k_anchors], strictly ascending in [0, R); 1 <= k < R.
 *   row_sim     float [H][F][R], device, written for the listed heads.
 *   heads       host int32 [n_heads] or NULL for all heads.
 * Asynchronous. calibatt_set_kernel_events times the similarity launch.
 */
calibatt_status_t calibatt_spatial_similarity(const void* q, const void* k, int32_t H, int32_t N, int32_t d,
                                              calibatt_dtype_t dtype, float scale, int32_t F, int32_t R,
                                              int32_t C, const int32_t* anchor_rows, int32_t k_anchors,
                                              float* row_sim, const int32_t* heads, int32_t n_heads,
                                              void* stream);

/*
 * Repetition flags ([Notes] Key Design 3: the similarities are averaged over
 * frames, rows and calibration prompts; a head is repetitive only when the
 * mean exceeds the threshold, 0.87 by default). The mean runs over the
 * non-anchor rows of every frame of every prompt, accumulated in double in a
 * fixed order; flag = mean > threshold (strict).
 *   row_sim     float [n_prompts][H][F][R], device (row_sim of each prompt).
 *   flags       uint8 [H], device, written (1 = repetitive), or NULL.
 *   mean        float [H], device, written, or NULL (not both NULL).
 * Asynchronous.
 */
calibatt_status_t calibatt_repetition_flags(const float* row_sim, int32_t n_prompts, int32_t H, int32_t F,
                                            int32_t R, const int32_t* anchor_rows, int32_t k_anchors,
                                            float threshold, uint8_t* flags, float* mean, void* stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* calibatt_last_error(void);

/*
 * Timing hook for benchmarks: the next attention or energy launch made on
 * this thread by calibatt_block_sparse_attn(_iv), calibatt_anchor_attn,
 * calibatt_layer_dispatch(_iv), calibatt_block_energy or
 * calibatt_spatial_similarity records hipEvent_t
 * `begin` right before that kernel and `end` right after it, on the same
 * stream; the hook then clears itself. Pass NULL, NULL to clear it explicitly.
 */
void calibatt_set_kernel_events(void* begin, void* end);

/* Library version as major*10000 + minor*100 + patch. */
int32_t calibatt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CALIBATT_H */
