// Internal declarations shared by the host entry points and the kernels of
// libcalibatt.so. Nothing here is part of the C ABI (see include/calibatt.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "calibatt.h"

namespace calibatt {

// One attention launch: a list of work items, each a tile of up to `blk`
// queries of one head together with the key blocks it visits.
//   * anchor items come first: head anchor_heads[i / anchor_tiles], tile
//     i % anchor_tiles of the gathered anchor queries (F*k*C of them, in
//     (frame, anchor, column) order), visiting every key block;
//   * block-sparse items follow: head sparse_heads[j / nb] visits the list of
//     query block j % nb (query blocks in block order: neighbours share most of
//     their key blocks; the compiled heaviest-first order is not read).
// Grid blocks map to items
// XCD-aware: workgroups are dispatched round-robin over the 8 XCDs, so each
// XCD's share of the grid is fixed in advance. Anchor items (all of one size)
// go one chunk of n/8 consecutive items per XCD; block-sparse items go in runs
// of 8 * xcd_group grid blocks,
// XCD x receiving xcd_group consecutive items per run (neighbouring query
// blocks share most of their key blocks, which then stay in that XCD's L2),
// and with xcd_rotate the chunk each XCD takes turns by one per run.
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t head_stride;      // N * d elements
  int32_t N;
  int32_t nb;               // key (and query) blocks of `blk` tokens
  float scale;              // softmax scale
  float scale_log2;         // scale * log2(e)
  // block-sparse items
  const int64_t* row_ptr;
  const int32_t* col_idx;
  const uint32_t* runs;     // interval form: packed runs lo | hi << 16 (row_ptr then
                            // offsets runs, col_idx is unused); NULL for index lists
  const uint64_t* bits;     // bitmap form: bm_words words per row (row_ptr, col_idx and
                            // runs unused); NULL otherwise
  int32_t bm_words;         // ceil(nb / 64)
  int64_t rec_row0;         // skip-list row of (t, l, head 0, block 0)
  int32_t rec_head_rows;    // rows per record (= nb)
  int32_t n_sparse;
  int32_t xcd_group;        // consecutive items given to one XCD (0: plain grid order)
  int32_t xcd_rotate;       // 1: the chunk of each XCD turns per run (runs that cover whole heads)
  // anchor items
  int32_t n_anchor;
  int32_t anchor_tiles;
  int32_t n_anchor_q;       // F * k * C
  int32_t F, R, C, ka;       // frames, rows, columns, anchor rows per frame
  int32_t anchors[CALIBATT_MAX_ANCHORS];
  int32_t sparse_heads[CALIBATT_MAX_HEADS];
  int32_t anchor_heads[CALIBATT_MAX_HEADS];
};

// Copy of anchor-row outputs to the other spatial rows of each frame.
struct BcastParams {
  void* o;
  float* lse;
  int64_t head_stride;      // N * d elements
  int32_t N, d, esize;      // esize: bytes per element of o
  int32_t F, R, C, ka;       // frames, rows, columns, anchor rows per frame
  int32_t n_heads;
  int32_t anchors[CALIBATT_MAX_ANCHORS];
  int32_t heads[CALIBATT_MAX_HEADS];
};

// Block energies of selected heads for one prompt: one work item per
// (head, query block) in head-major order; a launch covers the items
// [item0, item0 + grid size).
struct EnergyParams {
  const void* q;
  const void* k;
  float* energy;            // [H][nb][nb]
  float* work;              // bf16 one-pass kernel: [items][nb][B] floats, or null (two passes)
  int64_t item0;            // first item of the launch (item = head index in heads * nb + query block);
                            // the workspace holds the launch's items from item0 on
  int64_t head_stride;      // N * d elements
  int32_t N;
  int32_t nb;
  float scale;
  float scale_log2;
  int32_t dtype_f32;        // 1: fp32 inputs, 0: bf16
  int32_t n_heads;
  int32_t heads[CALIBATT_MAX_HEADS];
};

// Spatial-row similarities of selected heads for one prompt, in one pass over
// the keys (each query's softmax normaliser is accumulated alongside).
struct SimParams {
  const void* q;
  const void* k;
  float* row_sim;           // [H][F][R]
  int64_t head_stride;      // N * d elements
  int32_t N;
  int32_t F, R, C, ka;
  float scale;
  float scale_log2;
  int32_t n_heads;
  int32_t rows_per_group;   // bf16 path: non-anchor rows per workgroup (set by the launcher)
  int32_t anchors[CALIBATT_MAX_ANCHORS];
  int32_t heads[CALIBATT_MAX_HEADS];
};

struct RepFlagParams {
  int32_t anchors[CALIBATT_MAX_ANCHORS];
  int32_t ka;
  float threshold;
};

inline int64_t attn_items(const AttnParams& p) {
  return (int64_t)p.n_anchor * p.anchor_tiles + (int64_t)p.n_sparse * p.nb;
}

// Launchers (each returns the status of the launch itself).
hipError_t launch_attn_bf16(const AttnParams& p, int d, int blk, hipStream_t s);
hipError_t launch_attn_f32(const AttnParams& p, int d, int blk, hipStream_t s);
hipError_t launch_broadcast(const BcastParams& p, hipStream_t s);
hipError_t launch_energy(const EnergyParams& p, int d, int blk, hipStream_t s);
hipError_t launch_energy_onepass_items(const EnergyParams& p, int d, int blk, int64_t n_items, hipStream_t s);
hipError_t launch_similarity(const SimParams& p, int d, bool f32, hipStream_t s);
hipError_t launch_rep_flags(const float* sims, int P, int H, int F, int R, const RepFlagParams& q, uint8_t* flags,
                            float* mean, hipStream_t s);
hipError_t launch_select(const float* energy, int64_t rows, int nb, unsigned long long need, uint8_t* mask,
                         int32_t* counts, hipStream_t s);
hipError_t launch_keep(const int32_t* counts, int64_t n, int32_t k_min, uint8_t* out, hipStream_t s);

hipError_t launch_compile_count_scan(const uint8_t* masks, int64_t rows, int nb, int64_t* row_ptr,
                                     hipStream_t s);
hipError_t launch_compile_fill(const uint8_t* masks, int64_t rows, int nb, const int64_t* row_ptr,
                               int32_t* col_idx, hipStream_t s);
hipError_t launch_compile_order(const int64_t* row_ptr, int64_t records, int nb, int32_t* order,
                                hipStream_t s);
hipError_t launch_compile_runs_count_scan(const uint8_t* masks, int64_t rows, int nb, int64_t* iv_ptr,
                                          hipStream_t s);
hipError_t launch_compile_runs_fill(const uint8_t* masks, int64_t rows, int nb, const int64_t* iv_ptr,
                                    uint32_t* iv, int32_t* kept_out, hipStream_t s);
hipError_t launch_compile_runs_order(int64_t records, int nb, int32_t* order, hipStream_t s);
hipError_t launch_compile_bitmap(const uint8_t* masks, int64_t rows, int nb, uint64_t* bits, hipStream_t s);

}  // namespace calibatt
