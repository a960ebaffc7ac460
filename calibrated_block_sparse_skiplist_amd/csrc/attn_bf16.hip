// Block-sparse / anchor-row attention forward, bf16 inputs, for gfx950.
//
// Retained key blocks are computed densely from the current Q, K, V and the
// others are skipped (papernotes.org notes on "Accelerating Text-to-Video
// Generation with Calibrated Sparse Attention", Overall Architecture and Key
// Design 4). Anchor-row heads run the same core over gathered anchor queries
// and every key block (same notes, Key Design 3).
//
// Work decomposition. One workgroup owns one work item: a tile of BLK queries
// of one head; its BLK/32 waves own 32 queries each. Two workgroups share a
// CU (register budget capped at 256 per lane; 72 KB of LDS each: K and V
// double buffers plus the item's staged key-block list), so each SIMD runs
// two waves that cover each other's waits. Keys are visited in
// stages of 64 (two per 128-key block; 64-token blocks take stages of 32,
// which halve the K/V buffers so that four workgroups share a CU and each
// SIMD still runs two waves). In stage j each wave
//   1. computes S^T_j = K_j Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS,
//      B = Q^T held in registers): every lane owns one query column and half
//      of the stage's keys;
//   2. runs the online softmax in fp32: exp2 with log2(e) folded into the
//      scale, per-lane partial row sums of the bf16-rounded probabilities that
//      also feed the PV product, against a reference maximum that moves (and
//      rescales O) only when a stage's probabilities sum past 2^13 in some
//      lane (a stale reference is exact algebra: numerator and denominator
//      share it);
//   3. accumulates O^T += V_{j-1}^T P_{j-1}^T with the same MFMA, one stage
//      behind: A = V^T read from row-major LDS by ds_read_b64_tr_b16 (16-bit
//      transpose across 16-lane groups), B = P^T packed to bf16 straight from
//      the S^T accumulators; the contraction runs over keys in the order the
//      accumulator layout holds them, and V is read in that same order. The
//      exponentials of step 2 are issued between these MFMAs and the last
//      S^T MFMAs of the stage (those of key tile 0 once it is complete), so
//      the matrix pipe keeps running while the wave computes probabilities.
// K and V tiles move HBM -> LDS with global_load_lds_dwordx4 (no register
// staging), issued between the S^T MFMAs of the stage before they are used;
// s_waitcnt vmcnt plus a workgroup barrier publish each tile. A stage whose
// copies stay inside the sequence (nearly all) issues them straight; only a
// stage reaching past N takes the form with per-copy clamps.
//
// LDS rows are XOR-swizzled in 16-byte chunks: K by (row & 15), so the 16
// rows of an MFMA operand read hit distinct banks; V by 4*(row & 3), so the
// 8-row x 64-byte patch of a transposed read spreads over all banks.
#include "gfx950_device.h"

namespace calibatt {
namespace {

using namespace dev;

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kStageSumCap = 8192.0f;     // a lane's 32 probabilities of a stage may sum to this
constexpr int kPrefetchK = 4;               // K operand reads in flight ahead of their MFMA
constexpr int kPrefetchV = 3;               // V operand reads (2 instructions each) in flight
constexpr int kListCap = CALIBATT_MAX_NB;   // key-block indices staged in LDS per item (all of them)

struct Item {
  int head;
  bool anchor;
  int tile;              // query block (sparse) or anchor tile
  const int32_t* list;   // index-list form: the key blocks
  const uint32_t* runs;  // interval form: packed runs lo | hi << 16
  const uint64_t* bits;  // bitmap form: the row's words (expanded to an index list in LDS)
  int n;                 // key blocks to visit (index list, anchor), or runs (interval form);
                         // bitmap form: counted from the words
};

__device__ __forceinline__ Item decode_item(const AttnParams& p, int64_t item) {
  Item it;
  const int64_t n_anchor_items = (int64_t)p.n_anchor * p.anchor_tiles;
  if (item < n_anchor_items) {
    it.anchor = true;
    it.head = p.anchor_heads[item / p.anchor_tiles];
    it.tile = (int)(item % p.anchor_tiles);
    it.list = nullptr;
    it.runs = nullptr;
    it.bits = nullptr;
    it.n = p.nb;
  } else {
    const int64_t j = item - n_anchor_items;
    const int hi = (int)(j / p.nb);
    const int rank = (int)(j % p.nb);
    it.anchor = false;
    it.head = p.sparse_heads[hi];
    const int64_t rec_row = p.rec_row0 + (int64_t)it.head * p.rec_head_rows;
    it.tile = rank;   // query blocks in block order: neighbours share key blocks in cache
    if (p.bits) {
      it.list = nullptr;
      it.runs = nullptr;
      it.bits = p.bits + (rec_row + it.tile) * p.bm_words;
      it.n = 0;
    } else {
      const int64_t b = p.row_ptr[rec_row + it.tile];
      const int64_t e = p.row_ptr[rec_row + it.tile + 1];
      it.list = p.runs ? nullptr : p.col_idx + b;
      it.runs = p.runs ? p.runs + b : nullptr;
      it.bits = nullptr;
      it.n = (int)(e - b);
    }
  }
  return it;
}

// Token of query slot `qi` of an item (or -1 when the slot is past the end).
__device__ __forceinline__ int query_token(const AttnParams& p, const Item& it, int qi, int BLK) {
  if (!it.anchor) {
    const int tok = it.tile * BLK + qi;
    return tok < p.N ? tok : -1;
  }
  const int aq = it.tile * BLK + qi;
  if (aq >= p.n_anchor_q) return -1;
  const int per_frame = p.ka * p.C;
  const int f = aq / per_frame;
  const int rem = aq - f * per_frame;
  const int ai = rem / p.C;
  const int c = rem - ai * p.C;
  return (f * p.R + p.anchors[ai]) * p.C + c;
}

// LSE: the log-sum-exp output is requested (p.lse). O is normalised by the
// sum of the bf16 probabilities that also enter the PV product, so numerator
// and denominator share their rounding; that sum can be 2^-8 off the true row
// sum when a few rounded terms dominate a row, so lse takes a second, fp32 sum
// of the probabilities, kept only in this instantiation.
template <int D, int BLK, bool LSE>
// (d = 64 needs about 150 VGPRs and 40 KB of LDS, so three waves share each
// SIMD: 5 % faster dense and 15 % on sparse lists than at two.)
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2, D == 64 ? 3 : 2)))
void attn_bf16_kernel(const AttnParams p) {
  constexpr int NW = BLK / 32;           // waves per workgroup (32 queries each)
  constexpr int SUB = BLK >= 128 ? 64 : 32;   // keys per pipeline stage (32 for 64-token blocks: half the LDS)
  constexpr int SPB = BLK / SUB;         // stages per key block
  constexpr int CPR = D / 8;             // 16-byte chunks per K/V row
  constexpr int KT = SUB / 32;           // 32-key tiles of S^T per stage
  constexpr int DS = D / 16;             // 16-wide d slabs (QK contraction)
  constexpr int DT = D / 32;             // 32-wide d tiles of O^T
  constexpr int KS = SUB / 16;           // 16-key slabs (PV contraction)
  constexpr int STAGE = SUB * CPR;       // 16-byte slots per stage and tensor
  constexpr int LPW = STAGE / 64 / NW;   // DMA instructions per wave, tensor and stage
  constexpr int RPI = 64 / CPR;          // rows per DMA instruction

  // Two stages of K and of V (double buffer) in one array, so that the
  // buffer of an operand read is an immediate offset; and the item's
  // key-block list.
  __shared__ uint4 lds_kv[4 * STAGE];
  __shared__ uint32_t lds_list32[kListCap / 2];   // index list (as uint16) or runs
  uint16_t* const lds_list = reinterpret_cast<uint16_t*>(lds_list32);
  uint4* const lds_k0 = lds_kv;
  uint4* const lds_k1 = lds_kv + STAGE;
  uint4* const lds_v0 = lds_kv + 2 * STAGE;
  uint4* const lds_v1 = lds_kv + 3 * STAGE;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;               // half of the wave
  const int l32 = lane & 31;

  const Item it = decode_item(p, xcd_item_after(blockIdx.x, gridDim.x, p.xcd_group,
                                                (int64_t)p.n_anchor * p.anchor_tiles, p.xcd_rotate != 0));
  // Scalars used inside the loop, pinned in registers: if the compiler reloads
  // them from the kernel arguments, each scalar load (which returns out of
  // order) forces every following LDS wait to drain completely.
  int n_tok = p.N;
  float scale_log2 = p.scale_log2;
  asm volatile("" : "+s"(n_tok), "+s"(scale_log2));
  const u16* Q = static_cast<const u16*>(p.q) + (int64_t)it.head * p.head_stride;
  const char* Kb = reinterpret_cast<const char*>(static_cast<const u16*>(p.k) + (int64_t)it.head * p.head_stride);
  const char* Vb = reinterpret_cast<const char*>(static_cast<const u16*>(p.v) + (int64_t)it.head * p.head_stride);

  // The item's key-block list (or its runs: at most nb/2 of them) goes to LDS
  // once (nb <= CALIBATT_MAX_NB, as the host checks), so the loop reads
  // indices with LDS broadcasts instead of vector-memory loads, which would
  // join the vmcnt queue of the prefetch.
  // A bitmap row is expanded into the same index list: lane w of every wave
  // takes word w (bm_words <= 64) and the set bits are counted with a wave
  // prefix sum; wave 0 writes each lane's blocks, ascending, after those of
  // the lanes before it.
  int n_listed = it.n;
  if (it.list) {
    for (int i = threadIdx.x; i < it.n; i += NW * 64) lds_list[i] = (uint16_t)it.list[i];
  } else if (it.runs) {
    for (int i = threadIdx.x; i < it.n; i += NW * 64) lds_list32[i] = it.runs[i];
  } else if (it.bits) {
    uint64_t word = lane < p.bm_words ? it.bits[lane] : 0ull;
    // (bits past nb are zero in a compiled bitmap; they are dropped anyway, so
    // no listed block ever lies past the sequence)
    if (lane == p.bm_words - 1 && (p.nb & 63)) word &= (1ull << (p.nb & 63)) - 1ull;
    const int cnt = __popcll(word);
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    n_listed = __builtin_amdgcn_readlane(incl, 63);
    if (wave == 0) {
      int pos = incl - cnt;
      while (word) {
        lds_list[pos++] = (uint16_t)(64 * lane + __builtin_ctzll(word));
        word &= word - 1;
      }
    }
  }
  const bool idx_list = it.list || it.bits;   // key blocks staged as an index list

  // Q^T operand fragments: query = wave*32 + l32, d = 16*s + 8*h + [0, 8).
  const int qtok = query_token(p, it, wave * 32 + l32, BLK);
  bf16x8 qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (qtok >= 0) raw = ld_global16(Q + (int64_t)qtok * D + 16 * s + 8 * h);
    qf[s] = bitcast<bf16x8>(raw);
  }

  // DMA geometry. Copy instruction i of this wave fills the RPI stage rows
  // from R = (wave*LPW + i)*RPI (uniform); lane l writes row R + q, q = l / CPR,
  // chunk slot pos = l % CPR, with source chunk pos ^ swz(R + q). As R is a
  // multiple of RPI and q < RPI, swz_k(R + q) = (R & (CPR-1)) ^ (q & (CPR-1))
  // and swz_v(R + q) = swz_v(q): the byte offset of a lane is a fixed lane part,
  // XORed (K only) with uniform chunk bits.
  const int dq = lane / CPR;
  const int dpos = lane % CPR;
  const uint32_t dma_k_lane = (uint32_t)(dq * 2 * D + 16 * (dpos ^ (dq & (CPR - 1))));
  const uint32_t dma_v_lane = (uint32_t)(dq * 2 * D + 16 * (dpos ^ swz_v<CPR>(dq)));
  __syncthreads();

  // Sources of the copy of stage `half` of key block c: a uniform base per
  // tensor plus this lane's offsets. Rows past the end of the sequence (last
  // block only) read the last token instead: their scores are masked and their
  // probabilities are exactly 0.
  // On the last block the base row is min(row0, N-1) and clamped lane offsets
  // are taken from it, so every offset stays non-negative (the 32-bit lane
  // offset of the copy instruction is unsigned).
  struct StageSrc { const char* base; bool clamp; int row0; int base_row; };
  auto stage_src = [&](const char* T, int c, int half) -> StageSrc {
    const int row0 = c * BLK + half * SUB;
    const int b0 = min(row0, n_tok - 1);
    return {T + (int64_t)b0 * (D * 2), row0 + SUB > n_tok, row0, b0};
  };
  // Copy instruction i (0 <= i < LPW) of this wave for one tensor of a stage.
  auto issue_one = [&](const StageSrc& src, int i, bool is_k, uint4* dst_stage) {
    const int r = (wave * LPW + i) * RPI;   // first stage row of the instruction
    const uint32_t off = is_k ? dma_k_lane ^ (uint32_t)(16 * (r & (CPR - 1))) : dma_v_lane;
    if (!src.clamp) {
      dma16(src.base + (int64_t)r * (2 * D), off, dst_stage + (wave * LPW + i) * 64);
    } else {
      // (the empty statement keeps this rare path a branch instead of
      // selects evaluated on every copy)
      asm volatile("");
      const int grow = min(src.row0 + r + dq, n_tok - 1);
      const uint32_t coff = (uint32_t)((grow - src.base_row) * (2 * D)) + (off & (2 * D - 1));
      dma16(src.base, coff, dst_stage + (wave * LPW + i) * 64);
    }
  };

  // Lane part of the K operand reads (see read_k).
  const uint32_t k_lane = (uint32_t)(l32 * 2 * D + 16 * (h ^ (l32 & (CPR - 1))));

  // Key blocks in visiting order (uniform across the workgroup). Index lists
  // and anchor items are indexed by step; runs are walked with a cursor
  // (current run, its end), advanced once per block. The LDS entry a block
  // change needs (the next index, or the next run) is read one stage before
  // the change (pf_next), so its latency is not paid at a stage's start.
  int run_i = 0, run_hi = 0;
  uint32_t pf_next = 0;
  auto first_block = [&]() -> int {
    if (it.runs) {
      const uint32_t w = __builtin_amdgcn_readfirstlane(lds_list32[0]);
      run_hi = (int)(w >> 16);
      return (int)(w & 0xffffu);
    }
    return idx_list ? __builtin_amdgcn_readfirstlane((int)lds_list[0]) : 0;
  };
  auto next_block = [&](int c, int i) -> int {   // i: step of the block that follows c
    if (it.runs) {
      if (c + 1 < run_hi) return c + 1;
      const uint32_t w = __builtin_amdgcn_readfirstlane(pf_next);   // lds_list32[run_i + 1]
      ++run_i;
      run_hi = (int)(w >> 16);
      return (int)(w & 0xffffu);
    }
    // lds_list[i]: the 16-bit half of the word read at step i's first stage
    return idx_list ? (int)((__builtin_amdgcn_readfirstlane(pf_next) >> (16 * (i & 1))) & 0xffffu) : i;
  };
  // At the first stage of a block, the 32-bit LDS word next_block will need at
  // its last: the next run, or the word holding the next index (one load, its
  // address a uniform select; the list area holds kListCap/2 words, so every
  // word index below stays in it).
  auto prefetch_next = [&](int i) {   // i: step of the next block
    const int word = it.runs ? min(run_i + 1, kListCap / 2 - 1) : min(i >> 1, kListCap / 2 - 1);
    pf_next = lds_list32[word];
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int u = 0; u < DT; ++u) oacc[u] = f32x16{};
  float m_run = -INFINITY;   // reference maximum of scaled scores (log2 units)
  float l_run = 0.0f;        // this lane's partial sum of probabilities (bf16-rounded, as in PV)
  float lf_run = 0.0f;       // the same sum in fp32 (lse only)

  // Software pipeline over 64-key stages. Stage j computes S^T_j and its
  // probabilities P_j, while the matrix pipe runs the PV product of stage
  // j-1: the exponentials of stage j are issued between those MFMAs. So K_j
  // and V_{j-1} are read in stage j; the copy issued in stage j brings K_{j+1}
  // and V_j. Two LDS buffers per tensor suffice: K_{j+1} overwrites K_{j-1},
  // V_j overwrites V_{j-2}, and both were last read before the barrier that
  // opens stage j. Stage 0 multiplies zero probabilities with a zeroed V
  // buffer, so every stage runs the same code.
  uint32_t pkA[KS][4], pkB[KS][4];   // bf16 P^T fragments of even / odd stages
#pragma unroll
  for (int i = 0; i < KS; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) pkB[i][e] = 0u;
  for (int i = threadIdx.x; i < STAGE; i += NW * 64) lds_v1[i] = make_uint4(0, 0, 0, 0);

  // Blocks to visit: the run lengths summed (every wave sums the staged runs
  // itself, so no extra barrier), or the list length.
  int n_blocks = n_listed;
  if (it.runs) {
    int part = 0;
    for (int i = lane; i < it.n; i += 64) {
      const uint32_t w = lds_list32[i];
      part += (int)(w >> 16) - (int)(w & 0xffffu);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
    n_blocks = __builtin_amdgcn_readfirstlane(part);
  }
  const int n_stages = n_blocks * SPB;
  int c = n_stages > 0 ? first_block() : 0;
  if (n_stages > 0) {
    const StageSrc src0 = stage_src(Kb, c, 0);
#pragma unroll
    for (int i = 0; i < LPW; ++i) issue_one(src0, i, true, lds_k0);
  }

  // V^T operand of PV step idx (16-key slab sl, 32-wide d tile u) from a V
  // stage. Lane (g = lane/16, jj = lane%16) reads keys 16*sl + vk and
  // 16*sl + vk + 8, vk = 4*(g/2) + jj/4, at d = 32*u + 16*(g%2) + 4*(jj%4).
  // The swizzle of those rows, 4*(vk & 3), has no bits below 4 and the chunk
  // index is 4*u + (a part below 4), so the byte offset is a lane part XORed
  // with 64*u; sl and the +8 rows are immediates.
  const int g = lane >> 4;
  const int jj = lane & 15;
  const int vk = 4 * (g >> 1) + (jj >> 2);
  const uint32_t v_lane = (uint32_t)(vk * 2 * D + 16 * (swz_v<CPR>(vk) + 2 * (g & 1) + ((jj & 3) >> 1)) +
                                     8 * (jj & 1));
  auto read_v = [&](const char* sv, int idx) -> bf16x8 {
    const int sl = idx / DT, u = idx % DT;
    const char* p = sv + 16 * sl * (2 * D) + (v_lane ^ (uint32_t)(64 * u));
    struct { i16x4 lo, hi; } both;
    both.lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    both.hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * (2 * D)));
    return bitcast<bf16x8>(both);
  };
  // O^T += V^T P^T for one stage; `step(idx)` runs after PV MFMA idx (the
  // exponentials of the next stage go there). Transposed reads run
  // kPrefetchV MFMAs ahead.
  auto pv_product = [&](const uint4* svv, const uint32_t (&pkp)[KS][4], auto step) {
    const char* sv = reinterpret_cast<const char*>(svv);
    bf16x8 ring[kPrefetchV];
#pragma unroll
    for (int i = 0; i < kPrefetchV; ++i) ring[i] = read_v(sv, i);
#pragma unroll
    for (int idx = 0; idx < KS * DT; ++idx) {
      const int sl = idx / DT, u = idx % DT;
      const bf16x8 a = ring[idx % kPrefetchV];
      if (idx + kPrefetchV < KS * DT) ring[idx % kPrefetchV] = read_v(sv, idx + kPrefetchV);
      oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bitcast<bf16x8>(pkp[sl]), oacc[u], 0, 0, 0);
      step(idx);
      __builtin_amdgcn_sched_barrier(0);   // keep the interleaving as written
    }
  };
  auto no_step = [](int) {};

  // Stage j; the body is instantiated per parity of j, which fixes its buffers.
  auto stage_body = [&](int j, const uint4* sk, uint4* nk, const uint4* svp, uint4* nv,
                        const uint32_t (&pk_prev)[KS][4], uint32_t (&pk_cur)[KS][4]) {
    const int half = j % SPB;
    const bool has_next = j + 1 < n_stages;
    const int c_next = (has_next && half == SPB - 1) ? next_block(c, j / SPB + 1) : c;

    // ---- K_j and V_{j-1} resident in every wave's view; the other buffers are free ----
    wait_vmcnt<0>();
    barrier_no_fence();
    if (half == 0) prefetch_next(j / SPB + 1);
    const StageSrc ksrc = stage_src(Kb, c_next, (j + 1) % SPB);
    const StageSrc vsrc = stage_src(Vb, c, half);
    // Copy step d of this stage: K_{j+1} first (when there is a next stage), then V_j.
    auto issue_dma = [&](int d) {
      if (d < LPW) {
        if (has_next) issue_one(ksrc, d, true, nk);
      } else {
        issue_one(vsrc, d - LPW, false, nv);
      }
    };

    // Nearly every stage has a next stage and no clamped rows in either copy:
    // then the copies run straight, without the per-copy tests of issue_dma
    // (their branches cost more than the copies themselves). One uniform test
    // per stage picks the form.
    const bool plain = has_next && !ksrc.clamp && !vsrc.clamp;
    auto issue_plain = [&](int d) {
      if (d < LPW) {
        const int r = (wave * LPW + d) * RPI;
        dma16(ksrc.base + (int64_t)r * (2 * D), dma_k_lane ^ (uint32_t)(16 * (r & (CPR - 1))),
              nk + (wave * LPW + d) * 64);
      } else {
        const int r = (wave * LPW + d - LPW) * RPI;
        dma16(vsrc.base + (int64_t)r * (2 * D), dma_v_lane, nv + (wave * LPW + d - LPW) * 64);
      }
    };

    // ---- online softmax (fp32, log2 domain, lazy reference maximum) ----
    // Probabilities of stage j are formed against the reference m_run shared
    // by both key halves of a query. The reference moves only when some
    // lane's 32 probabilities of the stage sum past kStageSumCap or are not
    // finite (the first stage, while m_run is -inf; masked keys then give
    // NaN): then m_run becomes the maximum so far, O and l (which hold stages
    // up to j-1, relative to the old reference) are scaled by alpha, and the
    // stage's probabilities are formed again. So the row maximum is searched
    // only on those rare stages and every probability kept is at most 2^13;
    // numerator and denominator share the reference, so a stale one is exact
    // algebra. Probabilities go to bf16 in pairs; the row sum adds those same
    // bf16 values (v_dot2 against 1.0), so numerator and denominator of O use
    // identical weights.
    float neg_m = -m_run;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float psum0 = 0.0f, psum1 = 0.0f;
    float f32sum0 = 0.0f, f32sum1 = 0.0f;   // (LSE only)
    f32x16 sacc[KT];
    constexpr int NP = KT * 8;          // probability pairs per lane and stage
    constexpr int NPV = KS * DT;        // PV MFMAs per stage
    constexpr int NQK = KT * DS;        // QK MFMAs per stage
    // Placement of the exponentials: the MFMA pipe runs best when the VALU
    // work between its instructions is thin, so kEarlyPairs pairs of key tile
    // 0 are formed between the last QK MFMAs (those of the later tiles; tile 0
    // is complete kQkGap MFMAs before the first of them is read) and the rest
    // between the PV MFMAs. The order of the pairs, hence every sum, is the
    // same either way.
    constexpr int kEarlyPairs = KT > 1 ? 4 : 0;   // (a single key tile has no later QK MFMAs to host them)
    constexpr int kQkGap = 2;
    constexpr int QS = KT == 1 ? NQK : (DS + kQkGap < NQK) ? DS + kQkGap : NQK - 1;   // first QK step hosting pairs
    static_assert(kEarlyPairs <= 8 && (kEarlyPairs == 0 || QS >= DS), "early pairs come from key tile 0");
    auto exp_pair = [&](int q) -> uint32_t {
      const int t = q >> 3, a = 2 * (q & 7);
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][a], scale_log2, neg_m));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][a + 1], scale_log2, neg_m));
      const bf16x2 two = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
      if ((a >> 1) & 1) psum1 = __builtin_amdgcn_fdot2_f32_bf16(two, ones, psum1, false);
      else psum0 = __builtin_amdgcn_fdot2_f32_bf16(two, ones, psum0, false);
      if constexpr (LSE) {
        f32sum0 += p0;
        f32sum1 += p1;
      }
      const uint32_t bits = bitcast<uint32_t>(two);
      pk_cur[2 * t + (a >> 3)][(a & 7) >> 1] = bits;
      return bits;
    };
    auto exp_range = [&](int q0, int q1) {   // pairs [q0, q1)
#pragma unroll
      for (int q = q0; q < q1; ++q) {
        const uint32_t bits = exp_pair(q);
        // Anchors: the results are first used after the PV product, and the
        // compiler would otherwise sink this work below its MFMAs.
        asm volatile("" :: "v"(bits));
        asm volatile("" : "+v"(psum0), "+v"(psum1));
        if constexpr (LSE) asm volatile("" : "+v"(f32sum0), "+v"(f32sum1));
      }
    };
    // Keys past N (last block only; a stage wholly past N, the second half of
    // a short last block, is masked entirely), per 32-key tile of S^T.
    const int valid = n_tok - (c * BLK + half * SUB);
    auto mask_tile = [&](int t) {
      if (valid < SUB) {
        // (opaque bound: keeps the comparisons inside this rarely taken branch)
        int lv = valid - 4 * h;
        asm volatile("" : "+v"(lv));
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const int key = 32 * t + 8 * (a >> 2) + (a & 3);
          if (key >= lv) sacc[t][a] = -INFINITY;
        }
      }
    };

    // ---- S^T = K Q^T: operand reads run kPrefetchK MFMAs ahead; the copy of
    // the next stage is issued in small steps between the MFMAs, and the
    // early probability pairs after tile 0 is complete ----
    auto qk_product = [&](auto issue) {
      // K operand of step (t, s): key 32*t + l32, chunk 2*s + h, swizzled
      // by l32 & (CPR-1); the chunk bits of s enter as an XOR with 32*s.
      auto read_k = [&](int idx) -> bf16x8 {
        const int t = idx / DS, s = idx % DS;
        const char* p = reinterpret_cast<const char*>(sk) + 32 * t * (2 * D) + (k_lane ^ (uint32_t)(32 * s));
        return bitcast<bf16x8>(*reinterpret_cast<const uint4*>(p));
      };
      constexpr int kDmaEvery = (KT * DS) / (2 * LPW) > 0 ? (KT * DS) / (2 * LPW) : 1;
      bf16x8 ring[kPrefetchK];
#pragma unroll
      for (int i = 0; i < kPrefetchK; ++i) ring[i] = read_k(i);
#pragma unroll
      for (int idx = 0; idx < NQK; ++idx) {
        const int t = idx / DS, s = idx % DS;
        const bf16x8 a = ring[idx % kPrefetchK];
        if (idx + kPrefetchK < NQK) ring[idx % kPrefetchK] = read_k(idx + kPrefetchK);
        sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], s == 0 ? f32x16{} : sacc[t], 0, 0, 0);
        if (idx % kDmaEvery == kDmaEvery - 1 && idx / kDmaEvery < 2 * LPW) issue(idx / kDmaEvery);
        if constexpr (kEarlyPairs > 0) {
          if (idx >= QS) {
            if (idx == QS) mask_tile(0);
            const int i = idx - QS;
            exp_range(i * kEarlyPairs / (NQK - QS), (i + 1) * kEarlyPairs / (NQK - QS));
          }
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the read-ahead order as written
      }
      // (copies that did not fit between the MFMAs, if any)
#pragma unroll
      for (int d = NQK / kDmaEvery; d < 2 * LPW; ++d) issue(d);
    };
    if (plain) qk_product(issue_plain);
    else qk_product(issue_dma);
#pragma unroll
    for (int t = kEarlyPairs > 0 ? 1 : 0; t < KT; ++t) mask_tile(t);

    // ---- O^T += V_{j-1}^T P_{j-1}^T, with the remaining pairs of stage j in between ----
    auto exp_pairs = [&](int idx) {
      exp_range(kEarlyPairs + idx * (NP - kEarlyPairs) / NPV, kEarlyPairs + (idx + 1) * (NP - kEarlyPairs) / NPV);
    };
    pv_product(svp, pk_prev, exp_pairs);
    if (__ballot(!(psum0 + psum1 <= kStageSumCap)) != 0) {
      asm volatile("");   // rare: keep it a branch
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int a = 0; a < 16; ++a) mx = fmaxf(mx, sacc[t][a]);
      const float mb = mx * scale_log2;
      const float m_new = fmaxf(m_run, fmaxf(mb, __shfl_xor(mb, 32)));
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m_run is -inf
      m_run = m_new;
      l_run *= alpha;
      lf_run *= alpha;
#pragma unroll
      for (int u = 0; u < DT; ++u)
#pragma unroll
        for (int a = 0; a < 16; ++a) oacc[u][a] *= alpha;
      neg_m = -m_run;
      psum0 = 0.0f;
      psum1 = 0.0f;
      f32sum0 = 0.0f;
      f32sum1 = 0.0f;
#pragma unroll
      for (int q = 0; q < NP; ++q) exp_pair(q);
    }
    l_run += psum0 + psum1;
    if constexpr (LSE) lf_run += f32sum0 + f32sum1;
    c = c_next;
  };
  for (int j = 0; j < n_stages; j += 2) {
    stage_body(j, lds_k0, lds_k1, lds_v1, lds_v0, pkB, pkA);
    if (j + 1 < n_stages) stage_body(j + 1, lds_k1, lds_k0, lds_v0, lds_v1, pkA, pkB);
  }
  // The last stage's PV product: V_{n-1} arrives with the copies of the last stage.
  wait_vmcnt<0>();
  if (n_stages > 0) {
    barrier_no_fence();
    if ((n_stages - 1) & 1) pv_product(lds_v1, pkB, no_step);
    else pv_product(lds_v0, pkA, no_step);
  }

  // ---- epilogue ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  float lf_tot = 0.0f;
  if constexpr (LSE) lf_tot = lf_run + __shfl_xor(lf_run, 32);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qtok >= 0) {
    u16* O = static_cast<u16*>(p.o) + (int64_t)it.head * p.head_stride + (int64_t)qtok * D;
#pragma unroll
    for (int u = 0; u < DT; ++u)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * u + 8 * g4 + 4 * h;
        const bf16x2 v01 = __builtin_convertvector(
            (f32x2){oacc[u][4 * g4 + 0] * inv, oacc[u][4 * g4 + 1] * inv}, bf16x2);
        const bf16x2 v23 = __builtin_convertvector(
            (f32x2){oacc[u][4 * g4 + 2] * inv, oacc[u][4 * g4 + 3] * inv}, bf16x2);
        *reinterpret_cast<uint2*>(O + d0) = make_uint2(bitcast<uint32_t>(v01), bitcast<uint32_t>(v23));
      }
    if constexpr (LSE) {
      if (h == 0)
        p.lse[(int64_t)it.head * n_tok + qtok] = lf_tot > 0.0f ? (m_run + __log2f(lf_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, int BLK>
hipError_t launch_typed(const AttnParams& p, hipStream_t s) {
  const int64_t items = attn_items(p);
  if (items == 0) return hipSuccess;
  if (p.lse) hipLaunchKernelGGL((attn_bf16_kernel<D, BLK, true>), dim3((unsigned)items), dim3(BLK * 2), 0, s, p);
  else hipLaunchKernelGGL((attn_bf16_kernel<D, BLK, false>), dim3((unsigned)items), dim3(BLK * 2), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnParams& p, int d, int blk, hipStream_t s) {
  if (d == 128 && blk == 128) return launch_typed<128, 128>(p, s);
  if (d == 64 && blk == 128) return launch_typed<64, 128>(p, s);
  if (d == 128 && blk == 64) return launch_typed<128, 64>(p, s);
  if (d == 64 && blk == 64) return launch_typed<64, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace calibatt
