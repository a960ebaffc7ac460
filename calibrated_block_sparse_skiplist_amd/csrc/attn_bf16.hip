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
// CU (register budget capped at 256 per lane, 64 KB of LDS each), so one
// workgroup's softmax overlaps the other's matrix work. For every listed key
// block c each wave
//   1. computes S^T = K_c Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS,
//      B = Q^T held in registers): every lane owns one query column and half
//      of the keys, so a row maximum needs one exchange with lane ^ 32;
//   2. runs the online softmax in fp32: exp2 with log2(e) folded into the
//      scale, per-lane partial row sums of the bf16-rounded probabilities that
//      also feed the PV product, and a rescale of O only when some row maximum
//      grows by more than 2^8 (the stale maximum is exact algebra: numerator
//      and denominator share it);
//   3. accumulates O^T += V_c^T P^T with the same MFMA: A = V^T read from
//      row-major LDS by ds_read_b64_tr_b16 (16-bit transpose across 16-lane
//      groups), B = P^T packed to bf16 straight from the S^T accumulators; the
//      contraction runs over keys in the order the accumulator layout holds
//      them, and V is read in that same order.
// K and V tiles move HBM -> LDS with global_load_lds_dwordx4 (no register
// staging). The next block's K is fetched while this block's softmax and PV
// run, and the next V while the next S^T runs; s_waitcnt vmcnt plus a
// workgroup barrier publish each tile.
//
// LDS rows are XOR-swizzled in 16-byte chunks: K by (row & 15), so the 16
// rows of an MFMA operand read hit distinct banks; V by 4*(row & 3), so the
// 8-row x 64-byte patch of a transposed read spreads over all banks.
#include "internal.h"

namespace calibatt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;   // log2 units: stale maxima are allowed 2^8 headroom
constexpr int kPrefetchK = 4;               // K operand reads in flight ahead of their MFMA
constexpr int kPrefetchV = 3;               // V operand reads (2 instructions each) in flight
constexpr int kListCap = CALIBATT_MAX_NB;   // key-block indices staged in LDS per item (all of them)

template <int CPR>
__device__ __forceinline__ int swz_k(int row) { return row & (CPR - 1); }
template <int CPR>
__device__ __forceinline__ int swz_v(int row) { return (4 * (row & 3)) & (CPR - 1); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence. __syncthreads() fences, and a
// workgroup fence must drain every outstanding vector-memory operation,
// including the LDS DMA prefetch of the next tile; here each wave instead
// waits for its own DMA with wait_vmcnt before the barrier, and its LDS reads
// have returned (lgkmcnt 0). The memory clobber keeps LDS accesses on their
// side of the barrier.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint4 ld_global16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

template <typename T, typename S>
__device__ __forceinline__ T bitcast(const S& s) {
  static_assert(sizeof(T) == sizeof(S), "size");
  T t;
  __builtin_memcpy(&t, &s, sizeof(T));
  return t;
}

struct Item {
  int head;
  bool anchor;
  int tile;           // query block (sparse) or anchor tile
  const int32_t* list;
  int n;              // number of key blocks to visit
};

// Logical item of grid block b. Workgroups go round-robin over the 8 XCDs;
// each run of 8*G grid blocks gives XCD x the G consecutive items
// [run*8G + x*G, run*8G + (x+1)*G). The last, partial run keeps grid order.
__device__ __forceinline__ int64_t xcd_item(int64_t b, int64_t total, int G) {
  if (G <= 0) return b;
  const int64_t run = b / (8 * (int64_t)G);
  if ((run + 1) * 8 * (int64_t)G > total) return b;
  const int64_t s = b - run * 8 * (int64_t)G;
  return run * 8 * (int64_t)G + (s % 8) * G + s / 8;
}

__device__ __forceinline__ Item decode_item(const AttnParams& p, int64_t item) {
  Item it;
  const int64_t n_anchor_items = (int64_t)p.n_anchor * p.anchor_tiles;
  if (item < n_anchor_items) {
    it.anchor = true;
    it.head = p.anchor_heads[item / p.anchor_tiles];
    it.tile = (int)(item % p.anchor_tiles);
    it.list = nullptr;
    it.n = p.nb;
  } else {
    const int64_t j = item - n_anchor_items;
    const int hi = (int)(j / p.nb);
    const int rank = (int)(j % p.nb);
    it.anchor = false;
    it.head = p.sparse_heads[hi];
    const int64_t rec_row = p.rec_row0 + (int64_t)it.head * p.rec_head_rows;
    it.tile = (p.order && p.use_order) ? p.order[rec_row + rank] : rank;
    const int64_t b = p.row_ptr[rec_row + it.tile];
    const int64_t e = p.row_ptr[rec_row + it.tile + 1];
    it.list = p.col_idx + b;
    it.n = (int)(e - b);
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

// One 16-byte HBM -> LDS copy (global_load_lds_dwordx4): lane l's chunk lands
// in slot l of the 64-slot window at `lds` (LDS address = M0 + 16 * lane).
// The source is a uniform base (SGPR pair) plus this lane's 32-bit offset.
//
// Issued as inline assembly on purpose. The compiler does not know which LDS
// bytes the copy writes, so after the builtin form it turns every later LDS
// operand wait into lgkmcnt(0), serialising the MFMA operand reads. The
// hardware counts these copies in vmcnt only; the kernel waits for them
// explicitly (wait_vmcnt) before the barrier that publishes a stage. The
// statement has no register outputs, M0 is set inside it, and the memory
// clobber keeps it after the barrier that frees the destination buffer.
__device__ __forceinline__ void dma16(const char* base, uint32_t off, uint4* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void*)lds;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" :: "s"(m0), "v"(off), "s"(base) : "memory");
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(const AttnParams p) {
  constexpr int NW = BLK / 32;           // waves per workgroup (32 queries each)
  constexpr int SUB = 64;                // keys per pipeline stage
  constexpr int SPB = BLK / SUB;         // stages per key block
  constexpr int CPR = D / 8;             // 16-byte chunks per K/V row
  constexpr int KT = SUB / 32;           // 32-key tiles of S^T per stage
  constexpr int DS = D / 16;             // 16-wide d slabs (QK contraction)
  constexpr int DT = D / 32;             // 32-wide d tiles of O^T
  constexpr int KS = SUB / 16;           // 16-key slabs (PV contraction)
  constexpr int STAGE = SUB * CPR;       // 16-byte slots per stage and tensor
  constexpr int LPW = STAGE / 64 / NW;   // DMA instructions per wave, tensor and stage
  constexpr int RPI = 64 / CPR;          // rows per DMA instruction

  // Two stages of K and of V (double buffer) and the item's key-block list.
  // Each buffer is its own LDS object so that the compiler can see that reading
  // one stage never aliases the DMA filling the other (otherwise it drains the
  // DMA queue before every LDS read).
  __shared__ uint4 lds_k0[STAGE], lds_k1[STAGE];
  __shared__ uint4 lds_v0[STAGE], lds_v1[STAGE];
  __shared__ uint16_t lds_list[kListCap];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;               // half of the wave
  const int l32 = lane & 31;

  const Item it = decode_item(p, xcd_item(blockIdx.x, gridDim.x, p.xcd_group));
  // Scalars used inside the loop, pinned in registers: if the compiler reloads
  // them from the kernel arguments, each scalar load (which returns out of
  // order) forces every following LDS wait to drain completely.
  int n_tok = p.N;
  float scale_log2 = p.scale_log2;
  asm volatile("" : "+s"(n_tok), "+s"(scale_log2));
  const u16* Q = static_cast<const u16*>(p.q) + (int64_t)it.head * p.head_stride;
  const char* Kb = reinterpret_cast<const char*>(static_cast<const u16*>(p.k) + (int64_t)it.head * p.head_stride);
  const char* Vb = reinterpret_cast<const char*>(static_cast<const u16*>(p.v) + (int64_t)it.head * p.head_stride);

  // The item's key-block list goes to LDS once (n <= nb <= CALIBATT_MAX_NB, as
  // the host checks), so the loop reads indices with LDS broadcasts instead of
  // vector-memory loads, which would join the vmcnt queue of the prefetch.
  if (it.list) {
    for (int i = threadIdx.x; i < it.n; i += NW * 64) lds_list[i] = (uint16_t)it.list[i];
  }

  // Q^T operand fragments: query = wave*32 + l32, d = 16*s + 8*h + [0, 8).
  const int qtok = query_token(p, it, wave * 32 + l32, BLK);
  bf16x8 qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (qtok >= 0) raw = ld_global16(Q + (int64_t)qtok * D + 16 * s + 8 * h);
    qf[s] = bitcast<bf16x8>(raw);
  }

  // DMA geometry of this lane: stage row and swizzled source chunk of each of
  // its LPW instructions (byte offsets inside a stage of SUB rows).
  uint32_t off_k[LPW], off_v[LPW];
  int row_of[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = (wave * LPW + i) * RPI + lane / CPR;
    const int pos = lane % CPR;
    row_of[i] = row;
    off_k[i] = (uint32_t)(row * D + (pos ^ swz_k<CPR>(row)) * 8) * 2u;
    off_v[i] = (uint32_t)(row * D + (pos ^ swz_v<CPR>(row)) * 8) * 2u;
  }
  __syncthreads();

  // Sources of the copy of stage `half` of key block c: a uniform base per
  // tensor plus this lane's offsets. Rows past the end of the sequence (last
  // block only) read the last token instead: their scores are masked and their
  // probabilities are exactly 0.
  // On the last block the base row is min(row0, N-1) and clamped lane offsets
  // are taken from it, so every offset stays non-negative (the 32-bit lane
  // offset of the copy instruction is unsigned).
  struct StageSrc { const char* k; const char* v; bool clamp; int row0; int base_row; };
  auto stage_src = [&](int c, int half) -> StageSrc {
    const int row0 = c * BLK + half * SUB;
    const int b0 = min(row0, n_tok - 1);
    return {Kb + (int64_t)b0 * (D * 2), Vb + (int64_t)b0 * (D * 2), row0 + SUB > n_tok, row0, b0};
  };
  // DMA instruction i (0 <= i < 2*LPW) of this wave for a stage: K first, then V.
  auto issue_one = [&](const StageSrc& src, int i, uint4* lk, uint4* lv) {
    const int ii = i % LPW;
    uint32_t off = i < LPW ? off_k[ii] : off_v[ii];
    if (src.clamp) {
      const int grow = min(src.row0 + row_of[ii], n_tok - 1);
      off = off - (uint32_t)(row_of[ii] * (D * 2)) + (uint32_t)((grow - src.base_row) * (D * 2));
    }
    uint4* dst = (i < LPW ? lk : lv) + (wave * LPW + ii) * 64;
    dma16(i < LPW ? src.k : src.v, off, dst);
  };

  // Key block visited at step i (uniform across the workgroup).
  auto block_at = [&](int i) -> int {
    return it.list ? __builtin_amdgcn_readfirstlane((int)lds_list[i]) : i;
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int u = 0; u < DT; ++u) oacc[u] = f32x16{};
  float m_run = -INFINITY;   // reference maximum of scaled scores (log2 units)
  float l_run = 0.0f;        // this lane's partial sum of probabilities

  const int n_stages = it.n * SPB;
  int c = n_stages > 0 ? block_at(0) : 0;
  if (n_stages > 0) {
    const StageSrc src0 = stage_src(c, 0);
#pragma unroll
    for (int i = 0; i < 2 * LPW; ++i) issue_one(src0, i, lds_k0, lds_v0);
  }

  // Stage j lives in buffer j & 1; the loop body is instantiated per buffer.
  auto stage_body = [&](int j, const uint4* sk, const uint4* svv, uint4* nk, uint4* nv) {
    const int half = j % SPB;
    const bool has_next = j + 1 < n_stages;
    const int c_next = (has_next && half == SPB - 1) ? block_at(j / SPB + 1) : c;

    // ---- stage j resident in every wave's view; the other buffer is free ----
    wait_vmcnt<0>();
    barrier_no_fence();
    // The copy of stage j+1 is issued in small steps between the MFMAs below,
    // so the address unit streams it while the matrix pipe works instead of
    // every wave stalling on a burst right after the barrier.
    const StageSrc nsrc = stage_src(has_next ? c_next : c, (j + 1) % SPB);

    const int valid = n_tok - (c * BLK + half * SUB);   // keys of this stage inside the sequence
    if (valid > 0) {
      // Lane-dependent parts of the LDS operand addresses (loop-invariant; the
      // compiler keeps them in registers, the per-step parts are immediates).
      const int lo32 = l32;
      const int lh = h;
      const int g = lane >> 4;        // 16-lane group of the transposed reads
      const int jj = lane & 15;
      const char* sv = reinterpret_cast<const char*>(svv);

      // ---- S^T = K Q^T: operand reads run kPrefetchK MFMAs ahead ----
      f32x16 sacc[KT];
      {
        auto read_k = [&](int idx) -> bf16x8 {
          const int t = idx / DS, s = idx % DS;
          const int key = 32 * t + lo32;
          const int ch = 2 * s + lh;
          return bitcast<bf16x8>(sk[key * CPR + (ch ^ swz_k<CPR>(key))]);
        };
        bf16x8 ring[kPrefetchK];
#pragma unroll
        for (int i = 0; i < kPrefetchK; ++i) ring[i] = read_k(i);
#pragma unroll
        for (int idx = 0; idx < KT * DS; ++idx) {
          const int t = idx / DS, s = idx % DS;
          const bf16x8 a = ring[idx % kPrefetchK];
          if (idx + kPrefetchK < KT * DS) ring[idx % kPrefetchK] = read_k(idx + kPrefetchK);
          sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], s == 0 ? f32x16{} : sacc[t], 0, 0, 0);
          constexpr int kDmaEvery = (KT * DS) / (2 * LPW) > 0 ? (KT * DS) / (2 * LPW) : 1;
          if (has_next && idx % kDmaEvery == kDmaEvery - 1 && idx / kDmaEvery < 2 * LPW)
            issue_one(nsrc, idx / kDmaEvery, nk, nv);
          __builtin_amdgcn_sched_barrier(0);   // keep the read-ahead order as written
        }
        // (copies that did not fit between the MFMAs, if any)
        if (has_next) {
#pragma unroll
          for (int i = (KT * DS) / ((KT * DS) / (2 * LPW) > 0 ? (KT * DS) / (2 * LPW) : 1); i < 2 * LPW; ++i)
            issue_one(nsrc, i, nk, nv);
        }
      }

      // ---- mask keys past N (partial stage of the last block) ----
      if (valid < SUB) {
        // (opaque bound: keeps the comparisons inside this rarely taken branch)
        int lv = valid - 4 * lh;
        asm volatile("" : "+v"(lv));
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
          for (int a = 0; a < 16; ++a) {
            const int key = 32 * t + 8 * (a >> 2) + (a & 3);
            if (key >= lv) sacc[t][a] = -INFINITY;
          }
      }

      // ---- online softmax (fp32, log2 domain, lazy rescale) ----
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int a = 0; a < 16; ++a) mx = fmaxf(mx, sacc[t][a]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mb = mx * scale_log2;
      if (__ballot(mb > m_run + kRescaleThreshold) != 0) {
        const float m_new = fmaxf(m_run, mb);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m_run is -inf
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int u = 0; u < DT; ++u)
#pragma unroll
          for (int a = 0; a < 16; ++a) oacc[u][a] *= alpha;
      }
      // Probabilities go to bf16 in pairs; the row sum adds those same bf16
      // values (v_dot2 against 1.0), so numerator and denominator of O use
      // identical weights.
      const float neg_m = -m_run;
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      float psum0 = 0.0f, psum1 = 0.0f;
      uint32_t pk[KS][4];
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int a = 0; a < 16; a += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][a], scale_log2, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][a + 1], scale_log2, neg_m));
          const bf16x2 two = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
          if ((a >> 1) & 1) psum1 = __builtin_amdgcn_fdot2_f32_bf16(two, ones, psum1, false);
          else psum0 = __builtin_amdgcn_fdot2_f32_bf16(two, ones, psum0, false);
          pk[2 * t + (a >> 3)][(a & 7) >> 1] = bitcast<uint32_t>(two);
        }
      l_run += psum0 + psum1;

      // ---- O^T += V^T P^T: transposed reads run kPrefetchV MFMAs ahead ----
      {
        auto read_v = [&](int idx) -> bf16x8 {
          const int sl = idx / DT, u = idx % DT;
          const int key_lo = 16 * sl + 4 * (g >> 1) + (jj >> 2);
          const int key_hi = key_lo + 8;
          const int dcol = 32 * u + 16 * (g & 1) + 4 * (jj & 3);
          const int ch = dcol >> 3;
          const int hb = (dcol >> 2) & 1;
          struct { i16x4 lo, hi; } both;
          both.lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(sv + (key_lo * CPR + (ch ^ swz_v<CPR>(key_lo))) * 16 + hb * 8));
          both.hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(sv + (key_hi * CPR + (ch ^ swz_v<CPR>(key_hi))) * 16 + hb * 8));
          return bitcast<bf16x8>(both);
        };
        bf16x8 ring[kPrefetchV];
#pragma unroll
        for (int i = 0; i < kPrefetchV; ++i) ring[i] = read_v(i);
#pragma unroll
        for (int idx = 0; idx < KS * DT; ++idx) {
          const int sl = idx / DT, u = idx % DT;
          const bf16x8 a = ring[idx % kPrefetchV];
          if (idx + kPrefetchV < KS * DT) ring[idx % kPrefetchV] = read_v(idx + kPrefetchV);
          oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bitcast<bf16x8>(pk[sl]), oacc[u], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);   // keep the read-ahead order as written
        }
      }
    } else if (has_next) {
      // fully padded stage: nothing to compute, only the next copy to issue
#pragma unroll
      for (int i = 0; i < 2 * LPW; ++i) issue_one(nsrc, i, nk, nv);
    }
    c = c_next;
  };
  for (int j = 0; j < n_stages; j += 2) {
    stage_body(j, lds_k0, lds_v0, lds_k1, lds_v1);
    if (j + 1 < n_stages) stage_body(j + 1, lds_k1, lds_v1, lds_k0, lds_v0);
  }

  // ---- epilogue ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
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
    if (p.lse && h == 0) {
      p.lse[(int64_t)it.head * n_tok + qtok] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, int BLK>
hipError_t launch_typed(const AttnParams& p, hipStream_t s) {
  const int64_t items = attn_items(p);
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_bf16_kernel<D, BLK>), dim3((unsigned)items), dim3(BLK * 2), 0, s, p);
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
