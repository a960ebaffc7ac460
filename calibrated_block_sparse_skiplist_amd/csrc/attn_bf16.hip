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
//      scale, per-lane partial row sums, and a rescale of O only when some row
//      maximum grows by more than 2^8 (the stale maximum is exact algebra:
//      numerator and denominator share it);
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
    it.tile = p.order ? p.order[rec_row + rank] : rank;
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

// Issue this wave's share of the HBM -> LDS copy of one BLK x D tile. Each
// instruction fills 64 consecutive 16-byte LDS slots; lane l fetches the global
// chunk that the swizzle places in slot l. Rows past the sequence end are
// clamped to a valid row (their scores are masked, their probabilities are 0).
template <int D, int BLK, int NW, bool IS_V>
__device__ __forceinline__ void issue_tile(const u16* head_base, int c, int N, uint4* lds, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int LPW = BLK * CPR / 64 / NW;     // load instructions per wave
  constexpr int RPI = 64 / CPR;                // rows per instruction
  const u16* tile = head_base + (int64_t)c * BLK * D;
  const int last_row = N - 1 - c * BLK;
  const int pos = lane % CPR;
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int inst = wave * LPW + i;
    const int row = inst * RPI + lane / CPR;
    const int ch = pos ^ (IS_V ? swz_v<CPR>(row) : swz_k<CPR>(row));
    const u16* src = tile + min(row, last_row) * D + ch * 8;
    __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds + inst * 64), 16, 0, 0);
  }
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bf16_kernel(const AttnParams p) {
  constexpr int NW = BLK / 32;           // waves per workgroup
  constexpr int CPR = D / 8;             // 16-byte chunks per K/V row
  constexpr int KT = BLK / 32;           // 32-key tiles of S^T per block
  constexpr int DS = D / 16;             // 16-wide d slabs (QK contraction)
  constexpr int DT = D / 32;             // 32-wide d tiles of O^T
  constexpr int KS = BLK / 16;           // 16-key slabs (PV contraction)
  constexpr int LPW = BLK * CPR / 64 / NW;

  __shared__ uint4 lds_k[BLK * CPR];
  __shared__ uint4 lds_v[BLK * CPR];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;               // half of the wave
  const int l32 = lane & 31;

  const Item it = decode_item(p, blockIdx.x);
  const u16* Q = static_cast<const u16*>(p.q) + (int64_t)it.head * p.head_stride;
  const u16* K = static_cast<const u16*>(p.k) + (int64_t)it.head * p.head_stride;
  const u16* V = static_cast<const u16*>(p.v) + (int64_t)it.head * p.head_stride;

  // Q^T operand fragments: query = wave*32 + l32, d = 16*s + 8*h + [0, 8).
  const int qtok = query_token(p, it, wave * 32 + l32, BLK);
  bf16x8 qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (qtok >= 0) raw = ld_global16(Q + (int64_t)qtok * D + 16 * s + 8 * h);
    qf[s] = bitcast<bf16x8>(raw);
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int u = 0; u < DT; ++u) oacc[u] = f32x16{};
  float m_run = -INFINITY;   // reference maximum of scaled scores (log2 units)
  float l_run = 0.0f;        // this lane's partial sum of probabilities

  const int last_valid = p.N - (p.nb - 1) * BLK;   // tokens in the last block

  if (it.n > 0) {
    const int c0 = it.list ? it.list[0] : 0;
    issue_tile<D, BLK, NW, false>(K, c0, p.N, lds_k, wave, lane);
    issue_tile<D, BLK, NW, true>(V, c0, p.N, lds_v, wave, lane);
  }

  for (int step = 0; step < it.n; ++step) {
    const int c = it.list ? it.list[step] : step;
    // Lane-dependent LDS and tile addresses are rebuilt from an opaque copy of
    // the lane id every iteration: hoisted out of the loop they would need
    // ~30 extra registers and spill at two workgroups per CU.
    int lo = lane;
    asm volatile("" : "+v"(lo));
    const int lo32 = lo & 31;
    const int lh = lo >> 5;
    const int g = lo >> 4;          // 16-lane group of the transposed reads
    const int j = lo & 15;
    const bool has_next = step + 1 < it.n;
    const int cn = has_next ? (it.list ? it.list[step + 1] : step + 1) : 0;

    // ---- K_c resident (this wave's V_c loads may still be in flight) ----
    wait_vmcnt<LPW>();
    __syncthreads();

    // ---- S^T = K Q^T ----
    f32x16 sacc[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      sacc[t] = f32x16{};
      const int key = 32 * t + lo32;
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const int ch = 2 * s + lh;
        bf16x8 a = bitcast<bf16x8>(lds_k[key * CPR + (ch ^ swz_k<CPR>(key))]);
        sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[t], 0, 0, 0);
      }
    }
    __syncthreads();                              // every wave is done reading K_c
    if (has_next) issue_tile<D, BLK, NW, false>(K, cn, p.N, lds_k, wave, lo);

    // ---- mask keys past N in a partial last block ----
    if (c == p.nb - 1 && last_valid < BLK) {
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const int key = 32 * t + 8 * (a >> 2) + 4 * h + (a & 3);
          if (key >= last_valid) sacc[t][a] = -INFINITY;
        }
    }

    // ---- online softmax (fp32, log2 domain, lazy rescale) ----
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int a = 0; a < 16; ++a) mx = fmaxf(mx, sacc[t][a]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mb = mx * p.scale_log2;
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
    const float neg_m = -m_run;
    float psum = 0.0f;
    uint32_t pk[KS][4];
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int a = 0; a < 16; a += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][a], p.scale_log2, neg_m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][a + 1], p.scale_log2, neg_m));
        psum += p0;
        psum += p1;
        const bf16x2 two = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
        pk[2 * t + (a >> 3)][(a & 7) >> 1] = bitcast<uint32_t>(two);
      }
    l_run += psum;

    // ---- V_c resident ----
    if (has_next) wait_vmcnt<LPW>(); else wait_vmcnt<0>();
    __syncthreads();

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int sl = 0; sl < KS; ++sl) {
      const bf16x8 b = bitcast<bf16x8>(pk[sl]);
      const int key_lo = 16 * sl + 4 * (g >> 1) + (j >> 2);
      const int key_hi = key_lo + 8;
#pragma unroll
      for (int u = 0; u < DT; ++u) {
        const int dcol = 32 * u + 16 * (g & 1) + 4 * (j & 3);
        const int ch = dcol >> 3;
        const int half = (dcol >> 2) & 1;
        const char* base = reinterpret_cast<const char*>(lds_v);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(base + (key_lo * CPR + (ch ^ swz_v<CPR>(key_lo))) * 16 + half * 8));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(base + (key_hi * CPR + (ch ^ swz_v<CPR>(key_hi))) * 16 + half * 8));
        struct { i16x4 lo, hi; } both = {lo, hi};
        oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(both), b, oacc[u], 0, 0, 0);
      }
    }
    __syncthreads();                              // every wave is done reading V_c
    if (has_next) issue_tile<D, BLK, NW, true>(V, cn, p.N, lds_v, wave, lo);
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
      p.lse[(int64_t)it.head * p.N + qtok] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
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
