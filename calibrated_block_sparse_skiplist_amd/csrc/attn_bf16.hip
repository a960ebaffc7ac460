// Block-sparse / anchor-row attention forward, bf16 inputs, for gfx950.
//
// Retained key blocks are computed densely from the current Q, K, V and the
// others are skipped (papernotes.org notes on "Accelerating Text-to-Video
// Generation with Calibrated Sparse Attention", Overall Architecture and Key
// Design 4). Anchor-row heads run the same core over gathered anchor queries
// and every key block (same notes, Key Design 3).
//
// Work decomposition. One workgroup owns one work item: a tile of BLK queries
// of one head. Its BLK/32 waves own 32 queries each. For every listed key
// block the workgroup stages K and V (BLK x D bf16 each) in LDS and each wave
//   1. computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS,
//      B = Q^T held in registers), so every lane owns one query column and
//      half of the keys: row maxima need one cross-lane exchange (lane ^ 32);
//   2. runs the online softmax in fp32 (exp2 with log2(e) folded into the
//      scale, running max and per-lane partial sums);
//   3. accumulates O^T += V^T P^T with the same MFMA: A = V^T read from
//      row-major LDS with ds_read_b64_tr_b16 (transposing 16-bit elements
//      across 16-lane groups), B = P^T converted to bf16 straight from the
//      S^T accumulators. The MFMA contraction index runs over keys in the
//      order the accumulator layout produces; V is read in that same order.
// The epilogue divides by the row sum and writes bf16 O (and fp32 lse).
//
// LDS rows of K and V are XOR-swizzled in 16-byte chunks so that the MFMA
// operand reads of 32 consecutive keys (K) and of 4-key x 64-byte patches (V)
// spread over the banks.
#include "internal.h"

namespace calibatt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// LDS chunk swizzles (chunk = 16 bytes; CPR chunks per row).
template <int CPR>
__device__ __forceinline__ int swz_k(int row) { return row & (CPR - 1); }
template <int CPR>
__device__ __forceinline__ int swz_v(int row) { return ((row & 3) << 1) & (CPR - 1); }

__device__ __forceinline__ uint4 ld_global16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
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

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void attn_bf16_kernel(const AttnParams p) {
  constexpr int NW = BLK / 32;           // waves per workgroup
  constexpr int NT = NW * 64;            // threads
  constexpr int CPR = D / 8;             // 16-byte chunks per K/V row
  constexpr int KT = BLK / 32;           // 32-key tiles of S^T per block
  constexpr int DS = D / 16;             // 16-wide d slabs (QK contraction)
  constexpr int DT = D / 32;             // 32-wide d tiles of O^T
  constexpr int KS = BLK / 16;           // 16-key slabs (PV contraction)
  static_assert(NT == BLK * 2, "one wave per 32 queries");

  __shared__ uint4 lds_k[BLK * CPR];
  __shared__ uint4 lds_v[BLK * CPR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
    qf[s] = as_bf16x8(raw);
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int u = 0; u < DT; ++u) oacc[u] = f32x16{};
  float m_run = -INFINITY;   // running max of scaled scores (log2 units)
  float l_run = 0.0f;        // this lane's partial sum of probabilities

  const int last_valid = p.N - (p.nb - 1) * BLK;   // tokens in the last block

  for (int step = 0; step < it.n; ++step) {
    const int c = it.list ? it.list[step] : step;

    // ---- stage K_c and V_c into LDS (row-major, chunk-swizzled) ----
    __syncthreads();
#pragma unroll
    for (int i = 0; i < BLK * CPR / NT; ++i) {
      const int pidx = tid + i * NT;
      const int row = pidx / CPR;
      const int ch = pidx % CPR;
      const int grow = min(c * BLK + row, p.N - 1);
      const int64_t goff = (int64_t)grow * D + ch * 8;
      lds_k[row * CPR + (ch ^ swz_k<CPR>(row))] = ld_global16(K + goff);
      lds_v[row * CPR + (ch ^ swz_v<CPR>(row))] = ld_global16(V + goff);
    }
    __syncthreads();

    // ---- S^T = K Q^T ----
    f32x16 sacc[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      sacc[t] = f32x16{};
      const int key = 32 * t + l32;
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const int ch = 2 * s + h;
        bf16x8 a = as_bf16x8(lds_k[key * CPR + (ch ^ swz_k<CPR>(key))]);
        sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[t], 0, 0, 0);
      }
    }

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

    // ---- online softmax (fp32, log2 domain) ----
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int a = 0; a < 16; ++a) mx = fmaxf(mx, sacc[t][a]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * p.scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first block
    m_run = m_new;
    float psum = 0.0f;
    bf16x8 pf[KS];
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][a], p.scale_log2, -m_new));
        psum += pv;
        pf[2 * t + (a >> 3)][a & 7] = static_cast<__bf16>(pv);
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int u = 0; u < DT; ++u)
#pragma unroll
      for (int a = 0; a < 16; ++a) oacc[u][a] *= alpha;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int u = 0; u < DT; ++u) {
#pragma unroll
      for (int sl = 0; sl < KS; ++sl) {
        const int g = lane >> 4;
        const int j = lane & 15;
        const int dcol = 32 * u + 16 * (g & 1) + 4 * (j & 3);
        const int ch = dcol >> 3;
        const int half = (dcol >> 2) & 1;
        i16x4 lo, hi;
        {
          const int key = 16 * sl + 4 * (g >> 1) + (j >> 2);
          const char* base = reinterpret_cast<const char*>(lds_v) + (key * CPR + (ch ^ swz_v<CPR>(key))) * 16 + half * 8;
          lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)base);
        }
        {
          const int key = 16 * sl + 8 + 4 * (g >> 1) + (j >> 2);
          const char* base = reinterpret_cast<const char*>(lds_v) + (key * CPR + (ch ^ swz_v<CPR>(key))) * 16 + half * 8;
          hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)base);
        }
        bf16x8 a;
        __builtin_memcpy(&a, &lo, 8);
        __builtin_memcpy(reinterpret_cast<char*>(&a) + 8, &hi, 8);
        oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[sl], oacc[u], 0, 0, 0);
      }
    }
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
        __bf16 vals[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) vals[i] = static_cast<__bf16>(oacc[u][4 * g4 + i] * inv);
        uint2 packed;
        __builtin_memcpy(&packed, vals, 8);
        *reinterpret_cast<uint2*>(O + d0) = packed;
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
