// Block-sparse / anchor-row attention forward with fp32 arithmetic throughout.
//
// The correctness path for fp32 inputs: the same work items as the bf16 MFMA
// kernel (retained key blocks only, or all key blocks for anchor queries;
// papernotes.org notes on "Accelerating Text-to-Video Generation with
// Calibrated Sparse Attention", Key Designs 3 and 4), computed with fp32 FMA,
// expf and an online softmax. One thread owns one query; K and V tiles are
// staged in LDS and read as broadcasts.
#include "internal.h"

namespace calibatt {
namespace {

template <int BLK>
__device__ __forceinline__ int query_token_f32(const AttnParams& p, bool anchor, int tile, int qi) {
  if (!anchor) {
    const int tok = tile * BLK + qi;
    return tok < p.N ? tok : -1;
  }
  const int aq = tile * BLK + qi;
  if (aq >= p.n_anchor_q) return -1;
  const int per_frame = p.ka * p.C;
  const int f = aq / per_frame;
  const int rem = aq - f * per_frame;
  const int ai = rem / p.C;
  const int c = rem - ai * p.C;
  return (f * p.R + p.anchors[ai]) * p.C + c;
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK) void attn_f32_kernel(const AttnParams p) {
  extern __shared__ float smem[];
  float* ks = smem;                 // [BLK][D]
  float* vs = smem + BLK * D;       // [BLK][D]

  const int64_t item = blockIdx.x;
  const int64_t n_anchor_items = (int64_t)p.n_anchor * p.anchor_tiles;
  bool anchor;
  int head, tile, n;
  const int32_t* list;
  const uint32_t* runs = nullptr;
  const uint64_t* bits = nullptr;
  if (item < n_anchor_items) {
    anchor = true;
    head = p.anchor_heads[item / p.anchor_tiles];
    tile = (int)(item % p.anchor_tiles);
    list = nullptr;
    n = p.nb;
  } else {
    const int64_t j = item - n_anchor_items;
    anchor = false;
    head = p.sparse_heads[j / p.nb];
    const int rank = (int)(j % p.nb);
    const int64_t rec_row = p.rec_row0 + (int64_t)head * p.rec_head_rows;
    tile = rank;
    if (p.bits) {
      // bitmap form: visit the set bits word by word (n counts words)
      bits = p.bits + (rec_row + tile) * p.bm_words;
      list = nullptr;
      n = p.bm_words;
    } else {
      const int64_t b = p.row_ptr[rec_row + tile];
      list = p.runs ? nullptr : p.col_idx + b;
      runs = p.runs ? p.runs + b : nullptr;
      n = (int)(p.row_ptr[rec_row + tile + 1] - b);
    }
  }

  const float* Q = static_cast<const float*>(p.q) + (int64_t)head * p.head_stride;
  const float* K = static_cast<const float*>(p.k) + (int64_t)head * p.head_stride;
  const float* V = static_cast<const float*>(p.v) + (int64_t)head * p.head_stride;

  const int qtok = query_token_f32<BLK>(p, anchor, tile, threadIdx.x);
  float q[D], o[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    q[i] = qtok >= 0 ? Q[(int64_t)qtok * D + i] : 0.0f;
    o[i] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;

  // Visit key blocks run by run: a run of the interval form, or one block of
  // an index list (anchor items: every block); bitmap form: the set bits of
  // each word, ascending (bits past nb dropped).
  for (int step = 0; step < n; ++step) {
    const uint32_t w = runs ? runs[step] : 0u;
    uint64_t word = 0;
    if (bits) {
      word = bits[step];
      if (step == p.bm_words - 1 && (p.nb & 63)) word &= (1ull << (p.nb & 63)) - 1ull;
    }
    const int lo = runs ? (int)(w & 0xffffu) : (list ? list[step] : step);
    const int hi = runs ? (int)(w >> 16) : lo + 1;
    for (int c0 = bits ? 64 * step : lo; bits ? word != 0 : c0 < hi; ++c0) {
      int c = c0;
      if (bits) {
        c = 64 * step + __builtin_ctzll(word);
        word &= word - 1;
      }
      const int nk = min(BLK, p.N - c * BLK);
      __syncthreads();
      for (int e = threadIdx.x * 4; e < nk * D; e += BLK * 4) {
        *reinterpret_cast<float4*>(ks + e) = *reinterpret_cast<const float4*>(K + (int64_t)c * BLK * D + e);
        *reinterpret_cast<float4*>(vs + e) = *reinterpret_cast<const float4*>(V + (int64_t)c * BLK * D + e);
      }
      __syncthreads();
      for (int j = 0; j < nk; ++j) {
        float dot = 0.0f;
#pragma unroll
        for (int i = 0; i < D; ++i) dot = __builtin_fmaf(q[i], ks[j * D + i], dot);
        const float s = dot * p.scale;
        if (s > m) {
          const float a = expf(m - s);
          l *= a;
#pragma unroll
          for (int i = 0; i < D; ++i) o[i] *= a;
          m = s;
        }
        const float pj = expf(s - m);
        l += pj;
#pragma unroll
        for (int i = 0; i < D; ++i) o[i] = __builtin_fmaf(pj, vs[j * D + i], o[i]);
      }
    }
  }

  if (qtok >= 0) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* O = static_cast<float*>(p.o) + (int64_t)head * p.head_stride + (int64_t)qtok * D;
#pragma unroll
    for (int i = 0; i < D; ++i) O[i] = o[i] * inv;
    if (p.lse) p.lse[(int64_t)head * p.N + qtok] = l > 0.0f ? m + logf(l) : -INFINITY;
  }
}

template <int D, int BLK>
hipError_t launch_typed(const AttnParams& p, hipStream_t s) {
  const int64_t items = attn_items(p);
  if (items == 0) return hipSuccess;
  const size_t smem = (size_t)2 * BLK * D * sizeof(float);
  auto kern = attn_f32_kernel<D, BLK>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)items), dim3(BLK), smem, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnParams& p, int d, int blk, hipStream_t s) {
  if (d == 64 && blk == 64) return launch_typed<64, 64>(p, s);
  if (d == 128 && blk == 64) return launch_typed<128, 64>(p, s);
  if (d == 64 && blk == 128) return launch_typed<64, 128>(p, s);
  if (d == 128 && blk == 128) return launch_typed<128, 128>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace calibatt
