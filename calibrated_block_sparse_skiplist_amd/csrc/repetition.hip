// Spatial-repetition detection for calibration (papernotes.org notes on
// "Accelerating Text-to-Video Generation with Calibrated Sparse Attention",
// Key Design 3): the attention of each spatial row of a frame (its C tokens
// against all N keys, flattened) is compared by cosine similarity with the
// attention of its nearest anchor row; a head is repetitive when the mean over
// frames, non-anchor rows and prompts exceeds the threshold.
//
// For row r of frame f with nearest anchor a (ties to the smaller anchor):
//   sim = <P_r, P_a> / (|P_r| |P_a|),  <P_r, P_a> = sum_c sum_j P[(f,r,c)][j] P[(f,a,c)][j],
// P = softmax over all keys of scale * q . k, normalised with each query's
// log2-sum-exp from the first (log-sum-exp) pass. One workgroup per
// (head, frame, row): its waves own 32-column tiles of the row, compute the
// scores of the row's queries and of the anchor row's queries (the same
// columns) against one shared K stream, and accumulate the three sums per lane.
#include "gfx950_device.h"

namespace calibatt {
namespace {

using namespace dev;

constexpr int kPrefetch = 4;
constexpr int kWaves = 4;

// Nearest anchor row of r (ties to the smaller anchor).
__device__ __forceinline__ int nearest_anchor(const SimParams& p, int r) {
  int best = p.anchors[0];
  for (int i = 1; i < p.ka; ++i) {
    const int a = p.anchors[i];
    if (abs(r - a) < abs(r - best)) best = a;
  }
  return best;
}

template <int D>
__global__ __launch_bounds__(kWaves * 64) void similarity_bf16_kernel(const SimParams p) {
  constexpr int SUB = 64;
  constexpr int CPR = D / 8;
  constexpr int KT = SUB / 32;
  constexpr int DS = D / 16;
  constexpr int STAGE = SUB * CPR;
  constexpr int LPW = STAGE / 64 / kWaves;
  constexpr int RPI = 64 / CPR;

  __shared__ uint4 lds_k[2 * STAGE];
  __shared__ float red[kWaves][3];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  int n_tok = p.N;
  float scale_log2 = p.scale_log2;
  asm volatile("" : "+s"(n_tok), "+s"(scale_log2));

  const int64_t item = xcd_item(blockIdx.x, gridDim.x, 32);
  const int rows = p.F * p.R;
  const int head = p.heads[item / rows];
  const int fr = (int)(item % rows);
  const int f = fr / p.R, r = fr % p.R;
  const int a = nearest_anchor(p, r);
  float* out = p.row_sim + ((int64_t)head * p.F + f) * p.R + r;
  if (a == r) {                 // an anchor row: similarity with itself
    if (threadIdx.x == 0) *out = 1.0f;
    return;
  }
  const u16* Q = static_cast<const u16*>(p.q) + (int64_t)head * p.head_stride;
  const char* Kb = reinterpret_cast<const char*>(static_cast<const u16*>(p.k) + (int64_t)head * p.head_stride);
  const float* lse = p.lse2 + (int64_t)head * n_tok;

  const int dq = lane / CPR;
  const int dpos = lane % CPR;
  const uint32_t dma_lane = (uint32_t)(dq * 2 * D + 16 * (dpos ^ (dq & (CPR - 1))));
  const uint32_t k_lane = (uint32_t)(l32 * 2 * D + 16 * (h ^ (l32 & (CPR - 1))));
  auto issue = [&](int stage, int i, uint4* dst) {
    const int row0 = stage * SUB;
    const int rr = (wave * LPW + i) * RPI;
    const uint32_t off = dma_lane ^ (uint32_t)(16 * (rr & (CPR - 1)));
    if (row0 + SUB <= n_tok) {
      dma16(Kb + (int64_t)(row0 + rr) * (2 * D), off, dst + (wave * LPW + i) * 64);
    } else {
      asm volatile("");
      const int b0 = min(row0, n_tok - 1);
      const int grow = min(row0 + rr + dq, n_tok - 1);
      dma16(Kb + (int64_t)b0 * (2 * D), (uint32_t)((grow - b0) * (2 * D)) + (off & (2 * D - 1)),
            dst + (wave * LPW + i) * 64);
    }
  };

  const int n_stages = (n_tok + SUB - 1) / SUB;
  float dot_t = 0.0f, nr_t = 0.0f, na_t = 0.0f;   // thread 0: totals over column groups
  for (int c0 = 0; c0 < p.C; c0 += kWaves * 32) {
    // this wave's 32 columns; columns past C get lse = +inf (probabilities 0)
    const int c = c0 + wave * 32 + l32;
    const bool c_ok = c < p.C;
    const int tr = (f * p.R + r) * p.C + c, ta = (f * p.R + a) * p.C + c;
    const float lse_r = c_ok ? lse[tr] : INFINITY;
    const float lse_a = c_ok ? lse[ta] : INFINITY;
    bf16x8 qr[DS], qa[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0);
      if (c_ok) {
        x = ld_global16(Q + (int64_t)tr * D + 16 * s + 8 * h);
        y = ld_global16(Q + (int64_t)ta * D + 16 * s + 8 * h);
      }
      qr[s] = bitcast<bf16x8>(x);
      qa[s] = bitcast<bf16x8>(y);
    }
    if (c0 > 0) {             // the previous group's last stage is done everywhere
      wait_vmcnt<0>();
      barrier_no_fence();
    }
#pragma unroll
    for (int i = 0; i < LPW; ++i) issue(0, i, lds_k);
    float dot = 0.0f, nr = 0.0f, na = 0.0f;
    for (int j = 0; j < n_stages; ++j) {
      const uint4* sk = lds_k + (j & 1) * STAGE;
      uint4* nk = lds_k + ((j + 1) & 1) * STAGE;
      wait_vmcnt<0>();
      barrier_no_fence();
      const bool has_next = j + 1 < n_stages;
      f32x16 sr[KT], sa[KT];
      {
        auto read_k = [&](int idx) -> bf16x8 {
          const int t = idx / DS, s = idx % DS;
          const char* ptr = reinterpret_cast<const char*>(sk) + 32 * t * (2 * D) + (k_lane ^ (uint32_t)(32 * s));
          return bitcast<bf16x8>(*reinterpret_cast<const uint4*>(ptr));
        };
        constexpr int kEvery = (KT * DS) / LPW > 0 ? (KT * DS) / LPW : 1;
        bf16x8 ring[kPrefetch];
#pragma unroll
        for (int i = 0; i < kPrefetch; ++i) ring[i] = read_k(i);
#pragma unroll
        for (int idx = 0; idx < KT * DS; ++idx) {
          const int t = idx / DS, s = idx % DS;
          const bf16x8 kf = ring[idx % kPrefetch];
          if (idx + kPrefetch < KT * DS) ring[idx % kPrefetch] = read_k(idx + kPrefetch);
          sr[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qr[s], s == 0 ? f32x16{} : sr[t], 0, 0, 0);
          sa[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qa[s], s == 0 ? f32x16{} : sa[t], 0, 0, 0);
          if (has_next && idx % kEvery == kEvery - 1 && idx / kEvery < LPW) issue(j + 1, idx / kEvery, nk);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (has_next) {
#pragma unroll
          for (int i = (KT * DS) / kEvery; i < LPW; ++i) issue(j + 1, i, nk);
        }
      }
      const int valid = n_tok - j * SUB;
      if (valid < SUB) {
        int lv = valid - 4 * h;
        asm volatile("" : "+v"(lv));
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = 32 * t + 8 * (e >> 2) + (e & 3);
            if (key >= lv) {
              sr[t][e] = -INFINITY;
              sa[t][e] = -INFINITY;
            }
          }
      }
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sr[t][e], scale_log2, -lse_r));
          const float pa = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[t][e], scale_log2, -lse_a));
          dot = __builtin_fmaf(pr, pa, dot);
          nr = __builtin_fmaf(pr, pr, nr);
          na = __builtin_fmaf(pa, pa, na);
        }
    }
    // sum the wave's 64 lanes (both key halves of 32 columns), then the waves, in a fixed order
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      dot += __shfl_xor(dot, off);
      nr += __shfl_xor(nr, off);
      na += __shfl_xor(na, off);
    }
    if (lane == 0) {
      red[wave][0] = dot;
      red[wave][1] = nr;
      red[wave][2] = na;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 0; w < kWaves; ++w) {
        dot_t += red[w][0];
        nr_t += red[w][1];
        na_t += red[w][2];
      }
    }
  }
  if (threadIdx.x == 0) *out = dot_t / sqrtf(nr_t * na_t);
}

// fp32 inputs: one thread per column of the row pair, K tiles in LDS.
template <int D>
__global__ __launch_bounds__(64) void similarity_f32_kernel(const SimParams p) {
  constexpr int T = 64;                  // keys per LDS tile, columns per pass
  __shared__ float ks[T * D];
  __shared__ float red[T][3];
  const int rows = p.F * p.R;
  const int head = p.heads[blockIdx.x / rows];
  const int fr = (int)(blockIdx.x % rows);
  const int f = fr / p.R, r = fr % p.R;
  const int a = nearest_anchor(p, r);
  float* out = p.row_sim + ((int64_t)head * p.F + f) * p.R + r;
  if (a == r) {
    if (threadIdx.x == 0) *out = 1.0f;
    return;
  }
  const float* Q = static_cast<const float*>(p.q) + (int64_t)head * p.head_stride;
  const float* K = static_cast<const float*>(p.k) + (int64_t)head * p.head_stride;
  const float* lse = p.lse2 + (int64_t)head * p.N;
  const float ln2 = 0.6931471805599453f;
  float dot_t = 0.0f, nr_t = 0.0f, na_t = 0.0f;
  for (int c0 = 0; c0 < p.C; c0 += T) {
    const int c = c0 + threadIdx.x;
    const bool ok = c < p.C;
    const int tr = (f * p.R + r) * p.C + c, ta = (f * p.R + a) * p.C + c;
    float qr[D], qa[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {
      qr[i] = ok ? Q[(int64_t)tr * D + i] : 0.0f;
      qa[i] = ok ? Q[(int64_t)ta * D + i] : 0.0f;
    }
    const float lr = ok ? lse[tr] * ln2 : INFINITY, la = ok ? lse[ta] * ln2 : INFINITY;
    float dot = 0.0f, nr = 0.0f, na = 0.0f;
    for (int k0 = 0; k0 < p.N; k0 += T) {
      const int nk = min(T, p.N - k0);
      __syncthreads();
      for (int e = threadIdx.x; e < nk * D; e += T) ks[e] = K[(int64_t)k0 * D + e];
      __syncthreads();
      for (int j = 0; j < nk; ++j) {
        float sr = 0.0f, sa = 0.0f;
#pragma unroll
        for (int i = 0; i < D; ++i) {
          sr = __builtin_fmaf(qr[i], ks[j * D + i], sr);
          sa = __builtin_fmaf(qa[i], ks[j * D + i], sa);
        }
        const float pr = expf(sr * p.scale - lr), pa = expf(sa * p.scale - la);
        dot = __builtin_fmaf(pr, pa, dot);
        nr = __builtin_fmaf(pr, pr, nr);
        na = __builtin_fmaf(pa, pa, na);
      }
    }
    red[threadIdx.x][0] = dot;
    red[threadIdx.x][1] = nr;
    red[threadIdx.x][2] = na;
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int t = 0; t < T; ++t) {
        dot_t += red[t][0];
        nr_t += red[t][1];
        na_t += red[t][2];
      }
    }
  }
  if (threadIdx.x == 0) *out = dot_t / sqrtf(nr_t * na_t);
}

// One thread per head: mean over prompts, frames and non-anchor rows (double,
// fixed order), flag = mean > threshold.
__global__ void flags_kernel(const float* __restrict__ sims, int P, int H, int F, int R, const RepFlagParams q,
                             uint8_t* __restrict__ flags, float* __restrict__ mean) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  double acc = 0.0;
  int64_t n = 0;
  for (int pr = 0; pr < P; ++pr)
    for (int f = 0; f < F; ++f)
      for (int r = 0; r < R; ++r) {
        bool anchor = false;
        for (int i = 0; i < q.ka; ++i) anchor |= q.anchors[i] == r;
        if (anchor) continue;
        acc += (double)sims[(((int64_t)pr * H + h) * F + f) * R + r];
        ++n;
      }
  const double m = acc / (double)n;
  if (flags) flags[h] = m > (double)q.threshold ? 1 : 0;
  if (mean) mean[h] = (float)m;
}

}  // namespace

hipError_t launch_similarity(const SimParams& p, int d, bool f32, hipStream_t s) {
  const int64_t items = (int64_t)p.n_heads * p.F * p.R;
  if (items == 0) return hipSuccess;
  if (f32) {
    if (d == 128) hipLaunchKernelGGL(similarity_f32_kernel<128>, dim3((unsigned)items), dim3(64), 0, s, p);
    else if (d == 64) hipLaunchKernelGGL(similarity_f32_kernel<64>, dim3((unsigned)items), dim3(64), 0, s, p);
    else return hipErrorInvalidValue;
  } else {
    if (d == 128) hipLaunchKernelGGL(similarity_bf16_kernel<128>, dim3((unsigned)items), dim3(kWaves * 64), 0, s, p);
    else if (d == 64) hipLaunchKernelGGL(similarity_bf16_kernel<64>, dim3((unsigned)items), dim3(kWaves * 64), 0, s, p);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rep_flags(const float* sims, int P, int H, int F, int R, const RepFlagParams& q, uint8_t* flags,
                            float* mean, hipStream_t s) {
  hipLaunchKernelGGL(flags_kernel, dim3((unsigned)((H + 63) / 64)), dim3(64), 0, s, sims, P, H, F, R, q, flags, mean);
  return hipGetLastError();
}

}  // namespace calibatt
