// Spatial-repetition detection for calibration (papernotes.org notes on
// "Accelerating Text-to-Video Generation with Calibrated Sparse Attention",
// Key Design 3): the attention of each spatial row of a frame (its C tokens
// against all N keys, flattened) is compared by cosine similarity with the
// attention of its nearest anchor row; a head is repetitive when the mean over
// frames, non-anchor rows and prompts exceeds the threshold.
//
// For row r of frame f with nearest anchor a (ties to the smaller anchor):
//   sim = <P_r, P_a> / (|P_r| |P_a|),  <P_r, P_a> = sum_c sum_j P[(f,r,c)][j] P[(f,a,c)][j],
// P = softmax over all keys of scale * q . k. One pass over the keys: a slot
// keeps, relative to a reference maximum per query, the sums
//   l_r = sum e_r, l_a = sum e_a, D = sum e_r e_a, A = sum e_r^2, B = sum e_a^2
// (e = exp2(scale_log2 * s - m)); its column then contributes D / (l_r l_a),
// A / l_r^2 and B / l_a^2, which are the sums over the normalised
// probabilities. The non-anchor rows of a
// head, flattened over (frame, row), are split into groups of m whole rows;
// one workgroup per group gives each lane one (row, column) slot of the group,
// so m*C fills the waves' 32-lane tiles with few idle lanes whatever C is. All
// lanes of a workgroup score against one shared K stream, their own row's
// query and their anchor row's query at the same column, and accumulate the
// three sums per slot; the rows' totals are then added in column order.
#include "gfx950_device.h"

namespace calibatt {
namespace {

using namespace dev;

constexpr int kPrefetch = 4;
constexpr int kMaxWaves = 8;
// A lane's 32 terms of a stage may sum to this against the reference maxima
// before they move, so every term kept is <= 2^13 and the squared sums stay
// far from overflow.
constexpr float kStageSumCap = 8192.0f;
constexpr int kMaxSlots = kMaxWaves * 32;

// Nearest anchor row of r (ties to the smaller anchor).
__device__ __forceinline__ int nearest_anchor(const SimParams& p, int r) {
  int best = p.anchors[0];
  for (int i = 1; i < p.ka; ++i) {
    const int a = p.anchors[i];
    if (abs(r - a) < abs(r - best)) best = a;
  }
  return best;
}

// The i-th non-anchor row (anchors strictly ascending).
__device__ __forceinline__ int nonanchor_row(const SimParams& p, int i) {
  int r = i;
  for (int j = 0; j < p.ka; ++j) r += p.anchors[j] <= r ? 1 : 0;
  return r;
}

template <int D>
__global__ __launch_bounds__(kMaxWaves * 64) void similarity_bf16_kernel(const SimParams p) {
  constexpr int SUB = 64;
  constexpr int CPR = D / 8;
  constexpr int KT = SUB / 32;
  constexpr int DS = D / 16;
  constexpr int STAGE = SUB * CPR;
  constexpr int NCOP = STAGE / 64;       // 16-byte-per-lane copies per stage
  constexpr int RPI = 64 / CPR;          // K rows per copy

  __shared__ uint4 lds_k[2 * STAGE];
  // This pass's per-slot sums, 3 floats per slot, rows of the group one after
  // the other; one pad float after each row when 3*C is even, so a row starts
  // an odd number of words after the previous one and the rows' summing lanes
  // (one per row, reading their rows in step) fall in distinct banks.
  __shared__ float part[3 * kMaxSlots + kMaxSlots + 2];
  __shared__ float rowacc[kMaxSlots][3]; // per-row totals of the group

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  int n_tok = p.N;
  float scale_log2 = p.scale_log2;
  asm volatile("" : "+s"(n_tok), "+s"(scale_log2));

  const int nr = p.R - p.ka;                          // non-anchor rows per frame
  const int64_t rows_total = (int64_t)p.F * nr;
  const int m = p.rows_per_group;
  const int64_t groups = (rows_total + m - 1) / m;
  const int64_t item = xcd_item(blockIdx.x, gridDim.x, 32);
  const int head = p.heads[item / groups];
  const int64_t rho0 = (item % groups) * m;
  const int mrows = (int)min((int64_t)m, rows_total - rho0);
  const int slots = mrows * p.C;

  const u16* Q = static_cast<const u16*>(p.q) + (int64_t)head * p.head_stride;
  const char* Kb = reinterpret_cast<const char*>(static_cast<const u16*>(p.k) + (int64_t)head * p.head_stride);
  const int dq = lane / CPR;
  const int dpos = lane % CPR;
  const uint32_t dma_lane = (uint32_t)(dq * 2 * D + 16 * (dpos ^ (dq & (CPR - 1))));
  const uint32_t k_lane = (uint32_t)(l32 * 2 * D + 16 * (h ^ (l32 & (CPR - 1))));
  // copy ci of a stage fills K rows [ci*RPI, ci*RPI + RPI) of the stage buffer
  auto issue = [&](int stage, int ci, uint4* dst) {
    const int row0 = stage * SUB;
    const int rr = ci * RPI;
    const uint32_t off = dma_lane ^ (uint32_t)(16 * (rr & (CPR - 1)));
    if (row0 + SUB <= n_tok) {
      dma16(Kb + (int64_t)(row0 + rr) * (2 * D), off, dst + ci * 64);
    } else {
      asm volatile("");
      const int b0 = min(row0, n_tok - 1);
      const int grow = min(row0 + rr + dq, n_tok - 1);
      dma16(Kb + (int64_t)b0 * (2 * D), (uint32_t)((grow - b0) * (2 * D)) + (off & (2 * D - 1)), dst + ci * 64);
    }
  };
  // this wave's copies are ci = wave + n*W, n < my_n
  const int my_n = wave < NCOP ? (NCOP - wave + W - 1) / W : 0;

  for (int t = threadIdx.x; t < mrows; t += blockDim.x) rowacc[t][0] = rowacc[t][1] = rowacc[t][2] = 0.0f;
  const int n_stages = (n_tok + SUB - 1) / SUB;
  for (int base = 0; base < slots; base += W * 32) {
    // this lane's slot: row il of the group, column c (idle slots score q = 0; their sums are never read)
    const int slot = base + wave * 32 + l32;
    const bool ok = slot < slots;
    int tr = 0, ta = 0;
    if (ok) {
      const int il = slot / p.C, c = slot % p.C;
      const int64_t rho = rho0 + il;
      const int f = (int)(rho / nr);
      const int r = nonanchor_row(p, (int)(rho % nr));
      const int a = nearest_anchor(p, r);
      tr = (f * p.R + r) * p.C + c;
      ta = (f * p.R + a) * p.C + c;
    }
    bf16x8 qr[DS], qa[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0);
      if (ok) {
        x = ld_global16(Q + (int64_t)tr * D + 16 * s + 8 * h);
        y = ld_global16(Q + (int64_t)ta * D + 16 * s + 8 * h);
      }
      qr[s] = bitcast<bf16x8>(x);
      qa[s] = bitcast<bf16x8>(y);
    }
    for (int n = 0; n < my_n; ++n) issue(0, wave + n * W, lds_k);
    // the reference maxima are shared by a slot's two key halves (lanes l32, l32 + 32)
    float m_r = -INFINITY, m_a = -INFINITY;
    float l_r = 0.0f, l_a = 0.0f, dot = 0.0f, nr2 = 0.0f, na2 = 0.0f;
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
          // the next stage's copies go between the MFMAs, one every second step
          if (has_next && (idx & 1) && (idx >> 1) < my_n) issue(j + 1, wave + (idx >> 1) * W, nk);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (has_next) {
          for (int n = (KT * DS) / 2; n < my_n; ++n) issue(j + 1, wave + n * W, nk);
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
      // The stage's terms against the current reference maxima, summed apart
      // and then added to the totals (one fp32 chain over all of a lane's keys
      // would lose ~sqrt(N/2) ulps). The references move only when some lane's
      // 32 terms of either stream sum past kStageSumCap or are not finite (the
      // first stage, while they are -inf; masked keys then give NaN): then the
      // maxima are searched, the totals rescaled and the stage summed again.
      float s_lr, s_la, s_d, s_nr, s_na;
      auto stage_sums = [&]() {
        s_lr = s_la = s_d = s_nr = s_na = 0.0f;
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float er = __builtin_amdgcn_exp2f(__builtin_fmaf(sr[t][e], scale_log2, -m_r));
            const float ea = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[t][e], scale_log2, -m_a));
            s_lr += er;
            s_la += ea;
            s_d = __builtin_fmaf(er, ea, s_d);
            s_nr = __builtin_fmaf(er, er, s_nr);
            s_na = __builtin_fmaf(ea, ea, s_na);
          }
      };
      stage_sums();
      if (__ballot(!(s_lr <= kStageSumCap) || !(s_la <= kStageSumCap)) != 0) {
        asm volatile("");   // rare: keep it a branch
        float xr = -INFINITY, xa = -INFINITY;
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            xr = fmaxf(xr, sr[t][e]);
            xa = fmaxf(xa, sa[t][e]);
          }
        const float br = xr * scale_log2, ba = xa * scale_log2;
        const float nm_r = fmaxf(m_r, fmaxf(br, __shfl_xor(br, 32)));
        const float nm_a = fmaxf(m_a, fmaxf(ba, __shfl_xor(ba, 32)));
        const float fr = __builtin_amdgcn_exp2f(m_r - nm_r);   // 0 while m is -inf
        const float fa = __builtin_amdgcn_exp2f(m_a - nm_a);
        l_r *= fr;
        l_a *= fa;
        dot *= fr * fa;
        nr2 *= fr * fr;
        na2 *= fa * fa;
        m_r = nm_r;
        m_a = nm_a;
        stage_sums();
      }
      l_r += s_lr;
      l_a += s_la;
      dot += s_d;
      nr2 += s_nr;
      na2 += s_na;
    }
    // the two key halves of a slot sit in lanes l32 and l32 + 32 (same reference maxima)
    l_r += __shfl_xor(l_r, 32);
    l_a += __shfl_xor(l_a, 32);
    dot += __shfl_xor(dot, 32);
    nr2 += __shfl_xor(nr2, 32);
    na2 += __shfl_xor(na2, 32);
    // the column's sums over normalised probabilities
    dot = dot / (l_r * l_a);
    nr2 = nr2 / (l_r * l_r);
    na2 = na2 / (l_a * l_a);
    const int il0 = base / p.C;
    const int pad = (3 * p.C) % 2 == 0 ? 1 : 0;   // words after each row of part[]
    {
      // One store per row among this wave's slots: a store whose lanes spanned
      // two rows would put a padded lane in the bank of an unpadded one.
      const int row = slot / p.C - il0;
      const int first_slot = base + wave * 32;
      const int r_lo = first_slot / p.C - il0;
      const int r_hi = (first_slot + 31) / p.C - il0;
      for (int rr = r_lo; rr <= r_hi; ++rr) {
        if (h == 0 && row == rr) {
          const int at = 3 * (slot - base) + pad * rr;
          part[at + 0] = dot;
          part[at + 1] = nr2;
          part[at + 2] = na2;
        }
        __builtin_amdgcn_sched_barrier(0);   // (keep the rows' stores apart)
      }
    }
    __syncthreads();
    // rows touched by this pass add their slots in column order
    const int end = min(base + W * 32, slots);
    const int il1 = (end - 1) / p.C;
    for (int t = il0 + (int)threadIdx.x; t <= il1; t += blockDim.x) {
      const int s0 = max(t * p.C, base), s1 = min((t + 1) * p.C, end);
      const int row_pad = pad * (t - il0);
      float sd = 0.0f, sn = 0.0f, sa2 = 0.0f;
      for (int q = s0; q < s1; ++q) {
        const int at = 3 * (q - base) + row_pad;
        sd += part[at + 0];
        sn += part[at + 1];
        sa2 += part[at + 2];
      }
      rowacc[t][0] += sd;
      rowacc[t][1] += sn;
      rowacc[t][2] += sa2;
    }
    __syncthreads();   // part[] and the K buffers are reused by the next pass
  }
  for (int t = threadIdx.x; t < mrows; t += blockDim.x) {
    const int64_t rho = rho0 + t;
    const int f = (int)(rho / nr);
    const int r = nonanchor_row(p, (int)(rho % nr));
    p.row_sim[((int64_t)head * p.F + f) * p.R + r] = rowacc[t][0] / sqrtf(rowacc[t][1] * rowacc[t][2]);
  }
}

// Anchor rows compare with themselves: similarity 1.
__global__ void anchor_ones_kernel(const SimParams p) {
  const int head = p.heads[blockIdx.x];
  for (int i = threadIdx.x; i < p.F * p.ka; i += blockDim.x) {
    const int f = i / p.ka, j = i % p.ka;
    p.row_sim[((int64_t)head * p.F + f) * p.R + p.anchors[j]] = 1.0f;
  }
}

// fp32 inputs: one thread per column of the row pair, K tiles in LDS; the
// same one-pass sums with an exact running maximum (natural exponent).
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
    float m_r = -INFINITY, m_a = -INFINITY, l_r = 0.0f, l_a = 0.0f;
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
        const float xr = sr * p.scale, xa = sa * p.scale;
        if (xr > m_r) {
          const float g = expf(m_r - xr);
          l_r *= g;
          dot *= g;
          nr *= g * g;
          m_r = xr;
        }
        if (xa > m_a) {
          const float g = expf(m_a - xa);
          l_a *= g;
          dot *= g;
          na *= g * g;
          m_a = xa;
        }
        const float er = expf(xr - m_r), ea = expf(xa - m_a);
        l_r += er;
        l_a += ea;
        dot = __builtin_fmaf(er, ea, dot);
        nr = __builtin_fmaf(er, er, nr);
        na = __builtin_fmaf(ea, ea, na);
      }
    }
    red[threadIdx.x][0] = ok ? dot / (l_r * l_a) : 0.0f;
    red[threadIdx.x][1] = ok ? nr / (l_r * l_r) : 0.0f;
    red[threadIdx.x][2] = ok ? na / (l_a * l_a) : 0.0f;
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

// Rows per workgroup and waves for rows of C columns (bf16 path): the largest
// product of the busy fraction of the m*C slots and the fraction of a CU's
// wave slots (two waves per SIMD at this kernel's register use) the resident
// workgroups fill; ties go to more waves (a K stream shared more widely).
// Rows wider than the largest workgroup take one row per group, in passes.
static void pick_group(int C, int& m, int& W) {
  if (C > kMaxSlots) {
    m = 1;
    W = kMaxWaves;
    return;
  }
  double best = -1.0;
  for (int mm = 1; mm * C <= kMaxSlots; ++mm) {
    const int w = (mm * C + 31) / 32;
    const double score = (double)(mm * C) / (32.0 * w) * (double)((kMaxWaves / w) * w) / kMaxWaves;
    if (score > best + 1e-9 || (score > best - 1e-9 && w > W)) {
      best = score;
      m = mm;
      W = w;
    }
  }
}

hipError_t launch_similarity(const SimParams& p, int d, bool f32, hipStream_t s) {
  if (p.n_heads == 0) return hipSuccess;
  if (f32) {
    const int64_t items = (int64_t)p.n_heads * p.F * p.R;
    if (d == 128) hipLaunchKernelGGL(similarity_f32_kernel<128>, dim3((unsigned)items), dim3(64), 0, s, p);
    else if (d == 64) hipLaunchKernelGGL(similarity_f32_kernel<64>, dim3((unsigned)items), dim3(64), 0, s, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  SimParams q = p;
  int W = 0;
  pick_group(p.C, q.rows_per_group, W);
  const int64_t rows = (int64_t)p.F * (p.R - p.ka);
  const int64_t items = (int64_t)p.n_heads * ((rows + q.rows_per_group - 1) / q.rows_per_group);
  if (d == 128) hipLaunchKernelGGL(similarity_bf16_kernel<128>, dim3((unsigned)items), dim3(W * 64), 0, s, q);
  else if (d == 64) hipLaunchKernelGGL(similarity_bf16_kernel<64>, dim3((unsigned)items), dim3(W * 64), 0, s, q);
  else return hipErrorInvalidValue;
  hipLaunchKernelGGL(anchor_ones_kernel, dim3((unsigned)p.n_heads), dim3(64), 0, s, q);
  return hipGetLastError();
}

hipError_t launch_rep_flags(const float* sims, int P, int H, int F, int R, const RepFlagParams& q, uint8_t* flags,
                            float* mean, hipStream_t s) {
  hipLaunchKernelGGL(flags_kernel, dim3((unsigned)((H + 63) / 64)), dim3(64), 0, s, sims, P, H, F, R, q, flags, mean);
  return hipGetLastError();
}

}  // namespace calibatt
