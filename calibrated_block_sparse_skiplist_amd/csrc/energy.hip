// Offline calibration kernels: block energies, per-prompt block selection and
// cross-prompt keep frequency (papernotes.org notes on "Accelerating
// Text-to-Video Generation with Calibrated Sparse Attention", Key Designs 1, 2
// and 4; Eq. 5 and Eq. 8-9).
//
// Block energy (Eq. 5): for query block r and key block c of one head,
//   E[r][c] = (1 / |I_r|) * sum_{i in I_r} sum_{j in J_c} P[i][j],
// P = softmax over all N keys of scale * q_i . k_j. The full P is never
// stored: one workgroup owns one query block. Without a workspace it streams
// every key block twice: pass 1 finds each query's log-sum-exp, pass 2
// recomputes the scores, turns them into probabilities with that log-sum-exp
// and adds them up per key block. With a workspace it streams the keys once:
// each query keeps its log-sum-exp running and leaves, per key block, the
// base-2 log of its sum over that block (relative to its first reference
// maximum) in the workspace; once the query's total is known, the block sums
// are normalised and added up over the block's queries. Rows of a partial last
// query block are averaged over their actual count, so every row of E sums to
// one.
//
// Selection (Key Design 1): per row of E, sort energies descending (ties to
// the lower key block), keep the shortest prefix whose cumulative mass reaches
// tau. The cumulative mass is summed exactly in 64-bit fixed point
// (floor(E * 2^48) units; threshold ceil(tau * 2^48), computed on the host),
// so the decision does not depend on summation order. A block is kept iff the
// mass sorted before it is below the threshold; a row that never reaches tau
// keeps every block.
//
// Keep frequency (Key Design 2): selections of the calibration prompts are
// counted per block; a block is retained iff count >= rho * |D| (the integer
// bound is computed exactly on the host).
#include "gfx950_device.h"

namespace calibatt {
namespace {

using namespace dev;

constexpr int kPrefetch = 4;            // K operand reads in flight ahead of their MFMA
// One-pass kernel: a lane's 32 terms of a stage may sum to at most this
// against the reference maximum before the reference moves.
constexpr float kStageSumCap = 8192.0f;

// ---------------------------------------------------------------------------
// bf16 energies: S^T = K Q^T with v_mfma_f32_32x32x16_bf16 exactly as in the
// attention kernel (A = K from LDS, B = Q^T in registers; a lane owns one query
// column and half of the 64 keys of a stage); K moves HBM -> LDS by DMA,
// double-buffered per 64-key stage, the next stage issued between the MFMAs.
// ---------------------------------------------------------------------------
template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void energy_bf16_kernel(const EnergyParams p) {
  constexpr int NW = BLK / 32;
  constexpr int SUB = 64;
  constexpr int SPB = BLK / SUB;
  constexpr int CPR = D / 8;
  constexpr int KT = SUB / 32;
  constexpr int DS = D / 16;
  constexpr int STAGE = SUB * CPR;
  constexpr int LPW = STAGE / 64 / NW;   // copy instructions per wave and stage
  constexpr int RPI = 64 / CPR;

  __shared__ uint4 lds_k[2 * STAGE];
  extern __shared__ float lds_e[];       // [NW][nb] per-wave block sums

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int nb = p.nb;
  int n_tok = p.N;
  float scale_log2 = p.scale_log2;
  asm volatile("" : "+s"(n_tok), "+s"(scale_log2));

  const int64_t item = xcd_item(blockIdx.x, gridDim.x, 32);
  const int head = p.heads[item / nb];
  const int r = (int)(item % nb);
  const u16* Q = static_cast<const u16*>(p.q) + (int64_t)head * p.head_stride;
  const char* Kb = reinterpret_cast<const char*>(static_cast<const u16*>(p.k) + (int64_t)head * p.head_stride);

  const int qtok = r * BLK + wave * 32 + l32;
  const bool q_ok = qtok < n_tok;
  bf16x8 qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (q_ok) raw = ld_global16(Q + (int64_t)qtok * D + 16 * s + 8 * h);
    qf[s] = bitcast<bf16x8>(raw);
  }

  // Copy geometry (see the attention kernel): lane part of the byte offset,
  // XORed with the chunk bits of the instruction's first row.
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
      // rows past N read row N-1 (their scores are masked)
      const int b0 = min(row0, n_tok - 1);
      const int grow = min(row0 + rr + dq, n_tok - 1);
      dma16(Kb + (int64_t)b0 * (2 * D), (uint32_t)((grow - b0) * (2 * D)) + (off & (2 * D - 1)),
            dst + (wave * LPW + i) * 64);
    }
  };

  const int n_stages = nb * SPB;
  // Per lane: running maximum (log2 units of the scaled score) and sum over
  // this lane's keys; after the first pass, the query's log2-sum-exp.
  float m_run = -INFINITY, l_run = 0.0f, lse2 = 0.0f;
  float e_acc = 0.0f;

  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      // every wave is done with the last stage of the first pass before stage 0 is copied again
      wait_vmcnt<0>();
      barrier_no_fence();
    }
#pragma unroll
    for (int i = 0; i < LPW; ++i) issue(0, i, lds_k);
    for (int j = 0; j < n_stages; ++j) {
      const uint4* sk = lds_k + (j & 1) * STAGE;
      uint4* nk = lds_k + ((j + 1) & 1) * STAGE;
      wait_vmcnt<0>();
      barrier_no_fence();
      const bool has_next = j + 1 < n_stages;

      f32x16 sacc[KT];
      // copy i of the next stage: straight when that stage is full (nearly
      // always), else with the clamp of issue(); none after the last stage
      auto qk_product = [&](auto copy) {
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
          const bf16x8 a = ring[idx % kPrefetch];
          if (idx + kPrefetch < KT * DS) ring[idx % kPrefetch] = read_k(idx + kPrefetch);
          sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], s == 0 ? f32x16{} : sacc[t], 0, 0, 0);
          if (idx % kEvery == kEvery - 1 && idx / kEvery < LPW) copy(idx / kEvery);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = (KT * DS) / kEvery; i < LPW; ++i) copy(i);
      };
      if (has_next && (j + 2) * SUB <= n_tok) {
        const char* base = Kb + (int64_t)(j + 1) * SUB * (2 * D);
        qk_product([&](int i) {
          const int rr = (wave * LPW + i) * RPI;
          dma16(base + (int64_t)rr * (2 * D), dma_lane ^ (uint32_t)(16 * (rr & (CPR - 1))), nk + (wave * LPW + i) * 64);
        });
      } else {
        qk_product([&](int i) {
          if (has_next) issue(j + 1, i, nk);
        });
      }
      const int valid = n_tok - j * SUB;
      if (valid < SUB) {
        int lv = valid - 4 * h;
        asm volatile("" : "+v"(lv));
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
          for (int a = 0; a < 16; ++a) {
            const int key = 32 * t + 8 * (a >> 2) + (a & 3);
            if (key >= lv) sacc[t][a] = -INFINITY;
          }
      }

      if (pass == 0) {
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
          for (int a = 0; a < 16; ++a) mx = fmaxf(mx, sacc[t][a]);
        const float mb = mx * scale_log2;
        if (mb > m_run) {
          l_run *= __builtin_amdgcn_exp2f(m_run - mb);   // 0 while m_run is -inf
          m_run = mb;
        }
        const float neg_m = m_run == -INFINITY ? 0.0f : -m_run;   // no key of this lane yet: every term is 0
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
          for (int a = 0; a < 16; a += 2) {
            s0 += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][a], scale_log2, neg_m));
            s1 += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][a + 1], scale_log2, neg_m));
          }
        l_run += s0 + s1;
      } else {
        const float neg_l = -lse2;
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
          for (int a = 0; a < 16; a += 2) {
            s0 += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][a], scale_log2, neg_l));
            s1 += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][a + 1], scale_log2, neg_l));
          }
        e_acc += s0 + s1;
        if (j % SPB == SPB - 1) {
          // block c = j / SPB done: sum the wave's 64 lanes (fixed order)
          float v = e_acc;
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
          if (lane == 0) lds_e[wave * nb + j / SPB] = v;
          e_acc = 0.0f;
        }
      }
    }
    if (pass == 0) {
      // combine the two key halves of each query (lanes l and l ^ 32)
      const float m_o = __shfl_xor(m_run, 32);
      const float l_o = __shfl_xor(l_run, 32);
      const float M = fmaxf(m_run, m_o);
      const float L = l_run * __builtin_amdgcn_exp2f(m_run - M) + l_o * __builtin_amdgcn_exp2f(m_o - M);
      // queries past N get +inf, so every probability of theirs is exactly 0
      lse2 = q_ok ? M + __log2f(L) : INFINITY;
    }
  }

  __syncthreads();
  const int n_q = min(BLK, n_tok - r * BLK);
  const float inv = 1.0f / (float)n_q;
  float* out = p.energy + ((int64_t)head * nb + r) * nb;
  for (int c = threadIdx.x; c < nb; c += NW * 64) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += lds_e[w * nb + c];
    out[c] = v * inv;
  }
}

// One pass with a workspace p.work of [items][nb][BLK] floats (item = index
// of the head in p.heads * nb + query block; the launch's items from p.item0
// on, the first at p.work). The two key-half lanes of a
// query share a lazily moved reference maximum m; at the end of key block c,
// lane h = 0 stores log2(sum over the block of exp2(s - m)) + (m - m0), m0 the
// reference after the first stage. With the query's total
// lse' = (m_end - m0) + log2(l), its probability mass in block c is
// exp2(stored - lse'); one wave per key block adds those up over the block's
// queries in a fixed order.
template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void energy_bf16_onepass_kernel(const EnergyParams p) {
  constexpr int NW = BLK / 32;
  constexpr int SUB = 64;
  constexpr int SPB = BLK / SUB;
  constexpr int CPR = D / 8;
  constexpr int KT = SUB / 32;
  constexpr int DS = D / 16;
  constexpr int STAGE = SUB * CPR;
  constexpr int LPW = STAGE / 64 / NW;   // copy instructions per wave and stage
  constexpr int RPI = 64 / CPR;

  __shared__ uint4 lds_k[2 * STAGE];
  __shared__ float lds_lse[BLK];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int nb = p.nb;
  int n_tok = p.N;
  float scale_log2 = p.scale_log2;
  asm volatile("" : "+s"(n_tok), "+s"(scale_log2));

  const int64_t local = xcd_item(blockIdx.x, gridDim.x, 32);
  const int64_t item = p.item0 + local;
  const int head = p.heads[item / nb];
  const int r = (int)(item % nb);
  const u16* Q = static_cast<const u16*>(p.q) + (int64_t)head * p.head_stride;
  const char* Kb = reinterpret_cast<const char*>(static_cast<const u16*>(p.k) + (int64_t)head * p.head_stride);
  float* ws = p.work + local * (int64_t)nb * BLK;

  const int qtok = r * BLK + wave * 32 + l32;
  const bool q_ok = qtok < n_tok;
  bf16x8 qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (q_ok) raw = ld_global16(Q + (int64_t)qtok * D + 16 * s + 8 * h);
    qf[s] = bitcast<bf16x8>(raw);
  }

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

  const int n_stages = nb * SPB;
  float m_run = -INFINITY, m0 = 0.0f, l_run = 0.0f, b_run = 0.0f;
#pragma unroll
  for (int i = 0; i < LPW; ++i) issue(0, i, lds_k);
  for (int j = 0; j < n_stages; ++j) {
    const uint4* sk = lds_k + (j & 1) * STAGE;
    uint4* nk = lds_k + ((j + 1) & 1) * STAGE;
    wait_vmcnt<0>();
    barrier_no_fence();
    const bool has_next = j + 1 < n_stages;

    f32x16 sacc[KT];
    // copy i of the next stage: straight when that stage is full (nearly
    // always), else with the clamp of issue(); none after the last stage
    auto qk_product = [&](auto copy) {
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
        const bf16x8 a = ring[idx % kPrefetch];
        if (idx + kPrefetch < KT * DS) ring[idx % kPrefetch] = read_k(idx + kPrefetch);
        sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], s == 0 ? f32x16{} : sacc[t], 0, 0, 0);
        if (idx % kEvery == kEvery - 1 && idx / kEvery < LPW) copy(idx / kEvery);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = (KT * DS) / kEvery; i < LPW; ++i) copy(i);
    };
    if (has_next && (j + 2) * SUB <= n_tok) {
      const char* base = Kb + (int64_t)(j + 1) * SUB * (2 * D);
      qk_product([&](int i) {
        const int rr = (wave * LPW + i) * RPI;
        dma16(base + (int64_t)rr * (2 * D), dma_lane ^ (uint32_t)(16 * (rr & (CPR - 1))), nk + (wave * LPW + i) * 64);
      });
    } else {
      qk_product([&](int i) {
        if (has_next) issue(j + 1, i, nk);
      });
    }
    const int valid = n_tok - j * SUB;
    if (valid < SUB) {
      int lv = valid - 4 * h;
      asm volatile("" : "+v"(lv));
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const int key = 32 * t + 8 * (a >> 2) + (a & 3);
          if (key >= lv) sacc[t][a] = -INFINITY;
        }
    }

    // The stage's terms exp2(s - m) against the current reference m. The
    // reference moves only when some lane's 32 terms sum past 2^13 or are not
    // finite (the first stage, while m is still -inf; masked keys then give
    // NaN): then m becomes the maximum so far and the terms are redone. So
    // the row maximum is only searched on those rare stages, and every term
    // that is kept is at most 2^13.
    auto stage_terms = [&](float neg_m) {
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int a = 0; a < 16; a += 2) {
          s0 += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][a], scale_log2, neg_m));
          s1 += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][a + 1], scale_log2, neg_m));
        }
      return s0 + s1;
    };
    float st = stage_terms(-m_run);
    if (__ballot(!(st <= kStageSumCap)) != 0) {
      asm volatile("");   // rare: keep it a branch
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int a = 0; a < 16; ++a) mx = fmaxf(mx, sacc[t][a]);
      const float mb = mx * scale_log2;
      // (key 0 is in every query's first stage, so m is finite from stage 0 on)
      const float m_new = fmaxf(m_run, fmaxf(mb, __shfl_xor(mb, 32)));
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m_run is -inf
      l_run *= alpha;
      b_run *= alpha;
      m_run = m_new;
      st = stage_terms(-m_run);
    }
    if (j == 0) m0 = m_run;
    b_run += st;
    if (j % SPB == SPB - 1) {
      // key block c = j / SPB done: both key halves of the query, same reference
      const float bsum = b_run + __shfl_xor(b_run, 32);
      if (h == 0) ws[(int64_t)(j / SPB) * BLK + wave * 32 + l32] = __log2f(bsum) + (m_run - m0);
      l_run += b_run;
      b_run = 0.0f;
    }
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  // queries past N get +inf, so every probability of theirs is exactly 0
  if (h == 0) lds_lse[wave * 32 + l32] = q_ok ? (m_run - m0) + __log2f(l_tot) : INFINITY;
  __syncthreads();   // (also orders every wave's workspace stores before the reads below)

  const int n_q = min(BLK, n_tok - r * BLK);
  const float inv = 1.0f / (float)n_q;
  float* out = p.energy + ((int64_t)head * nb + r) * nb;
  for (int c = wave; c < nb; c += NW) {
    float v = 0.0f;
#pragma unroll
    for (int q = lane; q < BLK; q += 64)
      v += __builtin_amdgcn_exp2f(ws[(int64_t)c * BLK + q] - lds_lse[q]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) out[c] = v * inv;
  }
}

// fp32 energies: one thread per query, K tiles in LDS read as broadcasts,
// fp32 FMA and expf; the same two passes.
template <int D, int BLK>
__global__ __launch_bounds__(BLK) void energy_f32_kernel(const EnergyParams p) {
  extern __shared__ float smem[];
  float* ks = smem;                      // [BLK][D]
  float* red = smem + BLK * D;           // [BLK] block reduction
  const int nb = p.nb;
  const int head = p.heads[blockIdx.x / nb];
  const int r = (int)(blockIdx.x % nb);
  const float* Q = static_cast<const float*>(p.q) + (int64_t)head * p.head_stride;
  const float* K = static_cast<const float*>(p.k) + (int64_t)head * p.head_stride;
  const int qtok = r * BLK + threadIdx.x;
  const bool q_ok = qtok < p.N;
  float q[D];
#pragma unroll
  for (int i = 0; i < D; ++i) q[i] = q_ok ? Q[(int64_t)qtok * D + i] : 0.0f;
  float m = -INFINITY, l = 0.0f, lse = 0.0f;
  for (int pass = 0; pass < 2; ++pass) {
    for (int c = 0; c < nb; ++c) {
      const int nk = min(BLK, p.N - c * BLK);
      __syncthreads();
      for (int e = threadIdx.x * 4; e < nk * D; e += BLK * 4)
        *reinterpret_cast<float4*>(ks + e) = *reinterpret_cast<const float4*>(K + (int64_t)c * BLK * D + e);
      __syncthreads();
      float acc = 0.0f;
      for (int j = 0; j < nk; ++j) {
        float dot = 0.0f;
#pragma unroll
        for (int i = 0; i < D; ++i) dot = __builtin_fmaf(q[i], ks[j * D + i], dot);
        const float s = dot * p.scale;
        if (pass == 0) {
          if (s > m) {
            l *= expf(m - s);
            m = s;
          }
          l += expf(s - m);
        } else {
          acc += expf(s - lse);
        }
      }
      if (pass == 1) {
        red[threadIdx.x] = q_ok ? acc : 0.0f;
        __syncthreads();
        if (threadIdx.x == 0) {
          float v = 0.0f;
          for (int t = 0; t < BLK; ++t) v += red[t];
          p.energy[((int64_t)head * nb + r) * nb + c] = v / (float)min(BLK, p.N - r * BLK);
        }
      }
    }
    if (pass == 0) lse = m + logf(l);
  }
}

// ---------------------------------------------------------------------------
// Selection: one workgroup per row of E.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 256;

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ energy, int nb, int p2,
                                                             unsigned long long need, uint8_t* __restrict__ mask,
                                                             int32_t* __restrict__ counts) {
  // key = (fp32 bits of E) << 16 | (0xffff - c): descending key order is
  // descending energy, ties to the lower block (energies are >= 0, so their
  // bit patterns order like the values); padding keys are 0 and sort last.
  __shared__ unsigned long long key[CALIBATT_MAX_NB];
  __shared__ unsigned long long part[kSelThreads];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const float* e = energy + row * nb;
  for (int i = tid; i < p2; i += kSelThreads) {
    unsigned long long k = 0ull;
    if (i < nb) k = ((unsigned long long)__float_as_uint(e[i]) << 16) | (unsigned long long)(0xffff - i);
    key[i] = k;
  }
  __syncthreads();
  // bitonic sort, descending
  for (int k = 2; k <= p2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < p2; i += kSelThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long a = key[i], b = key[ixj];
          const bool first_half = (i & k) == 0;
          if (first_half ? (a < b) : (a > b)) {
            key[i] = b;
            key[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  // exclusive scan of the fixed-point units over sorted positions: each
  // thread owns a contiguous span, then a scan of the span totals
  const int per = (p2 + kSelThreads - 1) / kSelThreads;
  const int lo = tid * per, hi = min(p2, lo + per);
  auto units = [&](unsigned long long k) -> unsigned long long {
    const double v = (double)__uint_as_float((unsigned)(k >> 16));
    return (unsigned long long)floor(v * 281474976710656.0);   // E * 2^48, exact for E >= 2^-25
  };
  unsigned long long tot = 0ull;
  for (int i = lo; i < hi; ++i) tot += units(key[i]);
  part[tid] = tot;
  __syncthreads();
  for (int off = 1; off < kSelThreads; off <<= 1) {
    const unsigned long long add = tid >= off ? part[tid - off] : 0ull;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  unsigned long long before = tid > 0 ? part[tid - 1] : 0ull;
  for (int i = lo; i < hi; ++i) {
    const unsigned long long k = key[i];
    if (i < nb) {   // every real key precedes the padding
      const int c = 0xffff - (int)(k & 0xffffull);
      const uint8_t keep = before < need ? 1 : 0;
      if (mask) mask[row * nb + c] = keep;
      if (counts) counts[row * nb + c] += keep;
    }
    before += units(k);
  }
}

__global__ void keep_kernel(const int32_t* __restrict__ counts, int64_t n, int32_t k_min, uint8_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = counts[i] >= k_min ? 1 : 0;
}

template <int D, int BLK>
hipError_t launch_energy_typed(const EnergyParams& p, hipStream_t s) {
  const int64_t items = (int64_t)p.n_heads * p.nb;
  if (items == 0) return hipSuccess;
  if (p.work && !p.dtype_f32) {
    auto kern = energy_bf16_onepass_kernel<D, BLK>;
    hipLaunchKernelGGL(kern, dim3((unsigned)items), dim3(BLK * 2), 0, s, p);
  } else if (p.dtype_f32) {
    const size_t smem = (size_t)(BLK * D + BLK) * sizeof(float);
    auto kern = energy_f32_kernel<D, BLK>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)items), dim3(BLK), smem, s, p);
  } else {
    const size_t smem = (size_t)(BLK / 32) * p.nb * sizeof(float);
    auto kern = energy_bf16_kernel<D, BLK>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)items), dim3(BLK * 2), smem, s, p);
  }
  return hipGetLastError();
}

// The one-pass bf16 kernel over items [p.item0, p.item0 + n_items) (a launch
// whose workspace holds fewer items than the heads have).
template <int D, int BLK>
hipError_t launch_energy_onepass_typed(const EnergyParams& p, int64_t n_items, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  hipLaunchKernelGGL((energy_bf16_onepass_kernel<D, BLK>), dim3((unsigned)n_items), dim3(BLK * 2), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_energy_onepass_items(const EnergyParams& p, int d, int blk, int64_t n_items, hipStream_t s) {
  if (!p.work || p.dtype_f32 || n_items < 0 || p.item0 < 0 || p.item0 + n_items > (int64_t)p.n_heads * p.nb)
    return hipErrorInvalidValue;
  if (d == 128 && blk == 128) return launch_energy_onepass_typed<128, 128>(p, n_items, s);
  if (d == 64 && blk == 128) return launch_energy_onepass_typed<64, 128>(p, n_items, s);
  if (d == 128 && blk == 64) return launch_energy_onepass_typed<128, 64>(p, n_items, s);
  if (d == 64 && blk == 64) return launch_energy_onepass_typed<64, 64>(p, n_items, s);
  return hipErrorInvalidValue;
}

hipError_t launch_energy(const EnergyParams& p, int d, int blk, hipStream_t s) {
  if (p.item0 != 0) return hipErrorInvalidValue;   // whole heads per launch
  if (d == 128 && blk == 128) return launch_energy_typed<128, 128>(p, s);
  if (d == 64 && blk == 128) return launch_energy_typed<64, 128>(p, s);
  if (d == 128 && blk == 64) return launch_energy_typed<128, 64>(p, s);
  if (d == 64 && blk == 64) return launch_energy_typed<64, 64>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_select(const float* energy, int64_t rows, int nb, unsigned long long need, uint8_t* mask,
                         int32_t* counts, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  int p2 = 1;
  while (p2 < nb) p2 <<= 1;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)rows), dim3(kSelThreads), 0, s, energy, nb, p2, need, mask,
                     counts);
  return hipGetLastError();
}

hipError_t launch_keep(const int32_t* counts, int64_t n, int32_t k_min, uint8_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
  hipLaunchKernelGGL(keep_kernel, dim3((unsigned)blocks), dim3(256), 0, s, counts, n, k_min, out);
  return hipGetLastError();
}

}  // namespace calibatt
