// Skip-list compiler kernels: binary block masks -> CSR lists of key blocks.
//
// Each calibrated mask of a (timestep, layer, head) record becomes, for every
// query block, the read-only list of key blocks to compute, resident on the
// GPU before generation (papernotes.org notes on "Accelerating Text-to-Video
// Generation with Calibrated Sparse Attention", Key Design 4). Rows are the
// flattened (record, query block) pairs; lists are ascending.
//
// Passes (all integer work, so results are exact):
//   1. count: one wave per mask row counts nonzero bytes with ballots into
//      row_ptr[1 + row]; segment_scan then scans each segment of kSeg rows in place.
//   2. scan_totals: one workgroup turns the segment-end values into a global
//      inclusive scan.
//   3. add_offsets: every segment but the first adds the previous segment's
//      global end to its other entries.
//   4. fill: one wave per row compacts the column indices of nonzero bytes.
//   5. order: one workgroup per record ranks query blocks by (-count, index).
// The interval form (one [lo, hi) pair per maximal run of kept blocks: the
// contiguous key-block intervals of the same Key Design 4) reuses the scan:
// run_count counts run openings, run_fill writes each run's two ends, and
// run_order sums a row's run lengths for the same ranking.
// Mask bytes are read once in pass 1 and once in pass 4; every pass reads its
// rows with lanes on consecutive bytes so the loads coalesce.
#include "internal.h"

namespace calibatt {
namespace {

constexpr int kSeg = 1024;        // rows per scan segment
constexpr int kThreads = 256;     // threads per workgroup

__device__ inline int row_count(const uint8_t* row, int nb, int lane) {
  int cnt = 0;
  for (int base = 0; base < nb; base += 64) {
    int c = base + lane;
    bool nz = c < nb && row[c] != 0;
    cnt += __popcll(__ballot(nz));
  }
  return cnt;
}

// Inclusive scan of n <= kSeg int64 values in LDS by kThreads threads.
__device__ void block_inclusive_scan(int64_t* vals, int n, int64_t* partial) {
  const int tid = threadIdx.x;
  constexpr int per = kSeg / kThreads;
  int64_t local[per];
  int64_t run = 0;
  for (int j = 0; j < per; ++j) {
    int i = tid * per + j;
    run += (i < n) ? vals[i] : 0;
    local[j] = run;
  }
  partial[tid] = run;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    int64_t add = (tid >= off) ? partial[tid - off] : 0;
    __syncthreads();
    partial[tid] += add;
    __syncthreads();
  }
  int64_t prefix = (tid > 0) ? partial[tid - 1] : 0;
  for (int j = 0; j < per; ++j) {
    int i = tid * per + j;
    if (i < n) vals[i] = local[j] + prefix;
  }
  __syncthreads();
}

// One wave per mask row: row_ptr[1 + row] = number of nonzero bytes.
__global__ __launch_bounds__(kThreads) void count_kernel(const uint8_t* __restrict__ masks, int64_t rows, int nb,
                                                         int64_t* __restrict__ row_ptr) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int cnt = row_count(masks + row * nb, nb, lane);
  if (lane == 0) row_ptr[1 + row] = cnt;
  if (row == 0 && lane == 0) row_ptr[0] = 0;
}

// In-place inclusive scan of each segment of kSeg counts.
__global__ __launch_bounds__(kThreads) void segment_scan_kernel(int64_t rows, int64_t* __restrict__ row_ptr) {
  __shared__ int64_t vals[kSeg];
  __shared__ int64_t partial[kThreads];
  const int64_t row0 = (int64_t)blockIdx.x * kSeg;
  const int n = (int)min<int64_t>(kSeg, rows - row0);
  for (int i = threadIdx.x; i < n; i += kThreads) vals[i] = row_ptr[1 + row0 + i];
  __syncthreads();
  block_inclusive_scan(vals, n, partial);
  for (int i = threadIdx.x; i < n; i += kThreads) row_ptr[1 + row0 + i] = vals[i];
}

__global__ __launch_bounds__(kThreads) void scan_totals_kernel(int64_t rows, int64_t* __restrict__ row_ptr) {
  __shared__ int64_t vals[kSeg];
  __shared__ int64_t partial[kThreads];
  const int64_t nseg = (rows + kSeg - 1) / kSeg;
  int64_t carry = 0;
  for (int64_t s0 = 0; s0 < nseg; s0 += kSeg) {
    const int n = (int)min<int64_t>(kSeg, nseg - s0);
    for (int i = threadIdx.x; i < n; i += kThreads) {
      int64_t end = min<int64_t>((s0 + i + 1) * kSeg, rows);   // last row of segment, exclusive
      vals[i] = row_ptr[end];
    }
    __syncthreads();
    block_inclusive_scan(vals, n, partial);
    for (int i = threadIdx.x; i < n; i += kThreads) {
      int64_t end = min<int64_t>((s0 + i + 1) * kSeg, rows);
      row_ptr[end] = vals[i] + carry;
    }
    carry += vals[n - 1];
    __syncthreads();
  }
}

__global__ __launch_bounds__(kThreads) void add_offsets_kernel(int64_t rows, int64_t* __restrict__ row_ptr) {
  const int64_t seg = blockIdx.x + 1;             // segment 0 needs no offset
  const int64_t row0 = seg * kSeg;
  const int n = (int)min<int64_t>(kSeg, rows - row0);
  const int64_t offset = row_ptr[row0];           // global end of the previous segment
  for (int i = threadIdx.x; i < n - 1; i += kThreads) row_ptr[1 + row0 + i] += offset;
}

__global__ __launch_bounds__(kThreads) void fill_kernel(const uint8_t* __restrict__ masks, int64_t rows,
                                                        int nb, const int64_t* __restrict__ row_ptr,
                                                        int32_t* __restrict__ col_idx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint8_t* m = masks + row * nb;
  int64_t out = row_ptr[row];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < nb; base += 64) {
    int c = base + lane;
    bool nz = c < nb && m[c] != 0;
    uint64_t bal = __ballot(nz);
    if (nz) col_idx[out + __popcll(bal & below)] = c;
    out += __popcll(bal);
  }
}

__global__ __launch_bounds__(kThreads) void order_kernel(const int64_t* __restrict__ row_ptr, int nb,
                                                         int32_t* __restrict__ order) {
  extern __shared__ int32_t cnt[];
  const int64_t row0 = (int64_t)blockIdx.x * nb;
  for (int r = threadIdx.x; r < nb; r += kThreads)
    cnt[r] = (int32_t)(row_ptr[row0 + r + 1] - row_ptr[row0 + r]);
  __syncthreads();
  for (int r = threadIdx.x; r < nb; r += kThreads) {
    const int c = cnt[r];
    int rank = 0;
    for (int x = 0; x < nb; ++x) {
      const int cx = cnt[x];
      rank += (cx > c) || (cx == c && x < r);
    }
    order[row0 + rank] = r;
  }
}

// ---- interval form: one [lo, hi) pair per maximal run of kept key blocks ----
//
// Block c opens a run when it is kept and block c-1 is not (or c = 0); it
// closes a run when it is kept and block c+1 is not (or c = nb-1). The k-th
// opening and the k-th closing of a row belong to the same run.

// Kept bit of block c of a row, false outside [0, nb).
__device__ inline bool kept(const uint8_t* row, int nb, int c) { return c >= 0 && c < nb && row[c] != 0; }

// One wave per mask row: iv_ptr[1 + row] = number of runs.
__global__ __launch_bounds__(kThreads) void run_count_kernel(const uint8_t* __restrict__ masks, int64_t rows,
                                                             int nb, int64_t* __restrict__ iv_ptr) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint8_t* m = masks + row * nb;
  int cnt = 0;
  for (int base = 0; base < nb; base += 64) {
    const int c = base + lane;
    cnt += __popcll(__ballot(kept(m, nb, c) && !kept(m, nb, c - 1)));
  }
  if (lane == 0) iv_ptr[1 + row] = cnt;
  if (row == 0 && lane == 0) iv_ptr[0] = 0;
}

// One wave per mask row: writes lo into the low and hi into the high 16 bits
// of each packed run (little-endian halves of the uint32 entry).
__global__ __launch_bounds__(kThreads) void run_fill_kernel(const uint8_t* __restrict__ masks, int64_t rows,
                                                            int nb, const int64_t* __restrict__ iv_ptr,
                                                            uint16_t* __restrict__ iv16) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint8_t* m = masks + row * nb;
  int64_t n_open = iv_ptr[row], n_close = iv_ptr[row];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < nb; base += 64) {
    const int c = base + lane;
    const bool here = kept(m, nb, c);
    const bool opens = here && !kept(m, nb, c - 1);
    const bool closes = here && !kept(m, nb, c + 1);
    const uint64_t bo = __ballot(opens), bc = __ballot(closes);
    if (opens) iv16[2 * (n_open + __popcll(bo & below))] = (uint16_t)c;
    if (closes) iv16[2 * (n_close + __popcll(bc & below)) + 1] = (uint16_t)(c + 1);
    n_open += __popcll(bo);
    n_close += __popcll(bc);
  }
}

// Same ranking as order_kernel, with each row's kept count summed over its runs.
__global__ __launch_bounds__(kThreads) void run_order_kernel(const int64_t* __restrict__ iv_ptr,
                                                             const uint32_t* __restrict__ iv, int nb,
                                                             int32_t* __restrict__ order) {
  extern __shared__ int32_t cnt[];
  const int64_t row0 = (int64_t)blockIdx.x * nb;
  for (int r = threadIdx.x; r < nb; r += kThreads) {
    int c = 0;
    for (int64_t i = iv_ptr[row0 + r]; i < iv_ptr[row0 + r + 1]; ++i) c += (int)(iv[i] >> 16) - (int)(iv[i] & 0xffffu);
    cnt[r] = c;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < nb; r += kThreads) {
    const int c = cnt[r];
    int rank = 0;
    for (int x = 0; x < nb; ++x) {
      const int cx = cnt[x];
      rank += (cx > c) || (cx == c && x < r);
    }
    order[row0 + rank] = r;
  }
}

// Segmented in-place scan of row_ptr[1 .. rows] (counts -> running sums).
hipError_t scan_counts(int64_t rows, int64_t* row_ptr, hipStream_t s) {
  const int64_t nseg = (rows + kSeg - 1) / kSeg;
  hipLaunchKernelGGL(segment_scan_kernel, dim3((unsigned)nseg), dim3(kThreads), 0, s, rows, row_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nseg > 1) {
    hipLaunchKernelGGL(scan_totals_kernel, dim3(1), dim3(kThreads), 0, s, rows, row_ptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(add_offsets_kernel, dim3((unsigned)(nseg - 1)), dim3(kThreads), 0, s, rows, row_ptr);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_compile_count_scan(const uint8_t* masks, int64_t rows, int nb, int64_t* row_ptr,
                                     hipStream_t s) {
  const int64_t grid = (rows + kThreads / 64 - 1) / (kThreads / 64);
  hipLaunchKernelGGL(count_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, masks, rows, nb, row_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return scan_counts(rows, row_ptr, s);
}

hipError_t launch_compile_fill(const uint8_t* masks, int64_t rows, int nb, const int64_t* row_ptr,
                               int32_t* col_idx, hipStream_t s) {
  const int64_t grid = (rows + kThreads / 64 - 1) / (kThreads / 64);
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, masks, rows, nb, row_ptr, col_idx);
  return hipGetLastError();
}

hipError_t launch_compile_order(const int64_t* row_ptr, int64_t records, int nb, int32_t* order,
                                hipStream_t s) {
  hipLaunchKernelGGL(order_kernel, dim3((unsigned)records), dim3(kThreads), (size_t)nb * sizeof(int32_t), s,
                     row_ptr, nb, order);
  return hipGetLastError();
}

hipError_t launch_compile_runs_count_scan(const uint8_t* masks, int64_t rows, int nb, int64_t* iv_ptr,
                                          hipStream_t s) {
  const int64_t grid = (rows + kThreads / 64 - 1) / (kThreads / 64);
  hipLaunchKernelGGL(run_count_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, masks, rows, nb, iv_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return scan_counts(rows, iv_ptr, s);
}

hipError_t launch_compile_runs_fill(const uint8_t* masks, int64_t rows, int nb, const int64_t* iv_ptr,
                                    uint32_t* iv, hipStream_t s) {
  const int64_t grid = (rows + kThreads / 64 - 1) / (kThreads / 64);
  hipLaunchKernelGGL(run_fill_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, masks, rows, nb, iv_ptr,
                     reinterpret_cast<uint16_t*>(iv));
  return hipGetLastError();
}

hipError_t launch_compile_runs_order(const int64_t* iv_ptr, const uint32_t* iv, int64_t records, int nb,
                                     int32_t* order, hipStream_t s) {
  hipLaunchKernelGGL(run_order_kernel, dim3((unsigned)records), dim3(kThreads), (size_t)nb * sizeof(int32_t), s,
                     iv_ptr, iv, nb, order);
  return hipGetLastError();
}

}  // namespace calibatt
