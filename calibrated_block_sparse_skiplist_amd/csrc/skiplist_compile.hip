// Skip-list compiler kernels: binary block masks -> CSR lists of key blocks.
//
// Each calibrated mask of a (timestep, layer, head) record becomes, for every
// query block, the read-only list of key blocks to compute, resident on the
// GPU before generation (papernotes.org notes on "Accelerating Text-to-Video
// Generation with Calibrated Sparse Attention", Key Design 4). Rows are the
// flattened (record, query block) pairs; lists are ascending.
//
// Passes (all integer work, so results are exact):
//   1. count: one wave per mask row counts its nonzero bytes into
//      row_ptr[1 + row]; segment_scan then scans each segment of kSeg rows in place.
//   2. scan_totals: one workgroup turns the segment-end values into a global
//      inclusive scan.
//   3. add_offsets: every segment but the first adds the previous segment's
//      global end to its other entries.
//   4. fill: one wave per row compacts the column indices of nonzero bytes.
//   5. order: query blocks of each record ranked by (-count, index), one
//      workgroup per group of 64 rows of a record.
// The interval form (one [lo, hi) pair per maximal run of kept blocks: the
// contiguous key-block intervals of the same Key Design 4) reuses the scan:
// run_count counts run openings, run_fill writes each run's two ends (and,
// for the ranking, each row's kept count into the order array), and
// run_order ranks those counts in place.
// Mask bytes are read once in pass 1 and once in pass 4. A wave reads a row
// as 16-byte aligned chunks, one per lane (1 KB per load instruction), and
// turns each chunk into 16 "kept" bits with a few integer operations; waves
// stride over the rows. Outputs go through a small LDS buffer per wave so the
// stores are contiguous.
#include "internal.h"

namespace calibatt {
namespace {

constexpr int kSeg = 1024;        // rows per scan segment
constexpr int kThreads = 256;     // threads per workgroup

constexpr int kWaves = kThreads / 64;   // waves per workgroup
constexpr int kWin = 64 * 16;           // mask bytes one wave load covers

// Bits 0..3: which bytes of x are nonzero (bit 7 of each byte of
// ((x & 0x7f..) + 0x7f..) | x is set exactly for the nonzero bytes).
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t x) {
  const uint32_t y = (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) >> 7 & 0x01010101u;
  return (y | (y >> 7) | (y >> 14) | (y >> 21)) & 0xFu;
}

// Row r of the masks is the byte span [s, e) = [r*nb, r*nb + nb). cs0 is the
// offset of the first 16-byte aligned chunk (in memory) that meets it; mis =
// address of the masks modulo 16.
struct RowSpan {
  int64_t s, e, cs0;
};
__device__ __forceinline__ RowSpan row_span(int64_t row, int nb, int mis) {
  const int64_t s = row * nb;
  return {s, s + nb, ((s + mis) & ~(int64_t)15) - mis};
}

// Kept bits of the chunk at byte offset cs (16-byte aligned in memory): bit j
// is set when byte cs + j lies in [s, e) and is nonzero. A chunk that would
// reach outside the masks [0, total) reads only its bytes inside the row.
__device__ __forceinline__ uint32_t chunk_bits(const uint8_t* masks, int64_t total, int64_t s, int64_t e,
                                               int64_t cs) {
  const int64_t lo = s > cs ? s - cs : 0;
  const int64_t hi = e - cs < 16 ? e - cs : 16;
  if (hi <= lo) return 0u;
  uint32_t bits = 0u;
  if (cs >= 0 && cs + 16 <= total) {
    const uint4 x = *reinterpret_cast<const uint4*>(masks + cs);
    bits = nonzero_bytes(x.x) | (nonzero_bytes(x.y) << 4) | (nonzero_bytes(x.z) << 8) | (nonzero_bytes(x.w) << 12);
  } else {
    for (int64_t j = lo; j < hi; ++j) bits |= (masks[cs + j] != 0 ? 1u : 0u) << j;
  }
  return bits & (0xFFFFu >> (16 - (int)hi)) & (0xFFFFu << (int)lo);
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  return v;
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

// row_ptr[1 + row] = number of nonzero bytes of the row; waves stride over
// rows two at a time (both rows' loads in flight together).
__global__ __launch_bounds__(kThreads) void count_kernel(const uint8_t* __restrict__ masks, int64_t rows, int nb,
                                                         int64_t* __restrict__ row_ptr) {
  const int lane = threadIdx.x & 63;
  const int mis = (int)((uintptr_t)masks & 15);
  const int64_t total = rows * nb;
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  for (int64_t ra = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); ra < rows; ra += 2 * stride) {
    const int64_t rb = ra + stride;
    const RowSpan a = row_span(ra, nb, mis);
    const RowSpan b = row_span(rb < rows ? rb : ra, nb, mis);
    int ca = 0, cb = 0;
    // (the two rows may need different window counts: their alignment slack differs)
    for (int64_t w = 0; a.cs0 + w < a.e || b.cs0 + w < b.e; w += kWin) {
      const uint32_t ba = chunk_bits(masks, total, a.s, a.e, a.cs0 + w + 16 * lane);
      const uint32_t bb = chunk_bits(masks, total, b.s, b.e, b.cs0 + w + 16 * lane);
      ca += __popc(ba);
      cb += __popc(bb);
    }
    ca = wave_sum(ca);
    cb = wave_sum(cb);
    if (lane == 0) {
      row_ptr[1 + ra] = ca;
      if (rb < rows) row_ptr[1 + rb] = cb;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) row_ptr[0] = 0;
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

// col_idx[row_ptr[row] ..] = the row's nonzero byte positions, ascending.
// Per 1 KB window a wave places its indices in LDS (each lane after the
// lanes before it) and then stores them contiguously.
__global__ __launch_bounds__(kThreads) void fill_kernel(const uint8_t* __restrict__ masks, int64_t rows,
                                                        int nb, const int64_t* __restrict__ row_ptr,
                                                        int32_t* __restrict__ col_idx) {
  __shared__ int32_t stage[kWaves][kWin];
  const int lane = threadIdx.x & 63;
  int32_t* const buf = stage[threadIdx.x >> 6];
  const int mis = (int)((uintptr_t)masks & 15);
  const int64_t total = rows * nb;
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  for (int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); row < rows; row += stride) {
    const RowSpan r = row_span(row, nb, mis);
    int64_t out = row_ptr[row];
    for (int64_t w = r.cs0; w < r.e; w += kWin) {
      const int64_t cs = w + 16 * lane;
      const uint32_t bits = chunk_bits(masks, total, r.s, r.e, cs);
      const int n = __popc(bits);
      const int incl = wave_inclusive_scan(n, lane);
      const int n_win = __shfl(incl, 63);
      const int c0 = (int)(cs - r.s);        // column of bit 0 (bits before the row are clear)
      int pos = incl - n;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if ((bits >> j) & 1u) buf[pos++] = c0 + j;
      // (one wave: its LDS writes above complete before these reads)
      for (int i = lane; i < n_win; i += 64) col_idx[out + i] = buf[i];
      out += n_win;
    }
  }
}

// ---- heaviest-first order of the query blocks of each record ----
//
// Rows are ranked by (count descending, row ascending): with the key
// key(x) = count(x) * 4096 + (4095 - x), distinct per row since x < 4096,
// rank(r) = #{x : key(x) > key(r)} and order[rank] = r. A workgroup holds
// all keys of one record in LDS, padded to a multiple of four with -1 (below
// every key), and ranks groups of 64 rows: lane l of wave w ranks row
// 64*group + l against the w-th quarter of the keys, read four at a time with
// broadcast reads, and the quarters' partial ranks are added in LDS. With few
// records (one layer's) each workgroup takes one group, so the ranking spreads
// over the chip; with many, one workgroup takes all groups of a record.
__device__ __forceinline__ int order_padded(int nb) { return (nb + 3) & ~3; }

__device__ __forceinline__ int32_t order_key(int count, int x) { return count * 4096 + (4095 - x); }

template <int W>   // waves of the workgroup; wave w scans the w-th W-th of the keys
__device__ __forceinline__ void rank_groups(const int32_t* key, int nb, int64_t row0, int g0, int g1,
                                            int32_t* __restrict__ order) {
  __shared__ int32_t part[64 * W];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int4* k4 = reinterpret_cast<const int4*>(key);
  const int n4 = order_padded(nb) / 4;
  const int per = (n4 + W - 1) / W;
  const int i0 = wave * per;
  const int i1 = min(n4, i0 + per);
  for (int g = g0; g < g1; ++g) {
    const int r = 64 * g + lane;
    const int kr = r < nb ? key[r] : 0;   // (lanes past the record rank nothing)
    int rank = 0;
#pragma unroll 4
    for (int i = i0; i < i1; ++i) {
      const int4 v = k4[i];
      rank += (v.x > kr) + (v.y > kr) + (v.z > kr) + (v.w > kr);
    }
    part[threadIdx.x] = rank;
    __syncthreads();
    if (wave == 0 && r < nb) {
      int total = 0;
#pragma unroll
      for (int w = 0; w < W; ++w) total += part[64 * w + lane];
      order[row0 + total] = r;
    }
    __syncthreads();   // (part is reused by the next group)
  }
}

// Workgroup b: record b / per_rec, groups [(b % per_rec) * gpw, ... + gpw).
struct OrderSlice {
  int64_t row0;
  int g0, g1;
};
__device__ __forceinline__ OrderSlice order_slice(int nb, int gpw) {
  const int groups = (nb + 63) / 64;
  const int per_rec = (groups + gpw - 1) / gpw;
  const int64_t rec = blockIdx.x / per_rec;
  const int j = (int)(blockIdx.x - rec * per_rec);
  return {rec * nb, j * gpw, min(groups, (j + 1) * gpw)};
}

__global__ __launch_bounds__(kThreads) void order_kernel(const int64_t* __restrict__ row_ptr, int nb, int gpw,
                                                         int32_t* __restrict__ order) {
  extern __shared__ int4 order_lds[];
  int32_t* key = reinterpret_cast<int32_t*>(order_lds);
  const OrderSlice sl = order_slice(nb, gpw);
  for (int r = threadIdx.x; r < order_padded(nb); r += kThreads)
    key[r] = r < nb ? order_key((int)(row_ptr[sl.row0 + r + 1] - row_ptr[sl.row0 + r]), r) : -1;
  __syncthreads();
  rank_groups<kWaves>(key, nb, sl.row0, sl.g0, sl.g1, order);
}

// ---- interval form: one [lo, hi) pair per maximal run of kept key blocks ----
//
// Block c opens a run when it is kept and block c-1 is not (or c = 0); it
// closes a run when it is kept and block c+1 is not (or c = nb-1). The k-th
// opening and the k-th closing of a row belong to the same run.

// iv_ptr[1 + row] = number of runs of the row (kept bytes whose left
// neighbour is not kept; the last byte of the previous window is carried).
__global__ __launch_bounds__(kThreads) void run_count_kernel(const uint8_t* __restrict__ masks, int64_t rows,
                                                             int nb, int64_t* __restrict__ iv_ptr) {
  const int lane = threadIdx.x & 63;
  const int mis = (int)((uintptr_t)masks & 15);
  const int64_t total = rows * nb;
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  for (int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); row < rows; row += stride) {
    const RowSpan r = row_span(row, nb, mis);
    uint32_t carry = 0u;
    int cnt = 0;
    for (int64_t w = r.cs0; w < r.e; w += kWin) {
      const uint32_t bits = chunk_bits(masks, total, r.s, r.e, w + 16 * lane);
      uint32_t prev = (__shfl_up(bits, 1) >> 15) & 1u;   // last byte of the lane before
      if (lane == 0) prev = carry;
      cnt += __popc(bits & ~((bits << 1) | prev));
      carry = (__shfl(bits, 63) >> 15) & 1u;
    }
    cnt = wave_sum(cnt);
    if (lane == 0) iv_ptr[1 + row] = cnt;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) iv_ptr[0] = 0;
}

// The row's runs, lo in the low and hi in the high 16 bits of each entry: the
// k-th opening (kept byte, left neighbour not kept) gives lo of run k, the
// k-th closing (kept byte, right neighbour not kept) gives hi = position + 1.
// A run may span windows, so the row's runs are assembled in LDS (runs_cap =
// ceil(nb/2) entries per wave, dynamic) and stored contiguously at the end.
// kept_out (nullable) receives each row's kept-block count for run_order.
__global__ __launch_bounds__(kThreads) void run_fill_kernel(const uint8_t* __restrict__ masks, int64_t rows,
                                                            int nb, const int64_t* __restrict__ iv_ptr,
                                                            uint32_t* __restrict__ iv, int runs_cap,
                                                            int32_t* __restrict__ kept_out) {
  extern __shared__ uint32_t run_stage[];
  const int lane = threadIdx.x & 63;
  uint32_t* const buf = run_stage + (threadIdx.x >> 6) * runs_cap;
  uint16_t* const half = reinterpret_cast<uint16_t*>(buf);
  const int mis = (int)((uintptr_t)masks & 15);
  const int64_t total = rows * nb;
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  for (int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); row < rows; row += stride) {
    const RowSpan r = row_span(row, nb, mis);
    uint32_t carry = 0u;
    int n_open = 0, n_close = 0, n_kept = 0;
    for (int64_t w = r.cs0; w < r.e; w += kWin) {
      const int64_t cs = w + 16 * lane;
      const uint32_t bits = chunk_bits(masks, total, r.s, r.e, cs);
      n_kept += __popc(bits);
      uint32_t prev = (__shfl_up(bits, 1) >> 15) & 1u;
      if (lane == 0) prev = carry;
      uint32_t next = __shfl_down(bits, 1) & 1u;   // first byte of the lane after
      if (lane == 63) {                             // first byte of the next window, if in the row
        const int64_t nx = cs + 16;
        next = (nx >= r.s && nx < r.e && masks[nx] != 0) ? 1u : 0u;
      }
      const uint32_t opens = bits & ~((bits << 1) | prev);
      const uint32_t closes = bits & ~((bits >> 1) | (next << 15));
      const int no = __popc(opens), nc = __popc(closes);
      const int io = wave_inclusive_scan(no, lane), ic = wave_inclusive_scan(nc, lane);
      const int c0 = (int)(cs - r.s);
      int ko = n_open + io - no, kc = n_close + ic - nc;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if ((opens >> j) & 1u) half[2 * ko++] = (uint16_t)(c0 + j);
        if ((closes >> j) & 1u) half[2 * kc++ + 1] = (uint16_t)(c0 + j + 1);
      }
      n_open += __shfl(io, 63);
      n_close += __shfl(ic, 63);
      carry = (__shfl(bits, 63) >> 15) & 1u;
    }
    const int64_t base = iv_ptr[row];
    for (int i = lane; i < n_open; i += 64) iv[base + i] = buf[i];
    if (kept_out) {
      n_kept = wave_sum(n_kept);
      if (lane == 0) kept_out[row] = n_kept;
    }
  }
}

// Same ranking as order_kernel; each row's kept count was left in order[] by
// run_fill. One workgroup takes all groups of a record, and reads every count
// into LDS before the ranks overwrite them; it has 16 waves, so that a single
// layer's few records still keep every SIMD of their CUs busy.
constexpr int kRunOrderThreads = 1024;

__global__ __launch_bounds__(kRunOrderThreads) void run_order_kernel(int nb, int32_t* __restrict__ order) {
  extern __shared__ int4 order_lds[];
  int32_t* key = reinterpret_cast<int32_t*>(order_lds);
  const int groups = (nb + 63) / 64;
  const OrderSlice sl = order_slice(nb, groups);
  for (int r = threadIdx.x; r < order_padded(nb); r += kRunOrderThreads)
    key[r] = r < nb ? order_key(order[sl.row0 + r], r) : -1;
  __syncthreads();
  rank_groups<kRunOrderThreads / 64>(key, nb, sl.row0, sl.g0, sl.g1, order);
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

// Bitmap form: row r's key block c is bit c % 64 of word c / 64 of the row's
// `words` words. One wave per row, waves striding over rows two at a time. A
// window is 60 of the row's aligned 16-byte chunks (each lane loads one chunk
// of 64; the last 4 are the next window's first) and yields 15 words. With off
// = the row's first byte's place in its first chunk, the window's word k is
// bits 64k + off .. 64k + off + 63 of its chunk-bit stream: chunks 4k .. 4k + 4.
// Bytes outside the row count as 0, so the padding bits past nb stay 0.
constexpr int kWinChunks = 60;
constexpr int kWinWords = kWinChunks / 4;

__device__ __forceinline__ uint64_t window_word(uint32_t x, int lane, int off) {
  const int src = (4 * lane) & 63;   // lanes >= kWinWords compute a word that is not stored
  const uint64_t a0 = (uint32_t)__shfl((int)x, src);
  const uint64_t a1 = (uint32_t)__shfl((int)x, src + 1);
  const uint64_t a2 = (uint32_t)__shfl((int)x, src + 2);
  const uint64_t a3 = (uint32_t)__shfl((int)x, src + 3);
  const uint64_t a4 = (uint32_t)__shfl((int)x, (src + 4) & 63);
  uint64_t w = (a0 >> off) | (a1 << (16 - off)) | (a2 << (32 - off)) | (a3 << (48 - off));
  if (off) w |= a4 << (64 - off);
  return w;
}

__global__ __launch_bounds__(kThreads) void bitmap_kernel(const uint8_t* __restrict__ masks, int64_t rows, int nb,
                                                          int words, uint64_t* __restrict__ bits) {
  const int lane = threadIdx.x & 63;
  const int mis = (int)((uintptr_t)masks & 15);
  const int64_t total = rows * nb;
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  for (int64_t ra = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); ra < rows; ra += 2 * stride) {
    const int64_t rb = ra + stride;
    const bool has_b = rb < rows;
    const RowSpan a = row_span(ra, nb, mis);
    const RowSpan b = row_span(has_b ? rb : ra, nb, mis);
    for (int w0 = 0; w0 < words; w0 += kWinWords) {
      const int64_t c0 = (int64_t)w0 / kWinWords * kWinChunks * 16 + 16 * lane;
      const uint32_t xa = chunk_bits(masks, total, a.s, a.e, a.cs0 + c0);
      const uint32_t xb = chunk_bits(masks, total, b.s, b.e, b.cs0 + c0);
      const uint64_t wa = window_word(xa, lane, (int)(a.s - a.cs0));
      const uint64_t wb = window_word(xb, lane, (int)(b.s - b.cs0));
      const int k = w0 + lane;
      if (lane < kWinWords && k < words) {
        bits[ra * words + k] = wa;
        if (has_b) bits[rb * words + k] = wb;
      }
    }
  }
}

}  // namespace

// Workgroups of the row-striding kernels: enough waves to keep every CU's
// loads in flight, no more than the rows need.
unsigned stride_grid(int64_t rows) {
  const int64_t need = (rows + kWaves - 1) / kWaves;
  return (unsigned)(need < 4096 ? need : 4096);
}

hipError_t launch_compile_count_scan(const uint8_t* masks, int64_t rows, int nb, int64_t* row_ptr,
                                     hipStream_t s) {
  const unsigned grid = stride_grid(rows);
  hipLaunchKernelGGL(count_kernel, dim3(grid), dim3(kThreads), 0, s, masks, rows, nb, row_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return scan_counts(rows, row_ptr, s);
}

hipError_t launch_compile_bitmap(const uint8_t* masks, int64_t rows, int nb, uint64_t* bits, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int words = (nb + 63) / 64;
  if (words > 64) return hipErrorInvalidValue;   // (nb <= CALIBATT_MAX_NB: at most 64 words, one per lane)
  hipLaunchKernelGGL(bitmap_kernel, dim3(stride_grid(rows)), dim3(kThreads), 0, s, masks, rows, nb, words, bits);
  return hipGetLastError();
}

hipError_t launch_compile_fill(const uint8_t* masks, int64_t rows, int nb, const int64_t* row_ptr,
                               int32_t* col_idx, hipStream_t s) {
  const unsigned grid = stride_grid(rows);
  hipLaunchKernelGGL(fill_kernel, dim3(grid), dim3(kThreads), 0, s, masks, rows, nb, row_ptr, col_idx);
  return hipGetLastError();
}

// Groups of 64 rows per ordering workgroup: one, while the records' groups
// alone do not fill the chip many times over; else all groups of a record
// (its keys are then loaded once).
static int order_groups_per_wg(int64_t records, int nb) {
  const int groups = (nb + 63) / 64;
  return records * groups <= 8192 ? 1 : groups;
}

static unsigned order_grid(int64_t records, int nb, int gpw) {
  const int groups = (nb + 63) / 64;
  return (unsigned)(records * ((groups + gpw - 1) / gpw));
}

hipError_t launch_compile_order(const int64_t* row_ptr, int64_t records, int nb, int32_t* order,
                                hipStream_t s) {
  const int gpw = order_groups_per_wg(records, nb);
  const size_t lds = (size_t)((nb + 3) & ~3) * sizeof(int32_t);
  hipLaunchKernelGGL(order_kernel, dim3(order_grid(records, nb, gpw)), dim3(kThreads), lds, s, row_ptr, nb, gpw,
                     order);
  return hipGetLastError();
}

hipError_t launch_compile_runs_count_scan(const uint8_t* masks, int64_t rows, int nb, int64_t* iv_ptr,
                                          hipStream_t s) {
  const unsigned grid = stride_grid(rows);
  hipLaunchKernelGGL(run_count_kernel, dim3(grid), dim3(kThreads), 0, s, masks, rows, nb, iv_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return scan_counts(rows, iv_ptr, s);
}

hipError_t launch_compile_runs_fill(const uint8_t* masks, int64_t rows, int nb, const int64_t* iv_ptr,
                                    uint32_t* iv, int32_t* kept_out, hipStream_t s) {
  const unsigned grid = stride_grid(rows);
  const int runs_cap = (nb + 1) / 2;
  const size_t lds = (size_t)kWaves * runs_cap * sizeof(uint32_t);
  hipLaunchKernelGGL(run_fill_kernel, dim3(grid), dim3(kThreads), lds, s, masks, rows, nb, iv_ptr, iv, runs_cap,
                     kept_out);
  return hipGetLastError();
}

hipError_t launch_compile_runs_order(int64_t records, int nb, int32_t* order, hipStream_t s) {
  const size_t lds = (size_t)((nb + 3) & ~3) * sizeof(int32_t);
  hipLaunchKernelGGL(run_order_kernel, dim3((unsigned)records), dim3(kRunOrderThreads), lds, s, nb, order);
  return hipGetLastError();
}

}  // namespace calibatt
