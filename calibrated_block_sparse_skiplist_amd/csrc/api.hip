// Host entry points of libcalibatt.so (declared in include/calibatt.h).
//
// Every argument is checked here, before anything is enqueued; the kernels
// assume what these checks establish (sizes, supported d and block sizes,
// head and anchor ranges). The only synchronisation in the library is the
// read-back of the entry count in the two compile calls.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "internal.h"

// Device scratch of calibatt_block_energy_noalloc (CALIBATT_NOALLOC_SCRATCH_BYTES,
// include/calibatt.h): the one-pass energy workspace for callers that cannot
// allocate device memory. Each GPU the
// library runs on holds its own copy from the module's load until the process
// ends. Host code never uses the name `scratch` as an address (on the host it
// is only a stand-in): scratch_on_current_device() looks the device address
// up once per device with hipGetSymbolAddress and every launch takes that.
static __device__ __align__(256) float scratch[CALIBATT_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_ev_begin = nullptr;
thread_local hipEvent_t g_ev_end = nullptr;
thread_local bool g_checked = false;   // checked mode: validate the record's lists before each launch

calibatt_status_t fail(calibatt_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

calibatt_status_t ok() {
  g_err[0] = '\0';
  return CALIBATT_OK;
}

calibatt_status_t hip_fail(hipError_t e, const char* what) {
  return fail(CALIBATT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }



// Checks shared by all attention entry points.
calibatt_status_t check_tensors(const void* q, const void* k, const void* v, void* o, int32_t H, int32_t N,
                                int32_t d, calibatt_dtype_t dtype, float scale) {
  if (!q || !k || !v || !o) return fail(CALIBATT_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
  if (H < 1 || N < 1) return fail(CALIBATT_ERR_INVALID_ARG, "H (%d) and N (%d) must be >= 1", H, N);
  if (d != 64 && d != 128) return fail(CALIBATT_ERR_INVALID_ARG, "d = %d is not supported (64 or 128)", d);
  if (dtype != CALIBATT_BF16 && dtype != CALIBATT_F32)
    return fail(CALIBATT_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(CALIBATT_ERR_INVALID_ARG, "scale must be finite and > 0");
  return CALIBATT_OK;
}

calibatt_status_t check_heads(const int32_t* heads, int32_t n_heads, int32_t H, std::vector<int32_t>& out) {
  out.clear();
  if (!heads) {
    for (int32_t h = 0; h < H; ++h) out.push_back(h);
  } else {
    if (n_heads < 0) return fail(CALIBATT_ERR_INVALID_ARG, "n_heads must be >= 0");
    std::vector<char> seen(H, 0);
    for (int32_t i = 0; i < n_heads; ++i) {
      const int32_t h = heads[i];
      if (h < 0 || h >= H) return fail(CALIBATT_ERR_INVALID_ARG, "head index %d out of range [0, %d)", h, H);
      if (seen[h]) return fail(CALIBATT_ERR_INVALID_ARG, "head index %d listed twice", h);
      seen[h] = 1;
      out.push_back(h);
    }
  }
  if ((int)out.size() > CALIBATT_MAX_HEADS)
    return fail(CALIBATT_ERR_INVALID_ARG, "at most %d heads per call", CALIBATT_MAX_HEADS);
  return CALIBATT_OK;
}

// Any form of a compiled dictionary: index lists (row_ptr, col_idx), runs
// (row_ptr = iv_ptr, runs = iv) or bitmaps (bits, `words` per row).
struct ListView {
  int32_t T, L, H, N, B, nb;
  const int64_t* row_ptr;
  const int32_t* col_idx;
  const uint32_t* runs;
  const int32_t* order;
  const uint64_t* bits;
  int32_t words;
};

calibatt_status_t view_of(const calibatt_skiplist_t* sl, ListView* v) {
  if (!sl) return fail(CALIBATT_ERR_INVALID_ARG, "skip list view is NULL");
  if (!sl->row_ptr || !sl->col_idx) return fail(CALIBATT_ERR_INVALID_ARG, "skip list row_ptr/col_idx are NULL");
  *v = {sl->T, sl->L, sl->H, sl->N, sl->B, sl->nb, sl->row_ptr, sl->col_idx, nullptr, sl->order, nullptr, 0};
  return CALIBATT_OK;
}

calibatt_status_t view_of(const calibatt_intervals_t* il, ListView* v) {
  if (!il) return fail(CALIBATT_ERR_INVALID_ARG, "interval list view is NULL");
  if (!il->iv_ptr || !il->iv) return fail(CALIBATT_ERR_INVALID_ARG, "interval list iv_ptr/iv are NULL");
  *v = {il->T, il->L, il->H, il->N, il->B, il->nb, il->iv_ptr, nullptr, il->iv, il->order, nullptr, 0};
  return CALIBATT_OK;
}

calibatt_status_t view_of(const calibatt_bitmap_t* bm, ListView* v) {
  if (!bm) return fail(CALIBATT_ERR_INVALID_ARG, "bitmap view is NULL");
  if (!bm->bits) return fail(CALIBATT_ERR_INVALID_ARG, "bitmap bits are NULL");
  if (reinterpret_cast<uintptr_t>(bm->bits) % 8 != 0)
    return fail(CALIBATT_ERR_INVALID_ARG, "bitmap bits are not 8-byte aligned");
  if (bm->nb < 1 || bm->words != ceil_div(bm->nb, 64))
    return fail(CALIBATT_ERR_INVALID_ARG, "bitmap words (%d) != ceil(nb/64) with nb = %d", bm->words, bm->nb);
  *v = {bm->T, bm->L, bm->H, bm->N, bm->B, bm->nb, nullptr, nullptr, nullptr, nullptr, bm->bits, bm->words};
  return CALIBATT_OK;
}

calibatt_status_t check_skiplist(const ListView* sl, int32_t H, int32_t N, int32_t t, int32_t l) {
  if (sl->H != H || sl->N != N)
    return fail(CALIBATT_ERR_INVALID_ARG, "skip list is for H=%d N=%d, call has H=%d N=%d", sl->H, sl->N, H, N);
  if (sl->B != 64 && sl->B != 128) return fail(CALIBATT_ERR_INVALID_ARG, "block size %d is not supported", sl->B);
  if (sl->nb != ceil_div(N, sl->B)) return fail(CALIBATT_ERR_INVALID_ARG, "skip list nb != ceil(N/B)");
  if (sl->nb > CALIBATT_MAX_NB) return fail(CALIBATT_ERR_INVALID_ARG, "nb exceeds %d", CALIBATT_MAX_NB);
  if (sl->T < 1 || sl->L < 1) return fail(CALIBATT_ERR_INVALID_ARG, "skip list T and L must be >= 1");
  if (t < 0 || t >= sl->T || l < 0 || l >= sl->L)
    return fail(CALIBATT_ERR_INVALID_ARG, "record (t=%d, l=%d) outside the dictionary (T=%d, L=%d)", t, l, sl->T,
                sl->L);
  return CALIBATT_OK;
}

// ---- checked mode: validation of a caller's list view on the host ----
//
// What the kernels assume of a record's rows and the compile calls guarantee:
// row pointers non-decreasing (and 0 at the start of a whole dictionary);
// index lists strictly ascending inside [0, nb); runs lo < hi <= nb, strictly
// ascending with a gap between neighbours (maximal runs, hence at most
// ceil(nb/2) per row, the space the kernels stage them in); order, when
// given, a permutation of [0, nb) per record.
calibatt_status_t validate_rows(const int64_t* ptr, int64_t row0, int64_t rows, const int32_t* idx,
                                const uint32_t* runs, int64_t base, int32_t nb) {
  for (int64_t i = 0; i < rows; ++i) {
    const int64_t b = ptr[i], e = ptr[i + 1];
    if (b < 0 || e < b)
      return fail(CALIBATT_ERR_INVALID_ARG, "row %lld: row pointers %lld .. %lld are not non-decreasing",
                  (long long)(row0 + i), (long long)b, (long long)e);
    if (idx) {
      if (e - b > nb)
        return fail(CALIBATT_ERR_INVALID_ARG, "row %lld lists %lld key blocks, more than nb = %d",
                    (long long)(row0 + i), (long long)(e - b), nb);
      for (int64_t j = b; j < e; ++j) {
        const int32_t c = idx[j - base];
        if (c < 0 || c >= nb)
          return fail(CALIBATT_ERR_INVALID_ARG, "row %lld: key block %d outside [0, %d)", (long long)(row0 + i), c,
                      nb);
        if (j > b && c <= idx[j - 1 - base])
          return fail(CALIBATT_ERR_INVALID_ARG, "row %lld: key blocks not strictly ascending", (long long)(row0 + i));
      }
    } else {
      if (e - b > (nb + 1) / 2)
        return fail(CALIBATT_ERR_INVALID_ARG, "row %lld holds %lld runs, more than ceil(nb/2) = %d",
                    (long long)(row0 + i), (long long)(e - b), (nb + 1) / 2);
      int32_t prev_hi = -1;
      for (int64_t j = b; j < e; ++j) {
        const uint32_t w = runs[j - base];
        const int32_t lo = (int32_t)(w & 0xffffu), hi = (int32_t)(w >> 16);
        if (!(lo < hi) || hi > nb)
          return fail(CALIBATT_ERR_INVALID_ARG, "row %lld: run [%d, %d) is empty or reaches past nb = %d",
                      (long long)(row0 + i), lo, hi, nb);
        if (lo <= prev_hi)
          return fail(CALIBATT_ERR_INVALID_ARG, "row %lld: runs not ascending with a gap (run [%d, %d) after %d)",
                      (long long)(row0 + i), lo, hi, prev_hi);
        prev_hi = hi;
      }
    }
  }
  return CALIBATT_OK;
}

calibatt_status_t validate_order(const int32_t* order, int64_t records, int32_t nb) {
  std::vector<char> seen(nb);
  for (int64_t r = 0; r < records; ++r) {
    std::fill(seen.begin(), seen.end(), 0);
    for (int32_t i = 0; i < nb; ++i) {
      const int32_t q = order[r * nb + i];
      if (q < 0 || q >= nb || seen[q])
        return fail(CALIBATT_ERR_INVALID_ARG, "order of record %lld is not a permutation of [0, %d)",
                    (long long)r, nb);
      seen[q] = 1;
    }
  }
  return CALIBATT_OK;
}

// Validate the rows of record (t, l) (all heads), or of the whole dictionary
// when t = l = -1. Device arrays are copied to host memory on `s` first.
calibatt_status_t validate_view(const ListView* v, int32_t t, int32_t l, bool host_arrays, hipStream_t s) {
  if (v->T < 1 || v->L < 1 || v->H < 1 || v->N < 1)
    return fail(CALIBATT_ERR_INVALID_ARG, "view sizes T, L, H and N must be >= 1");
  if (v->B < 1 || v->nb != ceil_div(v->N, v->B)) return fail(CALIBATT_ERR_INVALID_ARG, "view nb != ceil(N/B)");
  if (v->nb > CALIBATT_MAX_NB) return fail(CALIBATT_ERR_INVALID_ARG, "nb exceeds %d", CALIBATT_MAX_NB);
  const bool whole = t == -1 && l == -1;
  if (!whole && (t < 0 || t >= v->T || l < 0 || l >= v->L))
    return fail(CALIBATT_ERR_INVALID_ARG, "record (t=%d, l=%d) outside the dictionary (T=%d, L=%d)", t, l, v->T,
                v->L);
  const int64_t rec0 = whole ? 0 : ((int64_t)t * v->L + l) * v->H;
  const int64_t recs = whole ? (int64_t)v->T * v->L * v->H : v->H;
  const int64_t row0 = rec0 * v->nb, rows = recs * v->nb;
  if (v->bits) {
    // bitmaps: the only constraint is that the bits past nb are zero
    const uint64_t* words = v->bits + row0 * v->words;
    std::vector<uint64_t> hw;
    if (!host_arrays) {
      hw.resize(rows * v->words);
      hipError_t e = hipMemcpyAsync(hw.data(), words, hw.size() * sizeof(uint64_t), hipMemcpyDeviceToHost, s);
      if (e == hipSuccess) e = hipStreamSynchronize(s);
      if (e != hipSuccess) return hip_fail(e, "reading the bitmaps");
      words = hw.data();
    }
    if (v->nb % 64) {
      const uint64_t pad = ~((1ull << (v->nb % 64)) - 1ull);
      for (int64_t i = 0; i < rows; ++i)
        if (words[i * v->words + v->words - 1] & pad)
          return fail(CALIBATT_ERR_INVALID_ARG, "row %lld: bits set past nb = %d", (long long)(row0 + i), v->nb);
    }
    return CALIBATT_OK;
  }
  std::vector<int64_t> hp;
  std::vector<int32_t> hi;
  std::vector<uint32_t> hr;
  std::vector<int32_t> ho;
  const int64_t* ptr = v->row_ptr + row0;
  if (!host_arrays) {
    hp.resize(rows + 1);
    hipError_t e = hipMemcpyAsync(hp.data(), ptr, (rows + 1) * sizeof(int64_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "reading the row pointers");
    ptr = hp.data();
  }
  if (whole && ptr[0] != 0) return fail(CALIBATT_ERR_INVALID_ARG, "row_ptr[0] = %lld, not 0", (long long)ptr[0]);
  for (int64_t i = 0; i < rows; ++i)
    if (ptr[i] < 0 || ptr[i + 1] < ptr[i])
      return fail(CALIBATT_ERR_INVALID_ARG, "row %lld: row pointers %lld .. %lld are not non-decreasing",
                  (long long)(row0 + i), (long long)ptr[i], (long long)ptr[i + 1]);
  const int64_t base = ptr[0], count = ptr[rows] - ptr[0];
  const int32_t* idx = v->col_idx ? v->col_idx + base : nullptr;
  const uint32_t* runs = v->runs ? v->runs + base : nullptr;
  const int32_t* order = v->order ? v->order + row0 : nullptr;
  if (!host_arrays) {
    hipError_t e = hipSuccess;
    if (idx && count > 0) {
      hi.resize(count);
      e = hipMemcpyAsync(hi.data(), idx, count * sizeof(int32_t), hipMemcpyDeviceToHost, s);
      idx = hi.data();
    }
    if (e == hipSuccess && runs && count > 0) {
      hr.resize(count);
      e = hipMemcpyAsync(hr.data(), runs, count * sizeof(uint32_t), hipMemcpyDeviceToHost, s);
      runs = hr.data();
    }
    if (e == hipSuccess && order) {
      ho.resize(rows);
      e = hipMemcpyAsync(ho.data(), order, rows * sizeof(int32_t), hipMemcpyDeviceToHost, s);
      order = ho.data();
    }
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "reading the lists");
  }
  calibatt_status_t st = validate_rows(ptr, row0, rows, idx, runs, base, v->nb);
  if (st != CALIBATT_OK) return st;
  if (order && (st = validate_order(order, recs, v->nb)) != CALIBATT_OK) return st;
  return CALIBATT_OK;
}

calibatt_status_t check_anchors(int32_t N, int32_t F, int32_t R, int32_t C, const int32_t* anchors, int32_t k) {
  if (F < 1 || R < 1 || C < 1) return fail(CALIBATT_ERR_INVALID_ARG, "F, R, C must be >= 1");
  if ((int64_t)F * R * C != N) return fail(CALIBATT_ERR_INVALID_ARG, "N (%d) != F*R*C (%d*%d*%d)", N, F, R, C);
  if (!anchors) return fail(CALIBATT_ERR_INVALID_ARG, "anchor_rows is NULL");
  if (k < 1 || k > R || k > CALIBATT_MAX_ANCHORS)
    return fail(CALIBATT_ERR_INVALID_ARG, "anchor count %d must be in [1, min(R, %d)]", k, CALIBATT_MAX_ANCHORS);
  for (int32_t i = 0; i < k; ++i) {
    if (anchors[i] < 0 || anchors[i] >= R)
      return fail(CALIBATT_ERR_INVALID_ARG, "anchor row %d outside [0, %d)", anchors[i], R);
    if (i > 0 && anchors[i] <= anchors[i - 1])
      return fail(CALIBATT_ERR_INVALID_ARG, "anchor rows must be strictly ascending");
  }
  return CALIBATT_OK;
}

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// check_heads without heap use: distinct heads in [0, H), at most CALIBATT_MAX_HEADS, into out[].
calibatt_status_t check_heads_fixed(const int32_t* heads, int32_t n_heads, int32_t H, int32_t* out, int32_t* n_out) {
  if (!heads) {
    if (H > CALIBATT_MAX_HEADS) return fail(CALIBATT_ERR_INVALID_ARG, "at most %d heads per call", CALIBATT_MAX_HEADS);
    for (int32_t h = 0; h < H; ++h) out[h] = h;
    *n_out = H;
    return CALIBATT_OK;
  }
  if (n_heads < 0) return fail(CALIBATT_ERR_INVALID_ARG, "n_heads must be >= 0");
  if (n_heads > CALIBATT_MAX_HEADS) return fail(CALIBATT_ERR_INVALID_ARG, "at most %d heads per call", CALIBATT_MAX_HEADS);
  for (int32_t i = 0; i < n_heads; ++i) {
    const int32_t h = heads[i];
    if (h < 0 || h >= H) return fail(CALIBATT_ERR_INVALID_ARG, "head index %d out of range [0, %d)", h, H);
    for (int32_t j = 0; j < i; ++j)
      if (out[j] == h) return fail(CALIBATT_ERR_INVALID_ARG, "head index %d listed twice", h);
    out[i] = h;
  }
  *n_out = n_heads;
  return CALIBATT_OK;
}

void fill_common(calibatt::AttnParams& p, const void* q, const void* k, const void* v, void* o, float* lse,
                 int32_t N, int32_t d, int32_t blk, float scale) {
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.head_stride = (int64_t)N * d;
  p.N = N;
  p.nb = (int32_t)ceil_div(N, blk);
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  // Work order: query blocks in block order (neighbours share key blocks), in
  // runs of consecutive items per XCD: about as many as an XCD runs at once, so
  // that the items running together start and walk their lists together (64 at
  // d = 128, B = 128: two workgroups on each of an XCD's 32 CUs; the smaller
  // variants run more at once; each value the fastest measured at the Wan-720p
  // shape). Heaviest-first order per record (the compiled `order`) measured no
  // faster on the Wan-shaped layers, so the kernels do not read it. Each XCD's
  // share of the grid is fixed by the round-robin dispatch, so when runs cover
  // whole heads (nb divides or is a multiple of 8 * xcd_group) the chunks turn
  // per run: otherwise an XCD would take the same, lighter or heavier, slice of
  // every head.
  p.xcd_group = (d == 128 && blk == 128) ? 64 : (d == 64 && blk == 64) ? 192 : 128;
  p.xcd_rotate = p.nb > 0 && (p.nb % (8 * p.xcd_group) == 0 || (8 * p.xcd_group) % p.nb == 0) ? 1 : 0;
}

void fill_sparse(calibatt::AttnParams& p, const ListView* sl, int32_t t, int32_t l,
                 const std::vector<int32_t>& heads) {
  p.row_ptr = sl->row_ptr;
  p.col_idx = sl->col_idx;
  p.runs = sl->runs;
  p.bits = sl->bits;
  p.bm_words = sl->words;
  p.rec_head_rows = sl->nb;
  p.rec_row0 = ((int64_t)t * sl->L + l) * sl->H * sl->nb;
  p.n_sparse = (int32_t)heads.size();
  for (size_t i = 0; i < heads.size(); ++i) p.sparse_heads[i] = heads[i];
}

void fill_anchor(calibatt::AttnParams& p, int32_t F, int32_t R, int32_t C, const int32_t* anchors, int32_t k,
                 const std::vector<int32_t>& heads, int32_t blk) {
  p.F = F;
  p.R = R;
  p.C = C;
  p.ka = k;
  for (int32_t i = 0; i < k; ++i) p.anchors[i] = anchors[i];
  p.n_anchor_q = F * k * C;
  p.anchor_tiles = (int32_t)ceil_div(p.n_anchor_q, blk);
  p.n_anchor = (int32_t)heads.size();
  for (size_t i = 0; i < heads.size(); ++i) p.anchor_heads[i] = heads[i];
}

calibatt_status_t run_attention(const calibatt::AttnParams& p, int32_t d, int32_t blk, calibatt_dtype_t dtype,
                                hipStream_t s) {
  hipEvent_t eb = g_ev_begin, ee = g_ev_end;
  g_ev_begin = g_ev_end = nullptr;
  hipError_t e;
  if (eb && (e = hipEventRecord(eb, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  e = dtype == CALIBATT_BF16 ? calibatt::launch_attn_bf16(p, d, blk, s) : calibatt::launch_attn_f32(p, d, blk, s);
  if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  if (ee && (e = hipEventRecord(ee, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  return CALIBATT_OK;
}

calibatt_status_t run_broadcast(void* o, float* lse, int32_t N, int32_t d, calibatt_dtype_t dtype, int32_t F,
                                int32_t R, int32_t C, const int32_t* anchors, int32_t k,
                                const std::vector<int32_t>& heads, hipStream_t s) {
  if (heads.empty() || k == R) return CALIBATT_OK;   // every row is an anchor row
  calibatt::BcastParams b;
  std::memset(&b, 0, sizeof(b));
  b.o = o;
  b.lse = lse;
  b.head_stride = (int64_t)N * d;
  b.N = N;
  b.d = d;
  b.esize = dtype == CALIBATT_BF16 ? 2 : 4;
  b.F = F;
  b.R = R;
  b.C = C;
  b.ka = k;
  for (int32_t i = 0; i < k; ++i) b.anchors[i] = anchors[i];
  b.n_heads = (int32_t)heads.size();
  for (size_t i = 0; i < heads.size(); ++i) b.heads[i] = heads[i];
  hipError_t e = calibatt::launch_broadcast(b, s);
  if (e != hipSuccess) return hip_fail(e, "broadcast kernel launch");
  return CALIBATT_OK;
}

// Both compile entry points: count (and scan) per row, read the total back,
// then fill and order. `runs` selects the interval form.
calibatt_status_t compile_impl(const uint8_t* masks, int32_t T, int32_t L, int32_t H, int32_t N, int32_t B,
                               int64_t* ptr, void* out, int64_t capacity, int32_t* order, int64_t* total_out,
                               bool runs, void* stream) {
  if (!masks || !ptr || !total_out)
    return fail(CALIBATT_ERR_INVALID_ARG, "masks, the row pointer array and the count output must be non-NULL");
  if (T < 1 || L < 1 || H < 1 || N < 1 || B < 1)
    return fail(CALIBATT_ERR_INVALID_ARG, "T, L, H, N and B must be >= 1");
  const int64_t nb = ceil_div(N, B);
  if (nb > CALIBATT_MAX_NB) return fail(CALIBATT_ERR_INVALID_ARG, "nb = %lld exceeds %d", (long long)nb, CALIBATT_MAX_NB);
  if (out && capacity < 0) return fail(CALIBATT_ERR_INVALID_ARG, "capacity must be >= 0");
  const int64_t records = (int64_t)T * L * H;
  const int64_t rows = records * nb;
  hipStream_t s = static_cast<hipStream_t>(stream);

  hipError_t e = runs ? calibatt::launch_compile_runs_count_scan(masks, rows, (int)nb, ptr, s)
                      : calibatt::launch_compile_count_scan(masks, rows, (int)nb, ptr, s);
  if (e != hipSuccess) return hip_fail(e, "skip-list count kernel launch");
  int64_t total = 0;
  e = hipMemcpyAsync(&total, ptr + rows, sizeof(int64_t), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "reading the entry count");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "synchronising after the count pass");
  *total_out = total;
  if (!out) return ok();
  if (capacity < total)
    return fail(CALIBATT_ERR_CAPACITY, "the output holds %lld entries, %lld needed", (long long)capacity,
                (long long)total);
  // (the interval fill leaves each row's kept count in order for the ranking)
  e = runs ? calibatt::launch_compile_runs_fill(masks, rows, (int)nb, ptr, static_cast<uint32_t*>(out), order, s)
           : calibatt::launch_compile_fill(masks, rows, (int)nb, ptr, static_cast<int32_t*>(out), s);
  if (e != hipSuccess) return hip_fail(e, "skip-list fill kernel launch");
  if (order) {
    e = runs ? calibatt::launch_compile_runs_order(records, (int)nb, order, s)
             : calibatt::launch_compile_order(ptr, records, (int)nb, order, s);
    if (e != hipSuccess) return hip_fail(e, "skip-list order kernel launch");
  }
  return ok();
}

calibatt_status_t sparse_impl(const void* q, const void* k, const void* v, void* o, float* lse, int32_t H,
                              int32_t N, int32_t d, calibatt_dtype_t dtype, float scale, const ListView* sl,
                              int32_t t, int32_t l, const int32_t* heads, int32_t n_heads, void* stream) {
  calibatt_status_t st = check_skiplist(sl, H, N, t, l);
  if (st != CALIBATT_OK) return st;
  if (g_checked && (st = validate_view(sl, t, l, false, static_cast<hipStream_t>(stream))) != CALIBATT_OK) return st;
  std::vector<int32_t> hs;
  if ((st = check_heads(heads, n_heads, H, hs)) != CALIBATT_OK) return st;
  calibatt::AttnParams p;
  fill_common(p, q, k, v, o, lse, N, d, sl->B, scale);
  fill_sparse(p, sl, t, l, hs);
  if ((st = run_attention(p, d, sl->B, dtype, static_cast<hipStream_t>(stream))) != CALIBATT_OK) return st;
  return ok();
}

calibatt_status_t dispatch_impl(const void* q, const void* k, const void* v, void* o, float* lse, int32_t H,
                                int32_t N, int32_t d, calibatt_dtype_t dtype, float scale, const ListView* sl,
                                int32_t t, int32_t l, const uint8_t* rep_flags, int32_t F, int32_t R, int32_t C,
                                const int32_t* anchor_rows, int32_t k_anchors, void* stream) {
  calibatt_status_t st = check_skiplist(sl, H, N, t, l);
  if (st != CALIBATT_OK) return st;
  if (!rep_flags) return fail(CALIBATT_ERR_INVALID_ARG, "rep_flags is NULL");
  if (g_checked && (st = validate_view(sl, t, l, false, static_cast<hipStream_t>(stream))) != CALIBATT_OK) return st;
  if (H > CALIBATT_MAX_HEADS) return fail(CALIBATT_ERR_INVALID_ARG, "at most %d heads", CALIBATT_MAX_HEADS);
  // Record selection: the flags of (t, l) split the heads into the two paths.
  std::vector<int32_t> sparse_heads, rep_heads;
  const uint8_t* fl = rep_flags + ((int64_t)t * sl->L + l) * sl->H;
  for (int32_t h = 0; h < H; ++h) (fl[h] ? rep_heads : sparse_heads).push_back(h);
  if (!rep_heads.empty() && (st = check_anchors(N, F, R, C, anchor_rows, k_anchors)) != CALIBATT_OK) return st;
  // One launch covers both paths: anchor tiles (every key block) first, then
  // the block-sparse query blocks.
  calibatt::AttnParams p;
  fill_common(p, q, k, v, o, lse, N, d, sl->B, scale);
  fill_sparse(p, sl, t, l, sparse_heads);
  if (!rep_heads.empty()) fill_anchor(p, F, R, C, anchor_rows, k_anchors, rep_heads, sl->B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = run_attention(p, d, sl->B, dtype, s)) != CALIBATT_OK) return st;
  if (!rep_heads.empty() &&
      (st = run_broadcast(o, lse, N, d, dtype, F, R, C, anchor_rows, k_anchors, rep_heads, s)) != CALIBATT_OK)
    return st;
  return ok();
}

}  // namespace

extern "C" {

const char* calibatt_last_error(void) { return g_err; }

int32_t calibatt_version(void) { return 100; }

void calibatt_set_kernel_events(void* begin, void* end) {
  g_ev_begin = static_cast<hipEvent_t>(begin);
  g_ev_end = static_cast<hipEvent_t>(end);
}

void calibatt_set_checked_mode(int32_t enabled) { g_checked = enabled != 0; }

calibatt_status_t calibatt_validate_skiplist(const calibatt_skiplist_t* sl, int32_t t, int32_t l,
                                             int32_t host_arrays, void* stream) {
  ListView view;
  calibatt_status_t st = view_of(sl, &view);
  if (st != CALIBATT_OK) return st;
  if ((st = validate_view(&view, t, l, host_arrays != 0, static_cast<hipStream_t>(stream))) != CALIBATT_OK) return st;
  return ok();
}

calibatt_status_t calibatt_validate_intervals(const calibatt_intervals_t* il, int32_t t, int32_t l,
                                              int32_t host_arrays, void* stream) {
  ListView view;
  calibatt_status_t st = view_of(il, &view);
  if (st != CALIBATT_OK) return st;
  if ((st = validate_view(&view, t, l, host_arrays != 0, static_cast<hipStream_t>(stream))) != CALIBATT_OK) return st;
  return ok();
}

calibatt_status_t calibatt_validate_bitmap(const calibatt_bitmap_t* bm, int32_t t, int32_t l, int32_t host_arrays,
                                           void* stream) {
  ListView view;
  calibatt_status_t st = view_of(bm, &view);
  if (st != CALIBATT_OK) return st;
  if ((st = validate_view(&view, t, l, host_arrays != 0, static_cast<hipStream_t>(stream))) != CALIBATT_OK) return st;
  return ok();
}

calibatt_status_t calibatt_compile_bitmap(const uint8_t* masks, int32_t T, int32_t L, int32_t H, int32_t N, int32_t B,
                                          uint64_t* bits, void* stream) {
  if (!masks || !bits) return fail(CALIBATT_ERR_INVALID_ARG, "masks and bits must be non-NULL");
  if (T < 1 || L < 1 || H < 1 || N < 1 || B < 1)
    return fail(CALIBATT_ERR_INVALID_ARG, "T, L, H, N and B must be >= 1");
  const int64_t nb = ceil_div(N, B);
  if (nb > CALIBATT_MAX_NB) return fail(CALIBATT_ERR_INVALID_ARG, "nb = %lld exceeds %d", (long long)nb, CALIBATT_MAX_NB);
  if (reinterpret_cast<uintptr_t>(bits) % 8 != 0) return fail(CALIBATT_ERR_INVALID_ARG, "bits is not 8-byte aligned");
  const int64_t rows = (int64_t)T * L * H * nb;
  hipError_t e = calibatt::launch_compile_bitmap(masks, rows, (int)nb, bits, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bitmap kernel launch");
  return ok();
}

calibatt_status_t calibatt_compile_skiplist(const uint8_t* masks, int32_t T, int32_t L, int32_t H, int32_t N,
                                            int32_t B, int64_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                            int32_t* order, int64_t* nnz_out, void* stream) {
  return compile_impl(masks, T, L, H, N, B, row_ptr, col_idx, col_capacity, order, nnz_out, false, stream);
}

calibatt_status_t calibatt_compile_intervals(const uint8_t* masks, int32_t T, int32_t L, int32_t H, int32_t N,
                                             int32_t B, int64_t* iv_ptr, uint32_t* iv, int64_t iv_capacity,
                                             int32_t* order, int64_t* n_iv_out, void* stream) {
  return compile_impl(masks, T, L, H, N, B, iv_ptr, iv, iv_capacity, order, n_iv_out, true, stream);
}

calibatt_status_t calibatt_block_sparse_attn(const void* q, const void* k, const void* v, void* o, float* lse,
                                             int32_t H, int32_t N, int32_t d, calibatt_dtype_t dtype, float scale,
                                             const calibatt_skiplist_t* sl, int32_t t, int32_t l,
                                             const int32_t* heads, int32_t n_heads, void* stream) {
  calibatt_status_t st = check_tensors(q, k, v, o, H, N, d, dtype, scale);
  if (st != CALIBATT_OK) return st;
  ListView view;
  if ((st = view_of(sl, &view)) != CALIBATT_OK) return st;
  return sparse_impl(q, k, v, o, lse, H, N, d, dtype, scale, &view, t, l, heads, n_heads, stream);
}

calibatt_status_t calibatt_block_sparse_attn_iv(const void* q, const void* k, const void* v, void* o, float* lse,
                                                int32_t H, int32_t N, int32_t d, calibatt_dtype_t dtype,
                                                float scale, const calibatt_intervals_t* il, int32_t t, int32_t l,
                                                const int32_t* heads, int32_t n_heads, void* stream) {
  calibatt_status_t st = check_tensors(q, k, v, o, H, N, d, dtype, scale);
  if (st != CALIBATT_OK) return st;
  ListView view;
  if ((st = view_of(il, &view)) != CALIBATT_OK) return st;
  return sparse_impl(q, k, v, o, lse, H, N, d, dtype, scale, &view, t, l, heads, n_heads, stream);
}

calibatt_status_t calibatt_block_sparse_attn_bm(const void* q, const void* k, const void* v, void* o, float* lse,
                                                int32_t H, int32_t N, int32_t d, calibatt_dtype_t dtype,
                                                float scale, const calibatt_bitmap_t* bm, int32_t t, int32_t l,
                                                const int32_t* heads, int32_t n_heads, void* stream) {
  calibatt_status_t st = check_tensors(q, k, v, o, H, N, d, dtype, scale);
  if (st != CALIBATT_OK) return st;
  ListView view;
  if ((st = view_of(bm, &view)) != CALIBATT_OK) return st;
  return sparse_impl(q, k, v, o, lse, H, N, d, dtype, scale, &view, t, l, heads, n_heads, stream);
}

calibatt_status_t calibatt_anchor_attn(const void* q, const void* k, const void* v, void* o, float* lse, int32_t H,
                                       int32_t N, int32_t d, calibatt_dtype_t dtype, float scale, int32_t F,
                                       int32_t R, int32_t C, const int32_t* anchor_rows, int32_t k_anchors,
                                       const int32_t* heads, int32_t n_heads, void* stream) {
  calibatt_status_t st = check_tensors(q, k, v, o, H, N, d, dtype, scale);
  if (st != CALIBATT_OK) return st;
  if ((st = check_anchors(N, F, R, C, anchor_rows, k_anchors)) != CALIBATT_OK) return st;
  std::vector<int32_t> hs;
  if ((st = check_heads(heads, n_heads, H, hs)) != CALIBATT_OK) return st;
  const int32_t blk = dtype == CALIBATT_BF16 ? 128 : 64;
  if (ceil_div(N, blk) > CALIBATT_MAX_NB) return fail(CALIBATT_ERR_INVALID_ARG, "N too large");
  calibatt::AttnParams p;
  fill_common(p, q, k, v, o, lse, N, d, blk, scale);
  fill_anchor(p, F, R, C, anchor_rows, k_anchors, hs, blk);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = run_attention(p, d, blk, dtype, s)) != CALIBATT_OK) return st;
  if ((st = run_broadcast(o, lse, N, d, dtype, F, R, C, anchor_rows, k_anchors, hs, s)) != CALIBATT_OK) return st;
  return ok();
}

calibatt_status_t calibatt_layer_dispatch(const void* q, const void* k, const void* v, void* o, float* lse,
                                          int32_t H, int32_t N, int32_t d, calibatt_dtype_t dtype, float scale,
                                          const calibatt_skiplist_t* sl, int32_t t, int32_t l,
                                          const uint8_t* rep_flags, int32_t F, int32_t R, int32_t C,
                                          const int32_t* anchor_rows, int32_t k_anchors, void* stream) {
  calibatt_status_t st = check_tensors(q, k, v, o, H, N, d, dtype, scale);
  if (st != CALIBATT_OK) return st;
  ListView view;
  if ((st = view_of(sl, &view)) != CALIBATT_OK) return st;
  return dispatch_impl(q, k, v, o, lse, H, N, d, dtype, scale, &view, t, l, rep_flags, F, R, C, anchor_rows,
                       k_anchors, stream);
}

calibatt_status_t calibatt_layer_dispatch_iv(const void* q, const void* k, const void* v, void* o, float* lse,
                                             int32_t H, int32_t N, int32_t d, calibatt_dtype_t dtype, float scale,
                                             const calibatt_intervals_t* il, int32_t t, int32_t l,
                                             const uint8_t* rep_flags, int32_t F, int32_t R, int32_t C,
                                             const int32_t* anchor_rows, int32_t k_anchors, void* stream) {
  calibatt_status_t st = check_tensors(q, k, v, o, H, N, d, dtype, scale);
  if (st != CALIBATT_OK) return st;
  ListView view;
  if ((st = view_of(il, &view)) != CALIBATT_OK) return st;
  return dispatch_impl(q, k, v, o, lse, H, N, d, dtype, scale, &view, t, l, rep_flags, F, R, C, anchor_rows,
                       k_anchors, stream);
}

calibatt_status_t calibatt_layer_dispatch_bm(const void* q, const void* k, const void* v, void* o, float* lse,
                                             int32_t H, int32_t N, int32_t d, calibatt_dtype_t dtype, float scale,
                                             const calibatt_bitmap_t* bm, int32_t t, int32_t l,
                                             const uint8_t* rep_flags, int32_t F, int32_t R, int32_t C,
                                             const int32_t* anchor_rows, int32_t k_anchors, void* stream) {
  calibatt_status_t st = check_tensors(q, k, v, o, H, N, d, dtype, scale);
  if (st != CALIBATT_OK) return st;
  ListView view;
  if ((st = view_of(bm, &view)) != CALIBATT_OK) return st;
  return dispatch_impl(q, k, v, o, lse, H, N, d, dtype, scale, &view, t, l, rep_flags, F, R, C, anchor_rows,
                       k_anchors, stream);
}

calibatt_status_t calibatt_block_energy(const void* q, const void* k, int32_t H, int32_t N, int32_t d,
                                        calibatt_dtype_t dtype, float scale, int32_t B, float* energy,
                                        const int32_t* heads, int32_t n_heads, float* work, int64_t work_bytes,
                                        void* stream) {
  // (v and o are not used: the placeholders pass the shared tensor checks)
  calibatt_status_t st = check_tensors(q, k, q, energy, H, N, d, dtype, scale);
  if (st != CALIBATT_OK) return st;
  if (B != 64 && B != 128) return fail(CALIBATT_ERR_INVALID_ARG, "block size %d is not supported", B);
  const int64_t nb = ceil_div(N, B);
  if (nb > CALIBATT_MAX_NB) return fail(CALIBATT_ERR_INVALID_ARG, "nb exceeds %d", CALIBATT_MAX_NB);
  std::vector<int32_t> hs;
  if ((st = check_heads(heads, n_heads, H, hs)) != CALIBATT_OK) return st;
  // one-pass workspace: nb * nb * B floats per head of a launch (bf16 only)
  const int64_t per_head = nb * nb * B * (int64_t)sizeof(float);
  const bool one_pass = work != nullptr && dtype == CALIBATT_BF16;
  if (work && work_bytes < per_head)
    return fail(CALIBATT_ERR_INVALID_ARG, "work_bytes %lld < %lld (nb*nb*B floats, one head)", (long long)work_bytes,
                (long long)per_head);
  if (reinterpret_cast<uintptr_t>(work) % 16 != 0) return fail(CALIBATT_ERR_INVALID_ARG, "work is not 16-byte aligned");
  const int64_t chunk = one_pass ? std::min<int64_t>((int64_t)hs.size(), work_bytes / per_head) : (int64_t)hs.size();
  calibatt::EnergyParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.energy = energy;
  p.work = one_pass ? work : nullptr;
  p.head_stride = (int64_t)N * d;
  p.N = N;
  p.nb = (int32_t)nb;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.dtype_f32 = dtype == CALIBATT_F32 ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t eb = g_ev_begin, ee = g_ev_end;
  g_ev_begin = g_ev_end = nullptr;
  hipError_t e;
  if (eb && (e = hipEventRecord(eb, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  // heads in launches of at most `chunk` (the workspace holds one launch)
  for (size_t h0 = 0; h0 < hs.size(); h0 += (size_t)std::max<int64_t>(chunk, 1)) {
    const size_t h1 = std::min(hs.size(), h0 + (size_t)std::max<int64_t>(chunk, 1));
    p.n_heads = (int32_t)(h1 - h0);
    for (size_t i = h0; i < h1; ++i) p.heads[i - h0] = hs[i];
    if ((e = calibatt::launch_energy(p, d, B, s)) != hipSuccess) return hip_fail(e, "block energy kernel launch");
  }
  if (ee && (e = hipEventRecord(ee, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  return ok();
}

calibatt_status_t calibatt_block_energy_noalloc(const void* q, const void* k, int32_t H, int32_t N, int32_t d,
                                                calibatt_dtype_t dtype, float scale, int32_t B, float* energy,
                                                const int32_t* heads, int32_t n_heads, void* stream) {
  calibatt_status_t st = check_tensors(q, k, q, energy, H, N, d, dtype, scale);
  if (st != CALIBATT_OK) return st;
  if (B != 64 && B != 128) return fail(CALIBATT_ERR_INVALID_ARG, "block size %d is not supported", B);
  const int64_t nb = ceil_div(N, B);
  if (nb > CALIBATT_MAX_NB) return fail(CALIBATT_ERR_INVALID_ARG, "nb exceeds %d", CALIBATT_MAX_NB);
  int32_t hs[CALIBATT_MAX_HEADS];
  int32_t nh = 0;
  if ((st = check_heads_fixed(heads, n_heads, H, hs, &nh)) != CALIBATT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (s) {
    int cur = -1, sdev = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_fail(e, "hipGetDevice");
    if ((e = hipStreamGetDevice(s, &sdev)) != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    if (sdev != cur)
      return fail(CALIBATT_ERR_INVALID_ARG, "stream is on device %d, the current device is %d", sdev, cur);
  }
  // one query block's workspace: nb * B floats; a launch holds as many as the scratch does
  const int64_t per_item = nb * B * (int64_t)sizeof(float);
  if (dtype == CALIBATT_BF16 && per_item > (int64_t)CALIBATT_NOALLOC_SCRATCH_BYTES)
    return fail(CALIBATT_ERR_CAPACITY, "a query block's workspace (%lld bytes) exceeds the scratch (%llu bytes)",
                (long long)per_item, (unsigned long long)CALIBATT_NOALLOC_SCRATCH_BYTES);
  calibatt::EnergyParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.energy = energy;
  p.head_stride = (int64_t)N * d;
  p.N = N;
  p.nb = (int32_t)nb;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.dtype_f32 = dtype == CALIBATT_F32 ? 1 : 0;
  p.n_heads = nh;
  for (int32_t i = 0; i < nh; ++i) p.heads[i] = hs[i];
  if (dtype == CALIBATT_BF16) {
    void* ptr = nullptr;
    if ((e = scratch_on_current_device(&ptr)) != hipSuccess) return hip_fail(e, "device scratch lookup");
    p.work = static_cast<float*>(ptr);
  }
  hipEvent_t eb = g_ev_begin, ee = g_ev_end;
  g_ev_begin = g_ev_end = nullptr;
  if (eb && (e = hipEventRecord(eb, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (dtype == CALIBATT_BF16) {
    const int64_t total = (int64_t)nh * nb;
    const int64_t cap = (int64_t)CALIBATT_NOALLOC_SCRATCH_BYTES / per_item;
    for (int64_t i0 = 0; i0 < total; i0 += cap) {
      p.item0 = i0;
      if ((e = calibatt::launch_energy_onepass_items(p, d, B, std::min(cap, total - i0), s)) != hipSuccess)
        return hip_fail(e, "block energy kernel launch");
    }
  } else if ((e = calibatt::launch_energy(p, d, B, s)) != hipSuccess) {
    return hip_fail(e, "block energy kernel launch");
  }
  if (ee && (e = hipEventRecord(ee, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  return ok();
}

calibatt_status_t calibatt_select_blocks(const float* energy, int64_t rows, int32_t nb, float tau, uint8_t* mask,
                                         int32_t* counts, void* stream) {
  if (!energy) return fail(CALIBATT_ERR_INVALID_ARG, "energy is NULL");
  if (!mask && !counts) return fail(CALIBATT_ERR_INVALID_ARG, "mask and counts are both NULL");
  if (rows < 0) return fail(CALIBATT_ERR_INVALID_ARG, "rows must be >= 0");
  if (nb < 1 || nb > CALIBATT_MAX_NB) return fail(CALIBATT_ERR_INVALID_ARG, "nb must be in [1, %d]", CALIBATT_MAX_NB);
  if (!std::isfinite(tau) || tau < 0.0f || tau > 1.0f) return fail(CALIBATT_ERR_INVALID_ARG, "tau must be in [0, 1]");
  // threshold in 2^-48 units, exact: tau * 2^48 is exact in double
  const unsigned long long need = (unsigned long long)std::ceil((double)tau * 281474976710656.0);
  hipError_t e = calibatt::launch_select(energy, rows, nb, need, mask, counts, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "selection kernel launch");
  return ok();
}

calibatt_status_t calibatt_keep_frequency(const int32_t* counts, int64_t n, int32_t n_prompts, float rho,
                                          uint8_t* mask, void* stream) {
  if (!counts || !mask) return fail(CALIBATT_ERR_INVALID_ARG, "counts and mask must be non-NULL");
  if (n < 0) return fail(CALIBATT_ERR_INVALID_ARG, "n must be >= 0");
  if (n_prompts < 1) return fail(CALIBATT_ERR_INVALID_ARG, "n_prompts must be >= 1");
  if (!std::isfinite(rho) || rho < 0.0f || rho > 1.0f) return fail(CALIBATT_ERR_INVALID_ARG, "rho must be in [0, 1]");
  // count / |D| >= rho  <=>  count >= rho * |D| (exact product in double)  <=>  count >= ceil(rho * |D|)
  const int32_t k_min = (int32_t)std::ceil((double)rho * (double)n_prompts);
  hipError_t e = calibatt::launch_keep(counts, n, k_min, mask, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "keep-frequency kernel launch");
  return ok();
}

calibatt_status_t calibatt_spatial_similarity(const void* q, const void* k, int32_t H, int32_t N, int32_t d,
                                              calibatt_dtype_t dtype, float scale, int32_t F, int32_t R, int32_t C,
                                              const int32_t* anchor_rows, int32_t k_anchors, float* row_sim,
                                              const int32_t* heads, int32_t n_heads, void* stream) {
  calibatt_status_t st = check_tensors(q, k, q, row_sim, H, N, d, dtype, scale);
  if (st != CALIBATT_OK) return st;
  if ((st = check_anchors(N, F, R, C, anchor_rows, k_anchors)) != CALIBATT_OK) return st;
  if (k_anchors >= R) return fail(CALIBATT_ERR_INVALID_ARG, "every row is an anchor row (k = R): nothing to compare");
  std::vector<int32_t> hs;
  if ((st = check_heads(heads, n_heads, H, hs)) != CALIBATT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  calibatt::SimParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.row_sim = row_sim;
  p.head_stride = (int64_t)N * d;
  p.N = N;
  p.F = F;
  p.R = R;
  p.C = C;
  p.ka = k_anchors;
  for (int32_t i = 0; i < k_anchors; ++i) p.anchors[i] = anchor_rows[i];
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.n_heads = (int32_t)hs.size();
  for (size_t i = 0; i < hs.size(); ++i) p.heads[i] = hs[i];
  hipEvent_t eb = g_ev_begin, ee = g_ev_end;
  g_ev_begin = g_ev_end = nullptr;
  hipError_t err;
  if (eb && (err = hipEventRecord(eb, s)) != hipSuccess) return hip_fail(err, "hipEventRecord");
  if ((err = calibatt::launch_similarity(p, d, dtype == CALIBATT_F32, s)) != hipSuccess)
    return hip_fail(err, "similarity kernel launch");
  if (ee && (err = hipEventRecord(ee, s)) != hipSuccess) return hip_fail(err, "hipEventRecord");
  return ok();
}

calibatt_status_t calibatt_repetition_flags(const float* row_sim, int32_t n_prompts, int32_t H, int32_t F, int32_t R,
                                            const int32_t* anchor_rows, int32_t k_anchors, float threshold,
                                            uint8_t* flags, float* mean, void* stream) {
  if (!row_sim) return fail(CALIBATT_ERR_INVALID_ARG, "row_sim is NULL");
  if (!flags && !mean) return fail(CALIBATT_ERR_INVALID_ARG, "flags and mean are both NULL");
  if (n_prompts < 1 || H < 1 || F < 1 || R < 1)
    return fail(CALIBATT_ERR_INVALID_ARG, "n_prompts, H, F and R must be >= 1");
  if (!anchor_rows) return fail(CALIBATT_ERR_INVALID_ARG, "anchor_rows is NULL");
  if (k_anchors < 1 || k_anchors >= R || k_anchors > CALIBATT_MAX_ANCHORS)
    return fail(CALIBATT_ERR_INVALID_ARG, "anchor count %d must be in [1, min(R - 1, %d)]", k_anchors,
                CALIBATT_MAX_ANCHORS);
  for (int32_t i = 0; i < k_anchors; ++i) {
    if (anchor_rows[i] < 0 || anchor_rows[i] >= R)
      return fail(CALIBATT_ERR_INVALID_ARG, "anchor row %d outside [0, %d)", anchor_rows[i], R);
    if (i > 0 && anchor_rows[i] <= anchor_rows[i - 1])
      return fail(CALIBATT_ERR_INVALID_ARG, "anchor rows must be strictly ascending");
  }
  if (!std::isfinite(threshold)) return fail(CALIBATT_ERR_INVALID_ARG, "threshold must be finite");
  calibatt::RepFlagParams q;
  std::memset(&q, 0, sizeof(q));
  for (int32_t i = 0; i < k_anchors; ++i) q.anchors[i] = anchor_rows[i];
  q.ka = k_anchors;
  q.threshold = threshold;
  hipError_t e = calibatt::launch_rep_flags(row_sim, n_prompts, H, F, R, q, flags, mean, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "repetition-flag kernel launch");
  return ok();
}

}  // extern "C"
