// Host entry points of libcalibatt.so (declared in include/calibatt.h).
//
// Every argument is checked here, before anything is enqueued; the kernels
// assume what these checks establish (sizes, supported d and block sizes,
// head and anchor ranges). The only synchronisation in the library is the
// read-back of the kept-block count in calibatt_compile_skiplist.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "internal.h"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_ev_begin = nullptr;
thread_local hipEvent_t g_ev_end = nullptr;

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

calibatt_status_t check_skiplist(const calibatt_skiplist_t* sl, int32_t H, int32_t N, int32_t t, int32_t l) {
  if (!sl) return fail(CALIBATT_ERR_INVALID_ARG, "skip list view is NULL");
  if (!sl->row_ptr || !sl->col_idx) return fail(CALIBATT_ERR_INVALID_ARG, "skip list row_ptr/col_idx are NULL");
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
  // runs of 32 consecutive items per XCD; heaviest-first order per record
  // (the compiled `order`) measured no faster on the Wan-shaped layers.
  p.use_order = 0;
  p.xcd_group = 32;
}

void fill_sparse(calibatt::AttnParams& p, const calibatt_skiplist_t* sl, int32_t t, int32_t l,
                 const std::vector<int32_t>& heads) {
  p.row_ptr = sl->row_ptr;
  p.col_idx = sl->col_idx;
  p.order = sl->order;
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

}  // namespace

extern "C" {

const char* calibatt_last_error(void) { return g_err; }

int32_t calibatt_version(void) { return 100; }

void calibatt_set_kernel_events(void* begin, void* end) {
  g_ev_begin = static_cast<hipEvent_t>(begin);
  g_ev_end = static_cast<hipEvent_t>(end);
}

calibatt_status_t calibatt_compile_skiplist(const uint8_t* masks, int32_t T, int32_t L, int32_t H, int32_t N,
                                            int32_t B, int64_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                            int32_t* order, int64_t* nnz_out, void* stream) {
  if (!masks || !row_ptr || !nnz_out) return fail(CALIBATT_ERR_INVALID_ARG, "masks, row_ptr and nnz_out must be non-NULL");
  if (T < 1 || L < 1 || H < 1 || N < 1 || B < 1)
    return fail(CALIBATT_ERR_INVALID_ARG, "T, L, H, N and B must be >= 1");
  const int64_t nb = ceil_div(N, B);
  if (nb > CALIBATT_MAX_NB) return fail(CALIBATT_ERR_INVALID_ARG, "nb = %lld exceeds %d", (long long)nb, CALIBATT_MAX_NB);
  if (col_idx && col_capacity < 0) return fail(CALIBATT_ERR_INVALID_ARG, "col_capacity must be >= 0");
  const int64_t records = (int64_t)T * L * H;
  const int64_t rows = records * nb;
  hipStream_t s = static_cast<hipStream_t>(stream);

  hipError_t e = calibatt::launch_compile_count_scan(masks, rows, (int)nb, row_ptr, s);
  if (e != hipSuccess) return hip_fail(e, "skip-list count kernel launch");
  int64_t nnz = 0;
  e = hipMemcpyAsync(&nnz, row_ptr + rows, sizeof(int64_t), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "reading the kept-block count");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "synchronising after the count pass");
  *nnz_out = nnz;
  if (!col_idx) return ok();
  if (col_capacity < nnz)
    return fail(CALIBATT_ERR_CAPACITY, "col_idx holds %lld entries, %lld needed", (long long)col_capacity,
                (long long)nnz);
  e = calibatt::launch_compile_fill(masks, rows, (int)nb, row_ptr, col_idx, s);
  if (e != hipSuccess) return hip_fail(e, "skip-list fill kernel launch");
  if (order) {
    e = calibatt::launch_compile_order(row_ptr, records, (int)nb, order, s);
    if (e != hipSuccess) return hip_fail(e, "skip-list order kernel launch");
  }
  return ok();
}

calibatt_status_t calibatt_block_sparse_attn(const void* q, const void* k, const void* v, void* o, float* lse,
                                             int32_t H, int32_t N, int32_t d, calibatt_dtype_t dtype, float scale,
                                             const calibatt_skiplist_t* sl, int32_t t, int32_t l,
                                             const int32_t* heads, int32_t n_heads, void* stream) {
  calibatt_status_t st = check_tensors(q, k, v, o, H, N, d, dtype, scale);
  if (st != CALIBATT_OK) return st;
  if ((st = check_skiplist(sl, H, N, t, l)) != CALIBATT_OK) return st;
  std::vector<int32_t> hs;
  if ((st = check_heads(heads, n_heads, H, hs)) != CALIBATT_OK) return st;
  calibatt::AttnParams p;
  fill_common(p, q, k, v, o, lse, N, d, sl->B, scale);
  fill_sparse(p, sl, t, l, hs);
  if ((st = run_attention(p, d, sl->B, dtype, static_cast<hipStream_t>(stream))) != CALIBATT_OK) return st;
  return ok();
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
  if ((st = check_skiplist(sl, H, N, t, l)) != CALIBATT_OK) return st;
  if (!rep_flags) return fail(CALIBATT_ERR_INVALID_ARG, "rep_flags is NULL");
  if (H > CALIBATT_MAX_HEADS) return fail(CALIBATT_ERR_INVALID_ARG, "at most %d heads", CALIBATT_MAX_HEADS);
  // Record selection: the flags of (t, l) split the heads into the two paths.
  std::vector<int32_t> sparse_heads, rep_heads;
  const uint8_t* fl = rep_flags + ((int64_t)t * sl->L + l) * sl->H;
  for (int32_t h = 0; h < H; ++h) (fl[h] ? rep_heads : sparse_heads).push_back(h);
  if (!rep_heads.empty() && (st = check_anchors(N, F, R, C, anchor_rows, k_anchors)) != CALIBATT_OK) return st;
  // One launch covers both paths: anchor tiles (every key block) first, then
  // the block-sparse query blocks, heaviest first within each head.
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

}  // extern "C"
