// Anchor-output broadcast: each spatial row of a frame receives the output of
// its nearest anchor row in the same frame, column by column (papernotes.org
// notes on "Accelerating Text-to-Video Generation with Calibrated Sparse
// Attention", Key Design 3). Nearest means minimal |r - a|; on a tie the
// smaller anchor row wins.
//
// One workgroup copies one (head, frame, row): C*d contiguous elements, read
// from the anchor row and written with 16-byte vector accesses by consecutive
// lanes, so both sides are fully coalesced; each lane issues kUnroll loads
// before its stores. lse (C floats) is copied alongside. Workgroups are
// dispatched round-robin over the 8 XCDs, so grid blocks map to rows such
// that the R rows of one frame run on one XCD: the frame's anchor rows are
// then fetched into that XCD's L2 once instead of by every XCD.
#include "gfx950_device.h"
#include "internal.h"

namespace calibatt {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void broadcast_kernel(const BcastParams p) {
  const int64_t rows = (int64_t)p.F * p.R;
  const int64_t item = dev::xcd_item(blockIdx.x, gridDim.x, p.R);   // head * F*R + frame * R + row
  const int hi = (int)(item / rows);
  const int fr = (int)(item - hi * rows);
  const int f = fr / p.R;
  const int r = fr - f * p.R;
  int a = p.anchors[0];
  for (int i = 1; i < p.ka; ++i) {
    const int cand = p.anchors[i];
    if (abs(r - cand) < abs(r - a)) a = cand;   // anchors ascend: ties keep the smaller
  }
  if (a == r) return;
  const int head = p.heads[hi];
  const int64_t src_tok = (int64_t)(f * p.R + a) * p.C;
  const int64_t dst_tok = (int64_t)(f * p.R + r) * p.C;
  char* base = static_cast<char*>(p.o) + (int64_t)head * p.head_stride * p.esize;
  const int64_t row_bytes = (int64_t)p.d * p.esize;
  // Distinct rows of one head: the two ranges never overlap.
  const u32x4* __restrict__ src = reinterpret_cast<const u32x4*>(base + src_tok * row_bytes);
  u32x4* __restrict__ dst = reinterpret_cast<u32x4*>(base + dst_tok * row_bytes);
  const int64_t n16 = (int64_t)p.C * row_bytes / 16;
  for (int64_t i0 = threadIdx.x; i0 < n16; i0 += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * kThreads;
      if (i < n16) v[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * kThreads;
      if (i < n16) dst[i] = v[u];
    }
  }
  if (p.lse) {
    float* l = p.lse + (int64_t)head * p.N;
    for (int c = threadIdx.x; c < p.C; c += kThreads) l[dst_tok + c] = l[src_tok + c];
  }
}

}  // namespace

hipError_t launch_broadcast(const BcastParams& p, hipStream_t s) {
  if (p.n_heads == 0) return hipSuccess;
  const int64_t blocks = (int64_t)p.F * p.R * p.n_heads;
  hipLaunchKernelGGL(broadcast_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace calibatt
