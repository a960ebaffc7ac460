// Anchor-output broadcast: each spatial row of a frame receives the output of
// its nearest anchor row in the same frame, column by column (papernotes.org
// notes on "Accelerating Text-to-Video Generation with Calibrated Sparse
// Attention", Key Design 3). Nearest means minimal |r - a|; on a tie the
// smaller anchor row wins.
//
// One workgroup copies one (head, frame, row): C*d contiguous elements, read
// from the anchor row and written with 16-byte vector stores by consecutive
// lanes, so both sides are fully coalesced. lse (C floats) is copied alongside.
#include "internal.h"

namespace calibatt {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void broadcast_kernel(const BcastParams p) {
  const int fr = blockIdx.x;                // frame * R + row
  const int f = fr / p.R;
  const int r = fr - f * p.R;
  int a = p.anchors[0];
  for (int i = 1; i < p.ka; ++i) {
    const int cand = p.anchors[i];
    if (abs(r - cand) < abs(r - a)) a = cand;   // anchors ascend: ties keep the smaller
  }
  if (a == r) return;
  const int head = p.heads[blockIdx.y];
  const int64_t src_tok = (int64_t)(f * p.R + a) * p.C;
  const int64_t dst_tok = (int64_t)(f * p.R + r) * p.C;
  char* base = static_cast<char*>(p.o) + (int64_t)head * p.head_stride * p.esize;
  const int64_t row_bytes = (int64_t)p.d * p.esize;
  const uint4* src = reinterpret_cast<const uint4*>(base + src_tok * row_bytes);
  uint4* dst = reinterpret_cast<uint4*>(base + dst_tok * row_bytes);
  const int64_t n16 = (int64_t)p.C * row_bytes / 16;
  for (int64_t i = threadIdx.x; i < n16; i += kThreads) dst[i] = src[i];
  if (p.lse) {
    float* l = p.lse + (int64_t)head * p.N;
    for (int c = threadIdx.x; c < p.C; c += kThreads) l[dst_tok + c] = l[src_tok + c];
  }
}

}  // namespace

hipError_t launch_broadcast(const BcastParams& p, hipStream_t s) {
  if (p.n_heads == 0) return hipSuccess;
  hipLaunchKernelGGL(broadcast_kernel, dim3((unsigned)(p.F * p.R), (unsigned)p.n_heads), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace calibatt
