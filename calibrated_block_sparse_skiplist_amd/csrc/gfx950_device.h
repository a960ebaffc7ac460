// Device helpers shared by the gfx950 MFMA kernels of libcalibatt.so (the
// attention and block-energy kernels): vector types, LDS swizzles, waits and
// barriers that leave the HBM -> LDS copy queue alone, and the copy itself.
#pragma once

#include "internal.h"

namespace calibatt {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 16-byte chunk swizzles of LDS rows of K and V: chunk ch of row `row` is
// stored at ch ^ swz(row). K: the 16 rows of an MFMA operand read hit distinct
// banks; V: the 8-row x 64-byte patch of a transposed read spreads over all banks.
template <int CPR>
__device__ __forceinline__ int swz_k(int row) { return row & (CPR - 1); }
template <int CPR>
__device__ __forceinline__ int swz_v(int row) { return (4 * (row & 3)) & (CPR - 1); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence. __syncthreads() fences, and a
// workgroup fence must drain every outstanding vector-memory operation,
// including the LDS DMA prefetch of the next tile; here each wave instead
// waits for its own DMA with wait_vmcnt before the barrier, and its LDS reads
// have returned (lgkmcnt 0). The memory clobber keeps LDS accesses on their
// side of the barrier.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint4 ld_global16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

template <typename T, typename S>
__device__ __forceinline__ T bitcast(const S& s) {
  static_assert(sizeof(T) == sizeof(S), "size");
  T t;
  __builtin_memcpy(&t, &s, sizeof(T));
  return t;
}

// Logical item of grid block b. Workgroups go round-robin over the 8 XCDs;
// each run of 8*G grid blocks gives XCD x the G consecutive items
// [run*8G + x*G, run*8G + (x+1)*G). The last, partial run keeps grid order.
__device__ __forceinline__ int64_t xcd_item(int64_t b, int64_t total, int G) {
  if (G <= 0) return b;
  const int64_t run = b / (8 * (int64_t)G);
  if ((run + 1) * 8 * (int64_t)G > total) return b;
  const int64_t s = b - run * 8 * (int64_t)G;
  return run * 8 * (int64_t)G + (s % 8) * G + s / 8;
}

// The same for a grid whose first `first` items are all of one size: XCD x
// takes one chunk of first/8 consecutive ones (equal counts, and neighbouring
// items on one L2), the few left over keep grid order, and the runs of 8*G
// blocks are counted from `first`. With `rotate`, run k gives XCD x the G
// items of chunk (x + k) mod 8 instead of chunk x. Where every run covers
// whole heads, chunk x would otherwise hold the same slice of every head on
// the same XCD; slices at the ends of the sequence carry less work, and the
// XCDs would finish at different times.
__device__ __forceinline__ int64_t xcd_item_after(int64_t b, int64_t total, int G, int64_t first, bool rotate) {
  if (b < first) {
    const int64_t per_xcd = first / 8;
    return b < 8 * per_xcd ? (b & 7) * per_xcd + b / 8 : b;
  }
  if (G <= 0) return b;
  const int64_t t = b - first;
  const int64_t run = t / (8 * (int64_t)G);
  if ((run + 1) * 8 * (int64_t)G > total - first) return b;
  const int64_t s = t - run * 8 * (int64_t)G;   // blocks of XCD b % 8 in this run: s / 8 = 0 .. G-1
  const int x = (int)(b & 7);
  const int chunk = rotate ? (int)((x + run) & 7) : x;
  return first + run * 8 * (int64_t)G + (int64_t)chunk * G + s / 8;
}

// One 16-byte HBM -> LDS copy (global_load_lds_dwordx4): lane l's chunk lands
// in slot l of the 64-slot window at `lds` (LDS address = M0 + 16 * lane).
// The source is a uniform base (SGPR pair) plus this lane's 32-bit offset.
//
// Issued as inline assembly on purpose. The compiler does not know which LDS
// bytes the copy writes, so after the builtin form it turns every later LDS
// operand wait into lgkmcnt(0), serialising the MFMA operand reads. The
// hardware counts these copies in vmcnt only; the kernel waits for them
// explicitly (wait_vmcnt) before the barrier that publishes a stage. The
// statement has no register outputs, M0 is set inside it (and declared
// clobbered, so the compiler keeps no value of its own in M0 across it), and
// the memory clobber keeps it after the barrier that frees the destination
// buffer. (clang warns about any clobber of M0, a register it reserves; the
// declaration is what is wanted here.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const char* base, uint32_t off, uint4* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void*)lds;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" :: "s"(m0), "v"(off), "s"(base) : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace dev
}  // namespace calibatt
