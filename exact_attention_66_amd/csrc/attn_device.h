// Device-side building blocks shared by the forward and backward kernels:
// 16-bit element traits, gfx950 MFMA wrappers, LDS transpose reads and
// cross-half wavefront exchange.
//
// MFMA operand layouts used throughout (wave64; h = lane / 32, r = lane % 32),
// checked on gfx950 with an in-bounds lane probe:
//   v_mfma_f32_32x32x16_{bf16,f16}:  D[32x32] += A[32x16] * B[16x32]
//     A: lane holds A[r][8h + i],  i = 0..7
//     B: lane holds B[8h + i][r],  i = 0..7
//     D: lane holds D[8*(j/4) + 4h + j%4][r],  j = 0..15
// Because the reduction index enters A and B the same way, any fixed
// relabelling of the 16 reduction slots is harmless as long as both operands
// use it; the kernels relabel keys so that a score accumulator can be fed
// back as an operand without moving data (see slot_key()).
//
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane j supplies
// the address of 4 consecutive 16-bit elements; lanes 4s..4s+3 together form
// row s (lane 4s+t gives columns 4t..4t+3) of a 4x16 block, and lane i
// receives column i of that block (4 elements, one per row).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace attn {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define ATTN_LDS __attribute__((address_space(3)))

struct bf16_t {
  typedef __bf16 T;
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  typedef __bf16 v4 __attribute__((ext_vector_type(4)));
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 mfma32(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ v4 tr_read(const T* lds_ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS v4*)(lds_ptr));
  }
  static __device__ __forceinline__ float dot2(v2 a, v2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
  }
};

struct f16_t {
  typedef _Float16 T;
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  typedef _Float16 v4 __attribute__((ext_vector_type(4)));
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 mfma32(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  typedef __fp16 raw4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
  static __device__ __forceinline__ v4 tr_read(const T* lds_ptr) {
    return __builtin_bit_cast(v4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((ATTN_LDS raw4*)(lds_ptr)));
  }
  static __device__ __forceinline__ float dot2(v2 a, v2 b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }
};

// Row of a 32x32 accumulator held in slot j by a lane of half h.
__device__ __forceinline__ constexpr int acc_row(int j, int h) { return 8 * (j / 4) + 4 * h + (j % 4); }

// Reduction slot relabelling: slot i (0..7) of a lane in half h inside one
// 16-wide reduction step carries key/row 8*(i/4) + 4h + i%4 of that step.
// This is exactly the set of rows a 32x32 accumulator keeps in slots
// 8*kk + i, so accumulator slots 8kk..8kk+7 form the B (or A) operand of
// reduction step kk with no data movement.
__device__ __forceinline__ constexpr int slot_key(int i, int h) { return 8 * (i / 4) + 4 * h + (i % 4); }

// Swizzled LDS tile of 16-bit elements, ROWLEN (32, 64 or 128) elements per row
// and no padding: the 16-byte chunk c of row r is stored at chunk c ^ f(r).
// f is chosen so that, with 64 four-byte banks, both access patterns the
// kernels use are free of bank conflicts:
//  * ds_read_b128 by 16 lanes of 16 consecutive rows at the same chunk:
//    f is one-to-one on any 16 consecutive rows;
//  * ds_read_b64_tr_b16 by 32 lanes of 4 consecutive rows (4-aligned) x 64
//    contiguous bytes (4 chunks 4m..4m+3): the rows' f differ in bits 2..3
//    (ROWLEN 128), or in bit 2 for rows of the same parity (ROWLEN 64, where
//    two rows share one 256-byte bank cycle), so the 16 (row, chunk) pairs
//    land on 16 distinct groups of 4 banks.
// ROWLEN 32 (four rows per bank cycle): f = (row >> 2) & 3 separates the 16
// consecutive rows of a b128 read; a transpose read covers 4 whole rows.
template <int ROWLEN>
__device__ __forceinline__ int swz(int row, int col) {
  static_assert(ROWLEN == 32 || ROWLEN == 64 || ROWLEN == 128, "row length");
  const int f = ROWLEN == 128  ? (4 * (row & 3) + ((row >> 2) & 3))
                : ROWLEN == 64 ? (4 * ((row >> 1) & 1) + ((row >> 2) & 3))
                               : ((row >> 2) & 3);
  return row * ROWLEN + (((col >> 3) ^ f) << 3) + (col & 7);
}

// Maximum of two / three floats with NaN propagation (IEEE maximum, gfx950
// v_maximum3_f32).  Unlike fmaxf it needs no quieting of its inputs, which
// would cost one extra instruction per MFMA result read.
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float fmax3(float a, float b, float c) { return fmax2(fmax2(a, b), c); }

// max / sum of a value across the two 32-lane halves (lane l and l ^ 32).
__device__ __forceinline__ float xhalf_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax2(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Ask the register allocator to keep an MFMA A/B operand in AGPRs (LDS reads
// can write AGPRs and MFMAs can read them).  A non-volatile asm statement is
// only a data dependence: it orders nothing else and forces no earlier wait
// than the MFMA that uses the operand.
template <typename V>
__device__ __forceinline__ void in_agpr(V& x) {
  asm("" : "+a"(x));
}

// Four f32x4 (accumulator rows 4jg .. 4jg+3) as one MFMA accumulator.
__device__ __forceinline__ f32x16 join16(const f32x4 (&x)[4]) {
  f32x16 r;
#pragma unroll
  for (int jg = 0; jg < 4; ++jg)
#pragma unroll
    for (int u = 0; u < 4; ++u) r[4 * jg + u] = x[jg][u];
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait for every outstanding vector-memory load of this wave (vmcnt = 0,
// other counters untouched).  Placed after loads issued before a main loop:
// otherwise the compiler may leave them in flight into the loop, and since
// the counter is in-order, its waits for them inside the loop end up waiting
// for the loop's own prefetches as well.
__device__ __forceinline__ void wait_all_vmem_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Pin a loaded value in registers at this point of the program: the (empty)
// volatile asm reads it, so the load must have completed here and cannot be
// sunk past later barriers into a loop.
template <typename V>
__device__ __forceinline__ void materialize(const V& x) { asm volatile("" : : "v"(x)); }

// An integer the compiler cannot see through (so it keeps the register
// instead of recomputing the expression inside a loop).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Wait out the latency of the MFMAs just issued, placed at the end of every
// tile iteration, before the barrier.  The compiler may put register copies
// of MFMA accumulators right after that barrier (loop header or epilogue)
// without counting the barrier as wait states; a barrier that releases at
// once would then let a copy read an accumulator before its MFMA has written
// it (seen as a wrong last element of dK with a single query tile).
// 32 cycles covers the 8-pass 32x32 MFMA.
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Scheduling fence: the compiler may not move any instruction across it.
// Used to keep a block of LDS reads ahead of the MFMAs that consume them, so
// that all reads are in flight at once instead of one pair at a time.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
enum : int {
  kSchedValu = 0x002 | 0x400,  // vector ALU, transcendental included
  kSchedMfma = 0x008,
  kSchedDsRead = 0x100,
};

// Ask the scheduler for REP repetitions of the group sequence
// (N1 of class M1, N2 of class M2, N3 of class M3) in the current scheduling
// region, e.g. one MFMA, then two LDS reads, then four VALU, 16 times over.
template <int REP, int M1, int N1, int M2 = 0, int N2 = 0, int M3 = 0, int N3 = 0>
__device__ __forceinline__ void sched_interleave() {
  if constexpr (REP > 0) {
    __builtin_amdgcn_sched_group_barrier(M1, N1, 0);
    if constexpr (N2 > 0) __builtin_amdgcn_sched_group_barrier(M2, N2, 0);
    if constexpr (N3 > 0) __builtin_amdgcn_sched_group_barrier(M3, N3, 0);
    sched_interleave<REP - 1, M1, N1, M2, N2, M3, N3>();
  }
}

// Direct global -> LDS copy (gfx950 global_load_lds_dwordx4 / _dword): lane
// l's 16 (4) bytes from gbase + voff (its own byte offset) land at
// lds_base + 16 l (4 l); gbase and lds_base are the same for the whole wave
// (scalar registers).  Completion is counted by vmcnt like an ordinary load.
// Issued as inline asm so that the compiler does not track the LDS write
// itself: its wait insertion cannot tell a copy into one buffer from reads
// of the other and would wait for every copy right after issuing it.  The
// kernels wait for their copies explicitly (wait_all_vmem_loads) before the
// barrier that publishes a buffer.  No other code in these kernels uses m0.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((ATTN_LDS const void*)p);
}
__device__ __forceinline__ void lds_copy16(const void* gbase, uint32_t voff, const void* lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_address(lds_base)), "v"(voff), "s"(gbase)
               : "memory");
}
__device__ __forceinline__ void lds_copy4(const void* gbase, uint32_t voff, const void* lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds_address(lds_base)), "v"(voff), "s"(gbase)
               : "memory");
}

// Workgroup order for kernels whose workgroups of one (batch, head) read the
// same tiles of that head: the dispatcher deals consecutive workgroup
// indices to the 8 XCDs in turn (index b runs on XCD b % 8, each XCD with
// its own L2), so index b is mapped to a head-major position L such that
// each XCD works through one contiguous range of L: the blocks of one head
// then share one L2 and run at about the same time, and the heads in flight
// at any moment are few (their tiles fit in the caches) instead of all.
// T is the grid size; returns (head, block) with block in [0, nblk).
__device__ __forceinline__ void xcd_head_major(int b, int T, int nblk, int& bh, int& blk) {
  constexpr int X = 8;
  const int x = b % X, p = b / X;
  const int C = T / X, rem = T % X;  // XCD x receives C + (x < rem) workgroups
  const int L = x * C + min(x, rem) + p;
  bh = L / nblk;
  blk = L % nblk;
}

// The wave index as a wave-uniform (scalar) value, so that branches on it
// are scalar branches.
// Work split of a persistent grid of G workgroups (G a multiple of 8) over
// T units listed heaviest first within each head: the units are dealt to the
// 8 XCDs in contiguous ranges (the same split as xcd_head_major, so the units
// of one head stay on one XCD and share its L2), and within an XCD the P =
// G / 8 workgroups take them in rounds of P, alternately front to back and
// back to front, so every workgroup gets about the same amount of work.
// Returns the unit of round k for workgroup b, or -1 when it has no more.
__device__ __forceinline__ int xcd_snake_unit(int b, int G, int T, int k) {
  constexpr int X = 8;
  const int x = b % X, p = b / X, P = G / X;
  const int C = T / X, rem = T % X;
  const int base = x * C + min(x, rem), cnt = C + (x < rem ? 1 : 0);
  const int i = P * k + ((k & 1) ? P - 1 - p : p);
  return i < cnt ? base + i : -1;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// 8 fp32 -> 8 16-bit values (round to nearest even) packed as an MFMA operand.
template <typename E>
__device__ __forceinline__ typename E::v8 pack8(float a0, float a1, float a2, float a3,
                                                float a4, float a5, float a6, float a7) {
  typename E::v8 r;
  r[0] = (typename E::T)a0; r[1] = (typename E::T)a1; r[2] = (typename E::T)a2; r[3] = (typename E::T)a3;
  r[4] = (typename E::T)a4; r[5] = (typename E::T)a5; r[6] = (typename E::T)a6; r[7] = (typename E::T)a7;
  return r;
}

// acc + sum of the 8 packed 16-bit values (exact products by 1.0, fp32 sums).
template <typename E>
__device__ __forceinline__ float sum8(typename E::v8 x, float acc) {
  const typename E::v2 one = {(typename E::T)1.0f, (typename E::T)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const typename E::v2 pr = {x[2 * i], x[2 * i + 1]};
    acc = E::dot2(pr, one, acc);
  }
  return acc;
}

template <typename E>
__device__ __forceinline__ typename E::v8 concat44(typename E::v4 lo, typename E::v4 hi) {
  typename E::v8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

}  // namespace attn
