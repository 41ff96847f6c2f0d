// Device-side helpers shared by the attention forward kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define FA_LDS __attribute__((address_space(3)))

// Race-check build (compiled with -DFA_RACE_CHECK=1). The kernels overlap the loads of the next
// K/V tiles into LDS with the products on the current ones; a missing wait or barrier there would
// let a wave read a tile before it has landed, or let a load overwrite a tile a wave still reads.
// In the race-check build every tile load completes, for every wave of the work-group, before
// any wave goes on (a full wait and a barrier right after the loads are issued, a barrier before a
// staged store), and LDS starts filled with all-ones bytes (NaN as bf16 and as fp32). The
// arithmetic and its order are unchanged, so a race-free fast build gives bit-identical outputs;
// a race shows as a difference, and a read of LDS that no load wrote shows as NaN.
#ifndef FA_RACE_CHECK
#define FA_RACE_CHECK 0
#endif

// Every thread of the work-group fills its share of an LDS array; followed by a barrier.
template <int BYTES>
__device__ __forceinline__ void race_check_poison(void* lds, int tid, int nthreads) {
  if constexpr (FA_RACE_CHECK != 0) {
    static_assert(BYTES % 16 == 0, "LDS arrays are filled 16 bytes at a time");
    typedef unsigned u32x4p __attribute__((ext_vector_type(4)));
    for (int i = 16 * tid; i < BYTES; i += 16 * nthreads)
      *(FA_LDS u32x4p*)((FA_LDS char*)lds + i) = u32x4p{~0u, ~0u, ~0u, ~0u};
  }
}
// A barrier in the race-check build only (called where the whole work-group passes).
__device__ __forceinline__ void race_check_barrier() {
  if constexpr (FA_RACE_CHECK != 0) __syncthreads();
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// LDS pointers are converted with a plain address-space cast (not through an integer) so that the
// compiler keeps track of which LDS array an access touches.
__device__ inline bf16x8 lds_read_b128(const char* p) {
  return *(const FA_LDS bf16x8*)(p);
}

// Transposing LDS read (ds_read_b64_tr_b16). Inside each group of 16 lanes, lane L supplies the
// address of 4 consecutive bf16 of row R0 + L/4 starting at column C0 + 4*(L%4); lane L then
// receives the 4 values of column C0 + L from rows R0..R0+3.
__device__ inline bf16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FA_LDS bf16x4*)(const_cast<char*>(p)));
}

// Value held by the lane 32 positions away (lane l <-> l ^ 32), combined with op.
__device__ inline float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Tree reductions over the 16 values a lane holds for one 32x32 block (short dependency chains).
__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);  // one v_max3_f32
}
__device__ __forceinline__ float max16(const f32x16& v) {
  const float a = max3(v[0], v[1], v[2]), b = max3(v[3], v[4], v[5]);
  const float c = max3(v[6], v[7], v[8]), d = max3(v[9], v[10], v[11]);
  const float e = max3(v[12], v[13], v[14]);
  return max3(max3(a, b, c), max3(d, e, v[15]), -INFINITY);
}
// The same maximum over 16 values held in an array (six v_max3_f32).
__device__ __forceinline__ float max16_arr(const float (&v)[16]) {
  float a = __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), v[2]);
  float b = __builtin_fmaxf(__builtin_fmaxf(v[3], v[4]), v[5]);
  float c = __builtin_fmaxf(__builtin_fmaxf(v[6], v[7]), v[8]);
  float d = __builtin_fmaxf(__builtin_fmaxf(v[9], v[10]), v[11]);
  float e = __builtin_fmaxf(__builtin_fmaxf(v[12], v[13]), v[14]);
  return __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(a, b), c),
                         __builtin_fmaxf(__builtin_fmaxf(d, e), v[15]));
}

__device__ __forceinline__ float sum16(const float (&p)[16]) {
  float t[8];
#pragma unroll
  for (int i = 0; i < 8; i++) t[i] = p[2 * i] + p[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; i++) t[i] = t[2 * i] + t[2 * i + 1];
  return (t[0] + t[1]) + (t[2] + t[3]);
}

// Hand-ordered instruction streams (the kernels with one wave per SIMD): an empty asm that names a
// value emits nothing and, unlike a real use, makes the compiler wait for nothing, but keeps it
// from moving the instruction that produces the value past that point (to its first use); a
// scheduling barrier closes a group of instructions.
__device__ __forceinline__ void pin(const f32x16& x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void pin(const bf16x8& x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void pin(float x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------------------------
// Workgroup -> (batch*head, query block). One workgroup owns one query block of one head for its
// whole life ("FlashAttention-2 -- Deeper Math", Fixes 3-4). The hardware hands workgroups to
// the 8 XCDs round-robin by id; when the grid divides by 8 the id is renumbered so that each
// XCD receives a contiguous range of logical ids, and the logical order keeps the workgroups of
// one head together on one XCD (sharing K/V in that XCD's L2). With a causal mask the heaviest
// query blocks (the last ones, which see the most keys) of a group of heads are dispatched first.
// ---------------------------------------------------------------------------------------------
// Causal grids: an XCD's heads are dispatched in groups of (up to) kCausalGroup, one group after
// another, the heaviest query blocks of the group first. Small groups keep the K/V of few heads
// hot in the XCD's L2; with one head per group the blocks of a single head leave too little to
// balance against. Measured (same box): 4 heads per group against all of an XCD's heads in one
// group: B=1 H=32 N=8192 unchanged (4 heads per XCD either way), B=4 N=8192 +6%, B=16 N=2048
// +12%, B=2 N=16384 +3%, backward B=4 N=4096 +4%.
constexpr int kCausalGroup = 4;
template <bool CAUSAL>
__device__ inline void map_block(int bid, int nblk, int BH, int n_qblk, int& bh, int& qblk) {
  if ((nblk & 7) == 0 && (BH & 7) == 0) {
    const int per_xcd = nblk >> 3;
    const int x = bid & 7;
    const int s = bid >> 3;  // position in this XCD's dispatch order
    const int hpx = BH >> 3; // heads per XCD
    if (CAUSAL) {
      int G = kCausalGroup;  // heads per dispatch group: the largest power of two dividing hpx
      while (hpx % G) G >>= 1;
      const int per_group = G * n_qblk;
      const int gi = s / per_group, p = s - gi * per_group;
      bh = x * hpx + gi * G + p % G;
      qblk = n_qblk - 1 - p / G;
    } else {
      bh = x * hpx + s / n_qblk;
      qblk = s % n_qblk;
    }
    (void)per_xcd;
  } else if (CAUSAL) {
    bh = bid % BH;
    qblk = n_qblk - 1 - bid / BH;
  } else {
    bh = bid / n_qblk;
    qblk = bid % n_qblk;
  }
}

}  // namespace fa
