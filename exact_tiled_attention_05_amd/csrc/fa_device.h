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

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------------------------
// LDS tile layout. A K or V tile is [rows][D] bf16, row-major, one row per key. Each row is cut
// into 16-byte chunks (8 elements); the chunk with logical index c of row r is stored at
// physical position c ^ swz(r). The XOR pattern is chosen so that both read patterns of the
// kernel touch 16 distinct 16-byte bank groups per 256 bytes:
//   * K reads (MFMA A operand): 16 consecutive rows at one logical chunk;
//   * V reads (transposing reads): 4 consecutive rows x 4 consecutive chunks.
// For D = 128 (16 chunks per 256-byte row) swz rotates the low 4 row bits by two; for D = 64
// (8 chunks, two rows per 256 bytes) it uses row bits 1..3.
// ---------------------------------------------------------------------------------------------
template <int D>
__device__ __host__ constexpr int swz(int row) {
  static_assert(D == 64 || D == 128, "head dim");
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
}

// Byte offset inside a tile of element (row, col), col a multiple of 4 (8-byte aligned).
template <int D>
__device__ __host__ constexpr int tile_off(int row, int col) {
  return row * (D * 2) + ((((col >> 3) ^ swz<D>(row))) << 4) + ((col & 7) << 1);
}

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

// Direct global -> LDS copy of 16 bytes per lane. `lds` must be the same for the whole wave;
// lane L's 16 bytes land at lds + 16 * L.
__device__ inline void global_to_lds16(const void* g, char* lds) {
  __builtin_amdgcn_global_load_lds(g, (FA_LDS void*)(lds), 16, 0, 0);
}

__device__ inline void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Workgroup barrier without a memory fence. Used where each wave has already waited for its own
// direct-to-LDS loads (vmcnt) and every LDS read of the buffer about to be refilled has been
// consumed: the barrier then only has to order the waves.
__device__ inline void barrier_only() { __builtin_amdgcn_s_barrier(); }

// Wait until at most N vector-memory operations of this wave are outstanding (they complete in
// issue order, so everything issued before the last N is done).
template <int N>
__device__ inline void wait_vmem_until() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
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

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------------------------
// Workgroup -> (batch*head, query block). One workgroup owns one query block of one head for its
// whole life ("FlashAttention-2 -- Deeper Math", Fixes 3-4). The hardware hands workgroups to
// the 8 XCDs round-robin by id; when the grid divides by 8 the id is renumbered so that each
// XCD receives a contiguous range of logical ids, and the logical order keeps the workgroups of
// one head together on one XCD (sharing K/V in that XCD's L2). With a causal mask the heaviest
// query blocks (the last ones, which see the most keys) are dispatched first.
// ---------------------------------------------------------------------------------------------
template <bool CAUSAL>
__device__ inline void map_block(int bid, int nblk, int BH, int n_qblk, int& bh, int& qblk) {
  if ((nblk & 7) == 0 && (BH & 7) == 0) {
    const int per_xcd = nblk >> 3;
    const int x = bid & 7;
    const int s = bid >> 3;  // position in this XCD's dispatch order
    const int hpx = BH >> 3; // heads per XCD
    if (CAUSAL) {
      bh = x * hpx + s % hpx;
      qblk = n_qblk - 1 - s / hpx;
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
