// Swizzled LDS tiles filled by direct global-to-LDS loads, and the MFMA operand reads from them
// (gfx950). Shared by the kernels whose tiles are read both as rows and transposed: the backward
// kernels and the forward kernel for the score variants and d = 256.
//
// LDS layout of a tile: unpadded rows of 2d bytes; the 16-byte chunk j of row r is stored at chunk
// position j ^ f(r). A row read gives each lane 16 bytes of one row (16 consecutive rows per group
// of 16 lanes); a transposing read (ds_read_b64_tr_b16) gives each lane 8 bytes of one of 4
// consecutive rows, 64 bytes per row, per group of 32 lanes. No padding serves both; the swizzle f
// is chosen so that both, and the DMA writes, touch every bank equally often.
#pragma once

#include "fa_device.h"

namespace fa {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// Swizzled tile geometry for head dim D (see the header comment).
template <int D>
struct Swz {
  static constexpr int ROW = 2 * D;  // bytes per row
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  template <int ROWS>
  static constexpr int bytes() { return ROWS * ROW; }
  // The LDS serves a 16-byte row read 16 lanes at a time (16 consecutive rows, one chunk each)
  // and a transposing 8-byte read 32 lanes at a time (4 consecutive rows x 4 chunks of one
  // 4-chunk group). d = 128 (16 chunks per 256-byte row): f must be injective on 16 consecutive
  // rows, and 4 consecutive rows must move a chunk group to 4 different groups (f / 4 distinct):
  // f(r) = 4 (r mod 4) + (r / 4) mod 4. d = 64 (8 chunks, two rows per 256 bytes): rows of equal
  // parity share banks, so f must be injective on the 8 rows of one parity among 16, and rows r,
  // r+2 must use different halves (bit 2 of f): f(r) = 4 ((r / 2) mod 2) + (r / 4) mod 4. Both
  // also keep the staging writes (whole rows) conflict-free. d = 256 (32 chunks, a row spans two
  // 256-byte bank lines) uses the d = 128 rule: it permutes chunk bits 0-3 only.
  __device__ static __forceinline__ int f(int r) {
    if constexpr (D >= 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  __device__ static __forceinline__ int off(int r, int j) { return r * ROW + 16 * (j ^ f(r)); }
};

typedef int i32x4v __attribute__((ext_vector_type(4)));

// Buffer resource (as four scalar registers, for the DMA instruction) over rows row0 .. N-1 of one
// head, rows rs bytes apart, ending after row min(N, row0 + ROWS) - 1: bytes past it read as
// zeros.
template <int D, int ROWS>
__device__ __forceinline__ i32x4v tile_rsrc(const char* head, long long rs, int row0, int N) {
  const int rows = min(N - row0, ROWS);  // >= 1: only tiles that start below N are loaded
  const unsigned long long base = reinterpret_cast<unsigned long long>(head + (long long)row0 * rs);
  i32x4v r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(base & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane((int)(base >> 32));
  r[2] = __builtin_amdgcn_readfirstlane((int)((rows - 1) * rs) + 2 * D);
  r[3] = 0x00020000;
  return r;
}

// Global memory -> LDS without registers: one 16-byte buffer load per lane (voff + soff bytes into
// the resource) whose data the hardware writes at (piece + 16 * lane), 1 KB per wave instruction.
// dma_piece: piece p of a tile (rows 4p..4p+3 of the
// swizzled tile for d = 128, 8p..8p+7 for d = 64, at LDS offset 1 KB * p). Lane l fills tile
// position (row, slot) = (RPP p + l / CPR, l % CPR), so it fetches chunk slot ^ f(row) of that
// row. The load counts on vmcnt; the caller waits for it before the barrier that publishes the
// tile. (The DMA form is written as inline assembly: the compiler would otherwise wait for it
// before every LDS access.)
__device__ __forceinline__ void dma16(char* piece, unsigned voff, const i32x4v& rsrc,
                                      unsigned soff) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((int)(unsigned)(size_t)(FA_LDS char*)piece);
  // s_nop 1: a VMEM instruction must not read an SGPR within two wait states of a VALU write to
  // it (v_readfirstlane of the offsets), and the compiler's hazard recognizer does not look
  // inside inline assembly; two wait states plus the s_mov cover it whatever precedes the block.
  asm volatile("s_nop 1\n\ts_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m0), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

template <int D>
__device__ __forceinline__ void dma_piece(char* tile, const i32x4v& rsrc, long long rs, int p,
                                          int lane) {
  constexpr int CPR = Swz<D>::CPR, RPP = 1024 / (2 * D);
  const int rin = lane / CPR, slot = lane % CPR;
  const unsigned voff = (unsigned)(rin * rs) + 16u * (unsigned)(slot ^ Swz<D>::f(RPP * p + rin));
  const unsigned soff = __builtin_amdgcn_readfirstlane((int)(RPP * p * rs));
  dma16(tile + 1024 * p, voff, rsrc, soff);
}

// The ROWS-row tile of rows row0.. by W waves (tile bytes / 1 KB pieces, spread over the waves).
template <int D, int ROWS, int W>
__device__ __forceinline__ void dma_tile(char* tile, const char* head, long long rs, int row0,
                                         int N, int wave, int lane) {
  constexpr int PIECES = Swz<D>::template bytes<ROWS>() / 1024;
  static_assert(PIECES % W == 0, "pieces must divide over the waves");
  const i32x4v r = tile_rsrc<D, ROWS>(head, rs, row0, N);
#pragma unroll
  for (int i = 0; i < PIECES / W; i++) dma_piece<D>(tile, r, rs, wave + W * i, lane);
}

// The waits are the compiler's own s_waitcnt (not inline assembly), so that its wait insertion
// knows the counter has drained: otherwise a load it issued before the loop (the Q operand)
// stays pending in its books and it waits for vmcnt(0) -- including the DMA just issued for the
// next tile -- at the first use inside the loop, on every iteration. The immediate holds vmcnt
// in bits 3:0 and 15:14, expcnt in 6:4 and lgkmcnt in 11:8 (the last two left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_dma() { wait_vmcnt<0>(); }
// Race-check build: the loads just issued land before any wave of the work-group goes on.
__device__ __forceinline__ void race_check_drain() {
  if constexpr (FA_RACE_CHECK != 0) {
    wait_dma();
    __syncthreads();
  }
}
// Wait for all but the N most recently issued loads (loads complete in issue order for vmcnt).
template <int N>
__device__ __forceinline__ void wait_dma_but() { wait_vmcnt<N>(); }

// Row operand: 8 consecutive elements (chunk 2 dk + h) of tile row r.
template <int D>
__device__ __forceinline__ bf16x8 tile_row(const char* tile, int r, int dk, int h) {
  return lds_read_b128(tile + Swz<D>::off(r, 2 * dk + h));
}

// Transposed operand of one 16-row k-step: for lane (c, h) the 8 values of column 32 db + c from
// rows r0 + {4h..4h+3, 8+4h..8+4h+3}, the row order of one k-step of the 32x32 accumulator.
template <int D>
__device__ __forceinline__ bf16x8 tile_tr(const char* tile, int r0, int db, int lane) {
  const int Lg = lane & 15, h = lane >> 5, hi = (lane >> 4) & 1;
  const int col = 64 * db + 32 * hi + 8 * (Lg & 3);  // byte column
  const int ra = r0 + 4 * h + (Lg >> 2), rb = ra + 8;
  const bf16x4 x = lds_read_tr16(tile + Swz<D>::off(ra, col >> 4) + (col & 15));
  const bf16x4 y = lds_read_tr16(tile + Swz<D>::off(rb, col >> 4) + (col & 15));
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Per-lane byte offsets of those reads, computed once. The swizzle depends on the row only
// through r mod 16, so a read at row offset 16 k (k a compile-time step index) is the lane's
// offset plus the immediate 16 k * ROW: no address arithmetic in the loops. It permutes only the
// low 4 bits of the chunk index, so the chunks of columns 128.. of a d = 256 row sit 256 bytes
// past those of columns 0..127: offsets are kept for the first 128 columns only.
template <int D>
struct LaneOffsets {
  static constexpr int DH = D > 128 ? 128 : D;
  int row[DH / 16];     // row c, chunk 2 dk + h
  int tr[DH / 32][2];   // transposing reads of rows 4h + L/4 (and + 8) of a 16-row k-step, block db
  __device__ __forceinline__ void init(int lane) {
    const int c = lane & 31, h = lane >> 5, Lg = lane & 15, hi = (lane >> 4) & 1;
#pragma unroll
    for (int dk = 0; dk < DH / 16; dk++) row[dk] = Swz<D>::off(c, 2 * dk + h);
#pragma unroll
    for (int db = 0; db < DH / 32; db++) {
      const int col = 64 * db + 32 * hi + 8 * (Lg & 3);
      const int ra = 4 * h + (Lg >> 2);
      tr[db][0] = Swz<D>::off(ra, col >> 4) + (col & 15);
      tr[db][1] = Swz<D>::off(ra + 8, col >> 4) + (col & 15);
    }
  }
};

// tile_row / tile_tr with precomputed offsets; r16 (a multiple of 16) is the row offset.
template <int D>
__device__ __forceinline__ bf16x8 tile_row_at(const char* tile, const LaneOffsets<D>& lo, int r16,
                                              int dk) {
  constexpr int NK = LaneOffsets<D>::DH / 16;
  return lds_read_b128(tile + lo.row[dk % NK] + 256 * (dk / NK) + r16 * Swz<D>::ROW);
}
template <int D>
__device__ __forceinline__ bf16x8 tile_tr_at(const char* tile, const LaneOffsets<D>& lo, int r16,
                                             int db) {
  constexpr int NB = LaneOffsets<D>::DH / 32;
  const int o = 256 * (db / NB) + r16 * Swz<D>::ROW;
  const bf16x4 x = lds_read_tr16(tile + lo.tr[db % NB][0] + o);
  const bf16x4 y = lds_read_tr16(tile + lo.tr[db % NB][1] + o);
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Row index (within a 32-row step) of accumulator register i of lane half h.
__device__ __forceinline__ constexpr int acc_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

}  // namespace fa
