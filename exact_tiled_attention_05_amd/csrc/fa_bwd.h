// Attention backward by recomputation, bf16 in / bf16 out, fp32 arithmetic, gfx950.
//
// "Understanding FlashAttention Pt 1", §3.6: the forward pass keeps O and one statistic per row;
// the backward pass rebuilds each tile of P from Q K^T and that statistic -- the logsumexp L of
// "FlashAttention-2 -- Deeper Math", Fix 2, so P_ij = exp(scale q_i.k_j - L_i) -- and forms, per
// tile,
//     dV += P^T dO,   dP = dO V^T,   dS = P * (dP - D),   dQ += scale dS K,   dK += scale dS^T Q,
// with D_i = sum_r dO_ir O_ir (the row identity of the same section) and masked entries
// contributing nothing. Nothing of size N x N is stored.
//
// Two kernels, so that every output element is summed by exactly one wave in a fixed order (no
// atomics, bit-reproducible):
//   fa_bwd_dq_kernel (queries outermost, like the forward): 4 waves x 32 query rows per
//     workgroup. A wave keeps its rows' Q^T and dO^T operands in registers and computes D for them
//     first (and stores it for the second kernel); per 32-key step of the K/V tiles in LDS:
//     S^T = K Q^T, dP^T = V dO^T (keys on M, queries on N, as in the forward kernel), P^T and dS^T
//     in fp32, then dQ^T += K^T dS^T with dS^T rounded to bf16 as the B operand and K^T read
//     with the transposing LDS read.
//   fa_bwd_dkdv_kernel (keys outermost; d = 64 -- at d = 128 its wide form in fa_bwd_wide.h,
//     with the same arithmetic in the same order): 8 waves x 32 keys per workgroup (two per
//     SIMD). A wave keeps its keys' K rows in registers and their V rows in LDS as B operands
//     and loops over the query tiles -- of every query
//     head that shares the K/V head, so grouped heads receive the sum of their query heads'
//     gradients -- with Q, dO, L and D of each 64-query tile in LDS: S = Q K^T, dP = dO V^T
//     (queries on M, keys on N), P and dS in fp32, then dV^T += dO^T P and dK^T += Q^T dS with
//     P, dS rounded to bf16 and dO^T, Q^T read with the transposing LDS read. When there are too
//     few (K/V head, key block) pairs to fill the GPU (grouped heads), the query heads of a group
//     are split over hsplit workgroups that write fp32 partial sums, and fa_bwd_combine_kernel
//     adds them in split order (still deterministic).
//
// Tiles are read both as rows and transposed, so they use the swizzled LDS layout and the direct
// global-to-LDS loads of fa_tiles.h.
#pragma once

#include <type_traits>

#include "fa_tiles.h"

namespace fa {

constexpr int kBwdQWaves = 4;                 // dQ kernel: waves per workgroup
constexpr int kBwdQRows = 32 * kBwdQWaves;    // query rows per dQ workgroup
constexpr int kBwdKvWaves = 8;                // dK/dV kernel: waves per workgroup
constexpr int kBwdKvRows = 32 * kBwdKvWaves;  // keys per dK/dV workgroup
constexpr int kBwdTile = 64;  // rows of a K/V tile (dQ kernel) or a Q/dO tile (dK/dV kernel)

struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const bf16* dout;
  const float* lse;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  float* dsum;  // D, [B * H][N] fp32 (written by the dQ kernel, read by the dK/dV kernel)
  float* part;  // with hsplit > 1: fp32 partial dK then dV, each [hsplit][B * H_kv][N][d]
  int hsplit;   // workgroups sharing one (K/V head, key block), each over group / hsplit query heads
  int N, H, Hkv, group;
  int BH, BHkv;  // B * H, B * H_kv
  int n_qblk, n_kblk;
  float scale, scale_log2;
  long long q_bs, q_hs, kv_bs, kv_hs;  // element strides of batch and head (q, o, dO, dQ share q's)
  int q_rs, kv_rs;                     // element stride between consecutive rows of one head
};

// ---------------------------------------------------------------------------------------------
// dQ (and D)
// ---------------------------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdQWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void fa_bwd_dq_kernel(BwdArgs a) {
  constexpr int DK = D / 16, DB = D / 32;
  // K/V operand reads in flight ahead of the S and dP products at d = 128: two (+2.5-2.8% on the
  // causal Llama backward, 192 -> 213 registers, still two waves per SIMD; four or six measured
  // lower). d = 64 keeps the compiler's order.
  constexpr int READ_AHEAD = D == 128 ? 2 : 0;
  using S = Swz<D>;
  __shared__ __attribute__((aligned(1024))) char sK2[2][S::template bytes<kBwdTile>()];  // two stages of K and V tiles
  __shared__ __attribute__((aligned(1024))) char sV2[2][S::template bytes<kBwdTile>()];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps wave tests scalar
  const int c = lane & 31, h = lane >> 5;
  race_check_poison<sizeof(sK2)>(sK2, tid, kBwdQWaves * 64);
  race_check_poison<sizeof(sV2)>(sV2, tid, kBwdQWaves * 64);
  race_check_barrier();
  int bh, qblk;
  map_block<CAUSAL>(blockIdx.x, gridDim.x, a.BH, a.n_qblk, bh, qblk);
  const int b = bh / a.H, hq = bh - b * a.H, hk = hq / a.group;
  const int N = a.N;
  const int qw0 = qblk * kBwdQRows + 32 * wave;
  const int qrow = qw0 + c;
  const long long qoff = b * a.q_bs + hq * a.q_hs + (long long)qrow * a.q_rs;
  const long long kvhead = b * a.kv_bs + hk * a.kv_hs;
  const long long rs = 2LL * a.kv_rs;

  // Q^T and dO^T operands of this lane's row; D = sum_r dO_r O_r over the row (two lanes hold
  // halves of it).
  bf16x8 qf[DK], df[DK];
  float dpart = 0.f;
#pragma unroll
  for (int dk = 0; dk < DK; dk++) {
    if (qrow < N) {
      qf[dk] = *reinterpret_cast<const bf16x8*>(a.q + qoff + dk * 16 + h * 8);
      df[dk] = *reinterpret_cast<const bf16x8*>(a.dout + qoff + dk * 16 + h * 8);
      const bf16x8 ov = *reinterpret_cast<const bf16x8*>(a.o + qoff + dk * 16 + h * 8);
#pragma unroll
      for (int e = 0; e < 8; e++) dpart = __builtin_fmaf((float)df[dk][e], (float)ov[e], dpart);
    } else {
      qf[dk] = bf16x8{};
      df[dk] = bf16x8{};
    }
  }
  const float drow = half_swap_sum(dpart);
  float lse2 = 0.f;
  if (qrow < N) {
    if (h == 0) a.dsum[(long long)bh * N + qrow] = drow;
    lse2 = a.lse[(long long)bh * N + qrow] * kLog2e;
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; db++) acc[db] = f32x16{};

  const int wave_last = CAUSAL ? min(N - 1, qw0 + 31) : N - 1;  // last key this wave needs
  const int blk_last = CAUSAL ? min(N - 1, qblk * kBwdQRows + kBwdQRows - 1) : N - 1;
  const int n_kt = blk_last / kBwdTile + 1;
  const char* kh = reinterpret_cast<const char*>(a.k + kvhead);
  const char* vh = reinterpret_cast<const char*>(a.v + kvhead);
  // Tile j sits in stage j % 2. Tile j+1 goes straight from memory into the other stage while
  // tile j is computed (that stage's readers finished tile j-1 before the last barrier); one
  // barrier per tile.
  constexpr int W = kBwdQWaves;
  dma_tile<D, kBwdTile, W>(sK2[0], kh, rs, 0, N, wave, lane);
  dma_tile<D, kBwdTile, W>(sV2[0], vh, rs, 0, N, wave, lane);
  wait_dma();
  __syncthreads();
  LaneOffsets<D> lo_;
  lo_.init(lane);
  // the stage is a compile-time constant of each copy of the loop body (immediate LDS offsets)
  auto tile = [&](auto stage_c, int j) {
    constexpr int stg = decltype(stage_c)::value;
    if (j + 1 < n_kt) {
      dma_tile<D, kBwdTile, W>(sK2[stg ^ 1], kh, rs, (j + 1) * kBwdTile, N, wave, lane);
      dma_tile<D, kBwdTile, W>(sV2[stg ^ 1], vh, rs, (j + 1) * kBwdTile, N, wave, lane);
    }
    race_check_drain();
    const char* sK = sK2[stg];
    const char* sV = sV2[stg];
#pragma unroll
    for (int sb = 0; sb < 2; sb++) {
      const int k0 = j * kBwdTile + 32 * sb;
      if (k0 > wave_last) continue;  // (next sb)
      f32x16 st = f32x16{}, dpt = f32x16{};
      if constexpr (READ_AHEAD > 0) {
        // the K and V operands read READ_AHEAD MFMAs ahead of the two products (left to itself
        // the compiler waits for each read right before its MFMA)
        bf16x8 kr[DK], vr[DK];
#pragma unroll
        for (int dk = 0; dk < DK; dk++) kr[dk] = tile_row_at<D>(sK, lo_, 32 * sb, dk);
#pragma unroll
        for (int dk = 0; dk < DK; dk++) vr[dk] = tile_row_at<D>(sV, lo_, 32 * sb, dk);
#pragma unroll
        for (int dk = 0; dk < DK; dk++) st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[dk], qf[dk], st, 0, 0, 0);
#pragma unroll
        for (int dk = 0; dk < DK; dk++) dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[dk], df[dk], dpt, 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, READ_AHEAD, 0);  // LDS reads
#pragma unroll
        for (int i = 0; i < 2 * DK - READ_AHEAD; i++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);           // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, READ_AHEAD, 0);
      } else {
#pragma unroll
        for (int dk = 0; dk < DK; dk++)
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_row_at<D>(sK, lo_, 32 * sb, dk), qf[dk], st, 0, 0, 0);
#pragma unroll
        for (int dk = 0; dk < DK; dk++)
          dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_row_at<D>(sV, lo_, 32 * sb, dk), df[dk], dpt, 0, 0, 0);
      }
      // P^T = exp(S^T scale - L), masked; dS^T = P^T (dP^T - D). Register i holds key
      // k0 + acc_row(i, h), visible iff acc_row(i, 0) <= lim (keys below N and, causal, <= qrow).
      const bool edge = (CAUSAL && k0 + 31 > qw0) || k0 + 31 >= N;  // wave-uniform
      const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - k0 - 4 * h;
      bf16x8 dsf[2];
#pragma unroll
      for (int i = 0; i < 16; i++) {
        float p = fast_exp2(__builtin_fmaf(st[i], a.scale_log2, -lse2));
        if (edge) p = acc_row(i, 0) <= lim ? p : 0.f;
        dsf[i >> 3][i & 7] = (bf16)(p * (dpt[i] - drow));
      }
#pragma unroll
      for (int ks = 0; ks < 2; ks++)
#pragma unroll
        for (int db = 0; db < DB; db++)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_tr_at<D>(sK, lo_, 32 * sb + 16 * ks, db),
                                                            dsf[ks], acc[db], 0, 0, 0);
    }
    if (j + 1 < n_kt) {
      wait_dma();
      __syncthreads();
    }
  };
  for (int j = 0; j < n_kt; j += 2) {
    tile(std::integral_constant<int, 0>{}, j);
    if (j + 1 < n_kt) tile(std::integral_constant<int, 1>{}, j + 1);
  }

  // dQ goes out through LDS (the K/V stages, free once every wave is past the last tile): each
  // wave writes its 32 rows into a swizzled region of its own and reads them back as whole rows.
  constexpr int OREG = 32 * S::ROW;  // one wave's 32 rows
  static_assert(kBwdQWaves * OREG <= (int)sizeof(sK2), "dQ staging fits");
  __syncthreads();
  char* const so = &sK2[0][0] + wave * OREG;
#pragma unroll
  for (int db = 0; db < DB; db++)
#pragma unroll
    for (int g4 = 0; g4 < 4; g4++) {
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; e++) v4[e] = (bf16)(acc[db][4 * g4 + e] * a.scale);
      *(FA_LDS bf16x4*)((FA_LDS char*)so + S::off(c, 4 * db + g4) + 8 * h) = v4;
    }
  constexpr int RPI = 64 / S::CPR;  // rows per read instruction
#pragma unroll
  for (int it = 0; it < 32 / RPI; it++) {
    const int r = RPI * it + lane / S::CPR, j = lane % S::CPR;
    const bf16x8 v8 = *(const FA_LDS bf16x8*)((FA_LDS char*)so + S::off(r, j));
    const int row = qw0 + r;
    if (row < N) *reinterpret_cast<bf16x8*>(a.dq + b * a.q_bs + hq * a.q_hs + (long long)row * a.q_rs + 8 * j) = v8;
  }
}

// ---------------------------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdKvWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void fa_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int DK = D / 16, DB = D / 32;
  using S = Swz<D>;
  __shared__ __attribute__((aligned(1024))) char sQ2[2][S::template bytes<kBwdTile>()];  // two stages of Q and dO tiles
  __shared__ __attribute__((aligned(1024))) char sO2[2][S::template bytes<kBwdTile>()];
  __shared__ __attribute__((aligned(16))) float sL2[2][kBwdTile];    // L * log2(e)
  __shared__ __attribute__((aligned(16))) float sD2[2][kBwdTile];    // D
  __shared__ __attribute__((aligned(1024))) char sVb[kBwdKvRows * S::ROW];  // this block's V rows

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps wave tests scalar
  const int c = lane & 31, h = lane >> 5;
  race_check_poison<sizeof(sQ2)>(sQ2, tid, kBwdKvWaves * 64);
  race_check_poison<sizeof(sO2)>(sO2, tid, kBwdKvWaves * 64);
  race_check_poison<sizeof(sL2)>(sL2, tid, kBwdKvWaves * 64);
  race_check_poison<sizeof(sD2)>(sD2, tid, kBwdKvWaves * 64);
  race_check_poison<sizeof(sVb)>(sVb, tid, kBwdKvWaves * 64);
  race_check_barrier();
  int vh, x;  // vh: (batch * K/V head, query-head split)
  map_block<CAUSAL>(blockIdx.x, gridDim.x, a.BHkv * a.hsplit, a.n_kblk, vh, x);
  const int kblk = CAUSAL ? a.n_kblk - 1 - x : x;  // causal: the first key blocks, which see the
                                                   // most queries, first
  const int bkv = vh / a.hsplit, split = vh - bkv * a.hsplit;
  const int gps = a.group / a.hsplit, g0 = split * gps;  // this workgroup's query heads g0..
  const int b = bkv / a.Hkv, hk = bkv - b * a.Hkv;
  const int N = a.N;
  const int kw0 = kblk * kBwdKvRows + 32 * wave;
  const int krow = kw0 + c;
  const long long kvoff = b * a.kv_bs + hk * a.kv_hs + (long long)krow * a.kv_rs;
  const long long rs = 2LL * a.q_rs;

  // K rows of this lane's key as the B operand of S = Q K^T, in registers for the whole kernel.
  // V rows (the B operand of dP = dO V^T) go to LDS once and are read per step: keeping both in
  // registers as well as the two accumulators does not fit two waves per SIMD.
  bf16x8 kf[DK];
#pragma unroll
  for (int dk = 0; dk < DK; dk++) {
    kf[dk] = krow < N ? *reinterpret_cast<const bf16x8*>(a.k + kvoff + dk * 16 + h * 8) : bf16x8{};
    const bf16x8 vv = krow < N ? *reinterpret_cast<const bf16x8*>(a.v + kvoff + dk * 16 + h * 8) : bf16x8{};
    *(FA_LDS bf16x8*)(sVb + S::off(32 * wave + c, 2 * dk + h)) = vv;
  }
  f32x16 acck[DB], accv[DB];
#pragma unroll
  for (int db = 0; db < DB; db++) {
    acck[db] = f32x16{};
    accv[db] = f32x16{};
  }

  const int t0 = CAUSAL ? (kblk * kBwdKvRows) / kBwdTile : 0;  // first query tile with a visible key
  const int n_qt = (N + kBwdTile - 1) / kBwdTile;
  const int n_steps = gps * (n_qt - t0);  // (query head, query tile) pairs, in that order
  // Step s (a query head and 64-query tile) sits in stage s % 2; step s+1's Q and dO tiles go
  // straight from memory into the other stage while step s is computed, its L and D through one
  // register of the first 128 threads; one barrier per step.
  constexpr int W = kBwdKvWaves;
  float lsd = 0.f;
  auto issue_step = [&](int s) {
    const int g = g0 + s / (n_qt - t0), t = t0 + s % (n_qt - t0);
    const int bh = b * a.H + hk * a.group + g;
    const long long qhead = b * a.q_bs + (long long)(hk * a.group + g) * a.q_hs;
    dma_tile<D, kBwdTile, W>(sQ2[s & 1], reinterpret_cast<const char*>(a.q + qhead), rs, t * kBwdTile, N,
                   wave, lane);
    dma_tile<D, kBwdTile, W>(sO2[s & 1], reinterpret_cast<const char*>(a.dout + qhead), rs, t * kBwdTile,
                   N, wave, lane);
    if (tid < 2 * kBwdTile) {
      const int r = t * kBwdTile + (tid & (kBwdTile - 1));
      const long long idx = (long long)bh * N + min(r, N - 1);
      // raw value: any arithmetic on it here would make the compiler wait for the load at once,
      // and with it (loads complete in order) for the DMA just issued
      lsd = tid < kBwdTile ? a.lse[idx] : a.dsum[idx];
    }
  };
  auto publish_step = [&](int s) {  // after the DMA and the L/D loads of step s have landed
    if (tid < kBwdTile) sL2[s & 1][tid] = lsd * kLog2e;
    else if (tid < 2 * kBwdTile) sD2[s & 1][tid - kBwdTile] = lsd;
  };
  issue_step(0);
  wait_dma();
  publish_step(0);
  __syncthreads();
  LaneOffsets<D> lo_;
  lo_.init(lane);
  const int vb_row = 32 * wave;  // this wave's V rows in sVb
  // the stage is a compile-time constant of each copy of the loop body (immediate LDS offsets)
  auto step = [&](auto stage_c, int s) {
    constexpr int stg = decltype(stage_c)::value;
    const int t = t0 + s % (n_qt - t0);
    if (s + 1 < n_steps) issue_step(s + 1);
    race_check_drain();
    const char* sQ = sQ2[stg];
    const char* sO = sO2[stg];
    const float* sL = sL2[stg];
    const float* sD = sD2[stg];
#pragma unroll
    for (int sb = 0; sb < 2; sb++) {
      const int q0 = t * kBwdTile + 32 * sb;
      if (q0 >= N || (CAUSAL && q0 + 31 < kw0)) continue;  // (next sb)
      // register i holds query q0 + acc_row(i, h): visible iff below N and (causal) >= krow, i.e.
      // lo <= acc_row(i, 0) <= hi
      const bool edge = (CAUSAL && q0 < kw0 + 31) || q0 + 31 >= N;  // wave-uniform
      const int hi = N - 1 - q0 - 4 * h;
      const int lo = CAUSAL ? krow - q0 - 4 * h : -1024;
      // S = Q K^T, then P (rows: queries 32 sb + acc_row(i, h); L of those from LDS) and its
      // bf16 copy, then dV^T += dO^T P -- so S and the bf16 P are dead before dP is formed.
      f32x16 sc = f32x16{};
#pragma unroll
      for (int dk = 0; dk < DK; dk++)
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_row_at<D>(sQ, lo_, 32 * sb, dk), kf[dk], sc, 0, 0, 0);
      float p[16];
      bf16x8 pf[2];
#pragma unroll
      for (int j4 = 0; j4 < 4; j4++) {
        const f32x4v lv = *(const FA_LDS f32x4v*)(&sL[32 * sb + 8 * j4 + 4 * h]);
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const int i = 4 * j4 + e;
          float pi = fast_exp2(__builtin_fmaf(sc[i], a.scale_log2, -lv[e]));
          if (edge) pi = (acc_row(i, 0) >= lo && acc_row(i, 0) <= hi) ? pi : 0.f;
          p[i] = pi;
          pf[i >> 3][i & 7] = (bf16)pi;
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ks++)
#pragma unroll
        for (int db = 0; db < DB; db++)
          accv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_tr_at<D>(sO, lo_, 32 * sb + 16 * ks, db),
                                                             pf[ks], accv[db], 0, 0, 0);
      // dP = dO V^T, dS = P (dP - D), then dK^T += Q^T dS
      f32x16 dp = f32x16{};
#pragma unroll
      for (int dk = 0; dk < DK; dk++)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_row_at<D>(sO, lo_, 32 * sb, dk),
                                                     tile_row_at<D>(sVb, lo_, vb_row, dk), dp, 0, 0, 0);
      bf16x8 dsf[2];
#pragma unroll
      for (int j4 = 0; j4 < 4; j4++) {
        const f32x4v dv = *(const FA_LDS f32x4v*)(&sD[32 * sb + 8 * j4 + 4 * h]);
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const int i = 4 * j4 + e;
          dsf[i >> 3][i & 7] = (bf16)(p[i] * (dp[i] - dv[e]));
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ks++)
#pragma unroll
        for (int db = 0; db < DB; db++)
          acck[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_tr_at<D>(sQ, lo_, 32 * sb + 16 * ks, db),
                                                             dsf[ks], acck[db], 0, 0, 0);
    }
    if (s + 1 < n_steps) {
      wait_dma();
      race_check_barrier();
      publish_step(s + 1);
      __syncthreads();
    }
  };
  for (int s = 0; s < n_steps; s += 2) {
    step(std::integral_constant<int, 0>{}, s);
    if (s + 1 < n_steps) step(std::integral_constant<int, 1>{}, s + 1);
  }

  if (krow < N && a.hsplit > 1) {
    // partial sums of this split, fp32; fa_bwd_combine_kernel adds the splits in order
    const long long prow = ((long long)(split * a.BHkv + bkv) * N + krow) * D;
    const long long pstride = (long long)a.hsplit * a.BHkv * N * D;  // dK part -> dV part
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        f32x4v k4, v4;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          k4[e] = acck[db][4 * g4 + e] * a.scale;
          v4[e] = accv[db][4 * g4 + e];
        }
        *reinterpret_cast<f32x4v*>(a.part + prow + 32 * db + 8 * g4 + 4 * h) = k4;
        *reinterpret_cast<f32x4v*>(a.part + pstride + prow + 32 * db + 8 * g4 + 4 * h) = v4;
      }
  } else if (krow < N) {
    bf16* dkr = a.dk + kvoff;
    bf16* dvr = a.dv + kvoff;
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        bf16x4 k4, v4;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          k4[e] = (bf16)(acck[db][4 * g4 + e] * a.scale);
          v4[e] = (bf16)accv[db][4 * g4 + e];
        }
        *reinterpret_cast<bf16x4*>(dkr + 32 * db + 8 * g4 + 4 * h) = k4;
        *reinterpret_cast<bf16x4*>(dvr + 32 * db + 8 * g4 + 4 * h) = v4;
      }
  }
}

// dK, dV = sum over the hsplit partials, in split order, rounded to bf16 once. One thread per 4
// consecutive elements of one K/V row.
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_combine_kernel(BwdArgs a) {
  const long long n4 = (long long)a.BHkv * a.N * (D / 4);
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const long long e = 4 * i;                  // element index in [B * H_kv][N][D]
  const int col = (int)(e % D);
  const long long row = e / D;                // (bkv, n)
  const int n = (int)(row % a.N), bkv = (int)(row / a.N);
  const int b = bkv / a.Hkv, hk = bkv - b * a.Hkv;
  const long long pstride = (long long)a.hsplit * a.BHkv * a.N * D, sstride = (long long)a.BHkv * a.N * D;
  f32x4v sk = *reinterpret_cast<const f32x4v*>(a.part + e);
  f32x4v sv = *reinterpret_cast<const f32x4v*>(a.part + pstride + e);
  for (int sp = 1; sp < a.hsplit; sp++) {
    sk += *reinterpret_cast<const f32x4v*>(a.part + sp * sstride + e);
    sv += *reinterpret_cast<const f32x4v*>(a.part + pstride + sp * sstride + e);
  }
  const long long off = b * a.kv_bs + hk * a.kv_hs + (long long)n * a.kv_rs + col;
  bf16x4 k4, v4;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    k4[j] = (bf16)sk[j];
    v4[j] = (bf16)sv[j];
  }
  *reinterpret_cast<bf16x4*>(a.dk + off) = k4;
  *reinterpret_cast<bf16x4*>(a.dv + off) = v4;
}

}  // namespace fa
