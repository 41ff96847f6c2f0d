// Wide dK/dV kernel of the attention backward pass for gfx950, head dim 128 (the choice is made in
// fa_api.hip). It computes what fa_bwd_dkdv_kernel (fa_bwd.h) computes, with the same products in
// the same order for every accumulator ("Understanding FlashAttention Pt 1", §3.6: P rebuilt from
// Q K^T and the logsumexp, dV += P^T dO, dP = dO V^T, dS = P * (dP - D), dK += scale dS^T Q), so
// its outputs are bit-identical to that kernel's; what differs is the shape of the work per wave.
//
//   * A workgroup is 4 waves, one per SIMD, over the same 256 keys. A wave owns 64 keys as two
//     32-key blocks A and B: their K rows (B operand of S = Q K^T) in registers, their V rows (B
//     operand of dP = dO V^T) in LDS, and their dK^T and dV^T accumulators (256 registers).
//   * Every Q and dO operand fragment read from LDS -- as rows for S and dP, transposed for dV^T
//     and dK^T -- feeds one MFMA of each block. Per 32x32x16 MFMA a wave issues 1.1 LDS reads
//     instead of 2 (the transposing reads deliver half the bytes of a row read per instruction,
//     and the LDS, shared by the 4 SIMDs of a CU, takes about one read instruction per 4 clocks).
//   * A 32-query sub-block is four phases of 16 MFMAs (8 groups of one MFMA per block):
//         P1  S   = Q K^T     (A and B)
//         P2  dP  = dO V^T    | P = 2^(S scale log2(e) - L), and its bf16 copy
//         P3  dV^T += dO^T P  | dS = P (dP - D), bf16
//         P4  dK^T += Q^T dS
//     Operand reads run two groups ahead of their MFMAs, across phase boundaries; the vector work
//     of a phase uses only results of the phases before it.
//   * Q and dO tiles of 64 queries go straight from memory into two swizzled LDS stages by 16-byte
//     DMA, with their logsumexp and D values; one barrier per tile. The tiles run over every
//     query head that shares the K/V head (or a split of them, as in fa_bwd.h), and over the query
//     tiles from the workgroup's first key on (causal). A wave skips the tiles whose queries all
//     precede its keys (it still meets their barriers); the steps that cross its causal diagonal or
//     the end of the sequence are masked after the exponentials, in a wave-uniform branch.
//   * dK and dV go out through LDS as whole rows (or, with query-head splits, as fp32 partial sums
//     that fa_bwd_combine_kernel adds in split order).
#pragma once

#include "fa_bwd.h"

namespace fa {

#ifndef FA_BWD_RA
#define FA_BWD_RA 2
#endif
constexpr int kBwdWideWaves = 4;
static_assert(64 * kBwdWideWaves == kBwdKvRows, "same key block as the 8-wave kernel");

// S = Q K^T and dP = dO V^T, written out so that their results land in VGPRs (the vector
// instructions read them) while the compiler keeps its own MFMAs -- the dK^T and dV^T
// accumulations, 256 accumulator registers -- in AGPRs (it picks one MFMA form per function).
// The compiler's hazard checks do not look inside inline assembly, so the waits these MFMAs need
// are written out too: their A/B operands come from LDS reads (covered by the compiler's lgkmcnt
// waits) or from registers set long before; a chain on one accumulator needs no wait between its
// MFMAs; and before a vector instruction reads the result, bwd_wide_ready() gives the wait states
// an 8-pass MFMA's result needs.
__device__ __forceinline__ void mfma_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_next(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// Every read of x and y comes after this statement: 20 wait states after the MFMAs that wrote them.
__device__ __forceinline__ void bwd_wide_ready(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(x), "+v"(y));
}

template <bool CAUSAL>
__global__ __launch_bounds__(kBwdWideWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void fa_bwd_dkdv_wide_kernel(BwdArgs a) {
  constexpr int D = 128, DK = 8, DB = 4, TQ = kBwdTile;
  constexpr int W = kBwdWideWaves;
  constexpr int RA = FA_BWD_RA;  // operand reads run RA groups ahead of their MFMAs
  using S = Swz<D>;
  constexpr int TILE = S::template bytes<TQ>();
  // One LDS array: two stages of the Q tile, two of the dO tile, the block's V rows, then the L
  // (times log2(e)) and D values of both stages. The tiles come first so that every tile read's
  // offset fits the 16-bit immediate of the LDS instruction.
  constexpr int OFF_O = 2 * TILE, OFF_V = 4 * TILE, OFF_L = OFF_V + kBwdKvRows * S::ROW;
  constexpr int OFF_D = OFF_L + 2 * TQ * 4, LDS_BYTES = OFF_D + 2 * TQ * 4;
  static_assert(OFF_V <= 65536, "tile offsets are immediates");
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  char (*const sQ2)[TILE] = reinterpret_cast<char (*)[TILE]>(smem);
  char (*const sO2)[TILE] = reinterpret_cast<char (*)[TILE]>(smem + OFF_O);
  float (*const sL2)[TQ] = reinterpret_cast<float (*)[TQ]>(smem + OFF_L);
  float (*const sD2)[TQ] = reinterpret_cast<float (*)[TQ]>(smem + OFF_D);
  char* const sVb = smem + OFF_V;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h = lane >> 5;
  race_check_poison<LDS_BYTES>(smem, tid, W * 64);
  race_check_barrier();
  int vh, x;  // vh: (batch * K/V head, query-head split)
  map_block<CAUSAL>(blockIdx.x, gridDim.x, a.BHkv * a.hsplit, a.n_kblk, vh, x);
  const int kblk = CAUSAL ? a.n_kblk - 1 - x : x;  // causal: the key blocks with most queries first
  const int bkv = vh / a.hsplit, split = vh - bkv * a.hsplit;
  const int gps = a.group / a.hsplit, g0 = split * gps;  // this workgroup's query heads g0..
  const int b = bkv / a.Hkv, hk = bkv - b * a.Hkv;
  const int N = a.N;
  const float sl2 = a.scale_log2;
  const int kw0 = kblk * kBwdKvRows + 64 * wave;  // first key of block A; block B starts 32 later
  const long long kvh = b * a.kv_bs + hk * a.kv_hs;
  const long long rs = 2LL * a.q_rs;

  // K rows of the lane's keys (c of block A, c of block B) in registers; V rows into this wave's
  // 64 rows of sVb, which no other wave reads.
  char* const vrows = sVb + 64 * wave * S::ROW;
  bf16x8 kf[2][DK];
#pragma unroll
  for (int blk = 0; blk < 2; blk++) {
    const int krow = kw0 + 32 * blk + c;
    const long long off = kvh + (long long)krow * a.kv_rs;
#pragma unroll
    for (int dk = 0; dk < DK; dk++) {
      kf[blk][dk] = krow < N ? *reinterpret_cast<const bf16x8*>(a.k + off + dk * 16 + h * 8) : bf16x8{};
      const bf16x8 vv = krow < N ? *reinterpret_cast<const bf16x8*>(a.v + off + dk * 16 + h * 8) : bf16x8{};
      *(FA_LDS bf16x8*)(vrows + S::off(32 * blk + c, 2 * dk + h)) = vv;
    }
  }
  f32x16 acck[2][DB], accv[2][DB];
#pragma unroll
  for (int blk = 0; blk < 2; blk++)
#pragma unroll
    for (int db = 0; db < DB; db++) acck[blk][db] = accv[blk][db] = f32x16{};

  const int t0 = CAUSAL ? (kblk * kBwdKvRows) / TQ : 0;  // first query tile with a visible key
  const int n_qt = (N + TQ - 1) / TQ;
  const int nt = n_qt - t0;        // query tiles per query head
  const int n_steps = gps * nt;    // (query head, query tile) pairs, in that order
  // first tile with a query that a key of this wave sees; none if its keys all lie past N
  const int t_act = kw0 >= N ? n_qt : (CAUSAL ? kw0 / TQ : 0);

  // Step s (a query head and 64-query tile) sits in stage s % 2; step s+1's Q and dO tiles go
  // straight from memory into the other stage while step s is computed, its L and D through one
  // register of the first 128 threads; one barrier per step.
  float lsd = 0.f;
  auto issue_step = [&](int s) {
    const int g = g0 + s / nt, t = t0 + s % nt;
    const int bh = b * a.H + hk * a.group + g;
    const long long qhead = b * a.q_bs + (long long)(hk * a.group + g) * a.q_hs;
    dma_tile<D, TQ, W>(sQ2[s & 1], reinterpret_cast<const char*>(a.q + qhead), rs, t * TQ, N, wave, lane);
    dma_tile<D, TQ, W>(sO2[s & 1], reinterpret_cast<const char*>(a.dout + qhead), rs, t * TQ, N, wave,
                       lane);
    if (tid < 2 * TQ) {
      const int r = t * TQ + (tid & (TQ - 1));
      const long long idx = (long long)bh * N + min(r, N - 1);
      // raw value: any arithmetic on it here would make the compiler wait for the load at once,
      // and with it (loads complete in order) for the DMA just issued
      lsd = tid < TQ ? a.lse[idx] : a.dsum[idx];
    }
  };
  auto publish_step = [&](int s) {  // after the DMA and the L/D loads of step s have landed
    if (tid < TQ) sL2[s & 1][tid] = lsd * kLog2e;
    else if (tid < 2 * TQ) sD2[s & 1][tid - TQ] = lsd;
  };
  issue_step(0);
  wait_dma();
  publish_step(0);
  __syncthreads();
  LaneOffsets<D> lo_;
  lo_.init(lane);

  // One 32-query sub-block (queries q0 = t TQ + 32 sb ..) of the tile in stage st: the four phases
  // of the header comment. Register i of a 32x32 result holds query q0 + acc_row(i, h) and key
  // kw0 + 32 blk + c.
  auto sub = [&](auto st_c, auto sb_c, int t) __attribute__((always_inline)) {
    constexpr int st = decltype(st_c)::value, sb = decltype(sb_c)::value;
    const char* sQ = sQ2[st];
    const char* sO = sO2[st];
    const float* sL = sL2[st];
    const float* sD = sD2[st];
    const int q0 = t * TQ + 32 * sb;
    auto rowQ = [&](int dk) __attribute__((always_inline)) { return tile_row_at<D>(sQ, lo_, 32 * sb, dk); };
    auto rowO = [&](int dk) __attribute__((always_inline)) { return tile_row_at<D>(sO, lo_, 32 * sb, dk); };
    auto rowV = [&](int blk, int dk) __attribute__((always_inline)) { return tile_row_at<D>(vrows, lo_, 32 * blk, dk); };
    auto trQ = [&](int i) __attribute__((always_inline)) { return tile_tr_at<D>(sQ, lo_, 32 * sb + 16 * (i >> 2), i & 3); };
    auto trO = [&](int i) __attribute__((always_inline)) { return tile_tr_at<D>(sO, lo_, 32 * sb + 16 * (i >> 2), i & 3); };

    bf16x8 fq[DK], fo[DK], fv[2][DK], tO[8], tQ[8];
    // L (D) of the rows of values 2i, 2i+1: rows acc_row(2i, h), +1, adjacent in LDS
    auto pair = [&](const float* v, int i) __attribute__((always_inline)) {
      return *(const FA_LDS f32x2v*)(&v[32 * sb + acc_row(2 * i, h)]);
    };
    f32x2v lp[8], dp[8];
    // P1: S = Q K^T
    f32x16 s0, s1;
#pragma unroll
    for (int i = 0; i < RA; i++) fq[i] = rowQ(i);
#pragma unroll
    for (int i = 0; i < DK; i++) {
      if (i + RA < DK) fq[i + RA] = rowQ(i + RA);
      if (i >= DK - RA) {
        fo[i - DK + RA] = rowO(i - DK + RA);
        fv[0][i - DK + RA] = rowV(0, i - DK + RA);
        fv[1][i - DK + RA] = rowV(1, i - DK + RA);
        lp[i - DK + RA] = pair(sL, i - DK + RA);
      }
      if (i == 0) {
        mfma_first(s0, fq[i], kf[0][i]);
        mfma_first(s1, fq[i], kf[1][i]);
      } else {
        mfma_next(s0, fq[i], kf[0][i]);
        mfma_next(s1, fq[i], kf[1][i]);
      }
      fence();
    }
    // P2: dP = dO V^T; P and its bf16 copy (values 2i, 2i+1 of both blocks in group i)
    f32x16 d0, d1;
    float p0[16], p1[16];
    bf16x8 pf0[2], pf1[2];
#pragma unroll
    for (int i = 0; i < DK; i++) {
      if (i + RA < DK) {
        fo[i + RA] = rowO(i + RA);
        fv[0][i + RA] = rowV(0, i + RA);
        fv[1][i + RA] = rowV(1, i + RA);
      }
      if (i + RA < DK) lp[i + RA] = pair(sL, i + RA);
      if (i >= DK - RA) {
        tO[i - DK + RA] = trO(i - DK + RA);
        dp[i - DK + RA] = pair(sD, i - DK + RA);
      }
      if (i == 0) {
        mfma_first(d0, fo[i], fv[0][i]);
        mfma_first(d1, fo[i], fv[1][i]);
        bwd_wide_ready(s0, s1);
      } else {
        mfma_next(d0, fo[i], fv[0][i]);
        mfma_next(d1, fo[i], fv[1][i]);
      }
      const f32x2v lv = lp[i];
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int k = 2 * i + u;
        const float L = lv[u];
        p0[k] = fast_exp2(__builtin_fmaf(s0[k], sl2, -L));
        p1[k] = fast_exp2(__builtin_fmaf(s1[k], sl2, -L));
        pf0[k >> 3][k & 7] = (bf16)p0[k];
        pf1[k >> 3][k & 7] = (bf16)p1[k];
        pin(p0[k]);
        pin(p1[k]);
      }
      fence();
    }
    // masks of the sub-blocks that cross a block's causal diagonal or the end of the sequence
    // (wave-uniform): query q0 + acc_row(i, h) and key krow are visible together iff the query is
    // below N and (causal) not before the key
    if (__builtin_expect((CAUSAL && q0 <= kw0 + 32) || q0 + 31 >= N, 0)) {
      const int hi = N - 1 - q0 - 4 * h;
      const int lo0 = CAUSAL ? kw0 + c - q0 - 4 * h : -1024, lo1 = lo0 + 32;
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int r = acc_row(i, 0);
        p0[i] = r >= lo0 && r <= hi ? p0[i] : 0.f;
        p1[i] = r >= lo1 && r <= hi ? p1[i] : 0.f;
        pf0[i >> 3][i & 7] = (bf16)p0[i];
        pf1[i >> 3][i & 7] = (bf16)p1[i];
      }
    }
    // P3: dV^T += dO^T P; dS = P (dP - D)
    bf16x8 ds0[2], ds1[2];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int ks = i >> 2, db = i & 3;
      if (i + RA < 8) tO[i + RA] = trO(i + RA);
      if (i + RA < 8) dp[i + RA] = pair(sD, i + RA);
      if (i >= 8 - RA) tQ[i - 8 + RA] = trQ(i - 8 + RA);
      if (i == 0) bwd_wide_ready(d0, d1);
      accv[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tO[i], pf0[ks], accv[0][db], 0, 0, 0);
      accv[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tO[i], pf1[ks], accv[1][db], 0, 0, 0);
      const f32x2v dv = dp[i];
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int k = 2 * i + u;
        const float Dv = dv[u];
        ds0[k >> 3][k & 7] = (bf16)(p0[k] * (d0[k] - Dv));
        ds1[k >> 3][k & 7] = (bf16)(p1[k] * (d1[k] - Dv));
      }
      pin(ds0[i >> 2]);
      pin(ds1[i >> 2]);
      fence();
    }
    // P4: dK^T += Q^T dS
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int ks = i >> 2, db = i & 3;
      if (i + RA < 8) tQ[i + RA] = trQ(i + RA);
      acck[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tQ[i], ds0[ks], acck[0][db], 0, 0, 0);
      acck[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tQ[i], ds1[ks], acck[1][db], 0, 0, 0);
      fence();
    }
  };

  // the stage is a compile-time constant of each copy of the loop body (immediate LDS offsets)
  auto step = [&](auto stage_c, int s) __attribute__((always_inline)) {
    constexpr int stg = decltype(stage_c)::value;
    const int t = t0 + s % nt;
    if (s + 1 < n_steps) issue_step(s + 1);
    race_check_drain();
    if (t >= t_act) {
      sub(stage_c, std::integral_constant<int, 0>{}, t);
      if (t * TQ + 32 < N) sub(stage_c, std::integral_constant<int, 1>{}, t);
    }
    (void)stg;
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

  if (a.hsplit > 1) {
    // partial sums of this split, fp32; fa_bwd_combine_kernel adds the splits in order
    const long long pstride = (long long)a.hsplit * a.BHkv * N * D;  // dK part -> dV part
#pragma unroll
    for (int blk = 0; blk < 2; blk++) {
      const int krow = kw0 + 32 * blk + c;
      if (krow >= N) continue;
      const long long prow = ((long long)(split * a.BHkv + bkv) * N + krow) * D;
#pragma unroll
      for (int db = 0; db < DB; db++)
#pragma unroll
        for (int g4 = 0; g4 < 4; g4++) {
          f32x4v k4, v4;
#pragma unroll
          for (int e = 0; e < 4; e++) {
            k4[e] = acck[blk][db][4 * g4 + e] * a.scale;
            v4[e] = accv[blk][db][4 * g4 + e];
          }
          *reinterpret_cast<f32x4v*>(a.part + prow + 32 * db + 8 * g4 + 4 * h) = k4;
          *reinterpret_cast<f32x4v*>(a.part + pstride + prow + 32 * db + 8 * g4 + 4 * h) = v4;
        }
    }
    return;
  }

  // dK and dV go out through LDS as whole rows: dK through a 16 KB region of the Q/dO stages
  // (free once every wave is past the last tile), dV through the wave's own V rows.
  __syncthreads();
  char* const sk = smem + wave * (64 * S::ROW);  // the Q and dO stages: 4 x 16 KB
#pragma unroll
  for (int blk = 0; blk < 2; blk++)
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        bf16x4 k4, v4;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          k4[e] = (bf16)(acck[blk][db][4 * g4 + e] * a.scale);
          v4[e] = (bf16)accv[blk][db][4 * g4 + e];
        }
        const int o = S::off(32 * blk + c, 4 * db + g4) + 8 * h;
        *(FA_LDS bf16x4*)((FA_LDS char*)sk + o) = k4;
        *(FA_LDS bf16x4*)((FA_LDS char*)vrows + o) = v4;
      }
#pragma unroll
  for (int it = 0; it < 16; it++) {
    const int r = 4 * it + (lane >> 4), j = lane & 15;
    const int krow = kw0 + r;
    const bf16x8 k8 = *(const FA_LDS bf16x8*)((FA_LDS char*)sk + S::off(r, j));
    const bf16x8 v8 = *(const FA_LDS bf16x8*)((FA_LDS char*)vrows + S::off(r, j));
    if (krow < N) {
      const long long off = kvh + (long long)krow * a.kv_rs + 8 * j;
      *reinterpret_cast<bf16x8*>(a.dk + off) = k8;
      *reinterpret_cast<bf16x8*>(a.dv + off) = v8;
    }
  }
}

}  // namespace fa
