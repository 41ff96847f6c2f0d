// 4-wave forward kernel, gfx950: the score variants, d = 256, and (with no variant enabled) the
// plain bf16 forward on causal d = 128 and on every grid past 2^16 query rows, where it is faster
// than the 8-wave kernel (the choice and its measurements are in fa_api.hip).
//
// "Understanding FlashAttention Pt 1" writes the scores as S = QK^T / sqrt(d) + B, B an optional
// additive mask or bias (§0.2), and lists local/sliding-window attention and ALiBi-style bias
// among the variants a tiled kernel executes (§3.5, §4.2); "FlashAttention-2 -- Deeper Math" and
// "Flash Attention" put the supported head dims at 64, 128 and 256. This kernel computes
//     S_ij = scale q_i.k_j + B_ij - m_h |i - j|,   key j visible iff causal rule and
//            i - window_left <= j <= i + window_right,
// with the same tiled online softmax as the 8-wave kernel: S and P stay in registers, a running
// maximum and sum per row, one division at the end, LSE = m + ln l. The bias B is a bf16 tensor
// (any batch/head/row strides; stride 0 shares it), the ALiBi slopes m_h one fp32 per query head.
// Tiles outside the window (or past the causal diagonal) are skipped for the whole workgroup, and
// 32-key steps outside a wave's window for that wave (§3.5: only tiles crossing the boundary need
// element-level masks).
//
// Structure: 4 waves x 32 query rows per workgroup (several workgroups per CU), queries outermost;
// K/V tiles (32 keys; 64 for d = 64) go straight from memory into two swizzled LDS stages
// (fa_tiles.h), one barrier per tile; so do 64-key tiles of the bias for the workgroup's rows,
// requested up to two K/V tiles ahead (BiasTile). Per 32-key step a wave forms S^T = K Q^T (keys
// on M, so a lane holds 16 keys of one query row), adds the bias and ALiBi terms in fp32, masks,
// moves the running reference lazily (as the 8-wave kernel does; with the -inf reference guard of
// "Online Softmax & FlashAttention", Listing 26.3), and accumulates O^T += V^T P^T with P rounded
// to bf16; O leaves through LDS as whole rows. A row that sees no key at all (possible only through
// -inf bias entries) ends with O = 0 and LSE = -inf.
#pragma once

#include <type_traits>

#include "fa_tiles.h"

namespace fa {

constexpr int kExtWaves = 4;
constexpr int kExtRows = 32 * kExtWaves;  // query rows per workgroup
constexpr int kExtNoWindow = 1 << 30;     // a window bound that never binds
constexpr float kExtSlack = 2.f;          // lazy reference: moved when exceeded by > 2 (log2)

// Keys per LDS tile: 32 for d = 128 and 256 (32 KB for both stages of K and V at d = 128, so three
// workgroups share a CU), 64 for d = 64. On the causal Llama layer 32-key tiles ran at 1109 TFLOP/s
// against 1063 for 64-key tiles (one box, round-robin).
template <int D>
struct ExtTile {
  static constexpr int ROWS = D == 64 ? 64 : 32;
};

// Bias tile in LDS: the workgroup's 128 query rows x 64 keys (bf16, 128-byte rows), i.e. one or two
// K/V tiles, filled by DMA in two stages. Each tile is requested as soon as its stage is free --
// a whole bias tile ahead, up to two K/V tiles -- because the bias is read once from HBM, with no
// L2 reuse to shorten the latency. A step reads 8 bytes per lane (4 keys of its row) and the LDS
// serves such reads 32 lanes (one row each) at a time; chunk j of row R sits at slot j ^ g(R),
// which spreads those 32 rows over all 16 (bank line half, slot) pairs: 2 rows per bank pair, the
// least 32 rows of 8 bytes allow.
struct BiasTile {
  static constexpr int KEYS = 64;
  static constexpr int ROW = 2 * KEYS;    // bytes per row
  static constexpr int CPR = KEYS / 8;    // 16-byte chunks per row
  static constexpr int RPP = 1024 / ROW;  // rows per 1 KB DMA piece
  static constexpr int BYTES = kExtRows * ROW;
  static constexpr int PIECES = BYTES / 1024;
  static constexpr int PER_WAVE = PIECES / kExtWaves;
  __device__ static __forceinline__ int g(int r) { return (r >> 1) & (CPR - 1); }
};

__device__ __forceinline__ bf16x4 lds_read_b64(const char* p) {
  return *(const FA_LDS bf16x4*)(p);
}

struct ExtArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  const bf16* bias;      // optional additive bias (element strides below, columns contiguous)
  const float* slopes;   // optional ALiBi slope per query head
  long long bias_bs, bias_hs;
  int bias_rs;
  int N, H, Hkv, group, BH, n_qblk;
  int wl, wr;            // window bounds (kExtNoWindow when unbounded)
  float scale_log2;
  long long q_bs, q_hs, kv_bs, kv_hs;
  int q_rs, kv_rs;
};

// Two waves per SIMD at least, d = 256 included: its 64 Q-operand and 128 accumulator registers
// per lane fit in 256 VGPRs (with the halved lane offsets of fa_tiles.h), and the second wave is
// what hides one wave's softmax behind the other's MFMAs (1.7x over one wave per SIMD). With a
// bias the d = 256 kernel needs more and runs one wave per SIMD.
template <int D, bool CAUSAL, bool ALIBI, bool BIAS>
__global__ __launch_bounds__(kExtWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void fa_fwd_ext_kernel(ExtArgs a) {
  constexpr int DK = D / 16, DB = D / 32;
  constexpr int TK = ExtTile<D>::ROWS;
  // K-operand reads in flight ahead of the score MFMAs: three for plain d = 128 (+0.7-1.3% on the
  // causal and windowed Llama layers, the same 168 registers); none with ALiBi or a bias (the
  // extra registers cost the third wave per SIMD) or at d = 64 and 256 (no measured gain).
  constexpr int K_AHEAD = D == 128 && !ALIBI && !BIAS ? 3 : 0;
  using S = Swz<D>;
  __shared__ __attribute__((aligned(1024))) char sK2[2][S::template bytes<TK>()];
  __shared__ __attribute__((aligned(1024))) char sV2[2][S::template bytes<TK>()];
  using BT = BiasTile;
  constexpr int TPB = BT::KEYS / TK;  // K/V tiles per bias tile
  __shared__ __attribute__((aligned(1024))) char sB2[2][BIAS ? BT::BYTES : 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h = lane >> 5;
  race_check_poison<sizeof(sK2)>(sK2, tid, kExtWaves * 64);
  race_check_poison<sizeof(sV2)>(sV2, tid, kExtWaves * 64);
  race_check_poison<sizeof(sB2)>(sB2, tid, kExtWaves * 64);
  race_check_barrier();
  int bh, qblk;
  map_block<CAUSAL>(blockIdx.x, gridDim.x, a.BH, a.n_qblk, bh, qblk);
  const int b = bh / a.H, hq = bh - b * a.H, hk = hq / a.group;
  const int N = a.N;
  const int bq0 = qblk * kExtRows, bq1 = min(N - 1, bq0 + kExtRows - 1);  // workgroup rows
  const int wq0 = bq0 + 32 * wave, wq1 = wq0 + 31;                        // wave rows
  const int qrow = wq0 + c;
  const long long qoff = b * a.q_bs + hq * a.q_hs + (long long)qrow * a.q_rs;
  const long long kvhead = b * a.kv_bs + hk * a.kv_hs;
  const long long rs = 2LL * a.kv_rs;

  // Keys the workgroup / the wave can see: [lo, hi] from the window and the causal rule.
  auto key_lo = [&](int q0) { return max(0, q0 - a.wl); };
  auto key_hi = [&](int q1) {
    int x = min(N - 1, q1 + a.wr);
    return CAUSAL ? min(x, q1) : x;
  };
  const int blo = key_lo(bq0), bhi = key_hi(bq1);
  const int wlo = key_lo(wq0), whi = key_hi(min(wq1, N - 1));

  bf16x8 qf[DK];
#pragma unroll
  for (int dk = 0; dk < DK; dk++)
    qf[dk] = qrow < N ? *reinterpret_cast<const bf16x8*>(a.q + qoff + dk * 16 + h * 8) : bf16x8{};
  LaneOffsets<D> lo_;
  lo_.init(lane);
  float slope2 = 0.f;
  if constexpr (ALIBI) slope2 = a.slopes[hq] * kLog2e;
  // Causal ALiBi separates: every visible key has j <= i, so -m |i - j| = m (j - w0) - m (i - w0)
  // (w0 the wave's first row). Register r of a step holds key k0 + acc_row(r, h), so in log2 units
  // the score is fma(s, scale log2 e, C_r) + u with C_r = m log2(e) acc_row(r, 0) the same for
  // every lane (scalar registers) and u = m log2(e) (k0 - w0 + 4h - c) one value per lane and step,
  // which folds into the row maximum and the exponent's reference: one fma per score instead of
  // a subtract, an absolute value and an fma. (Without the causal rule keys on both sides of the
  // diagonal are visible and the absolute value stays; at d = 256 the 16 extra registers would
  // spill.) Masked scores are -inf either way.
  constexpr bool SEP = ALIBI && CAUSAL && D <= 128;
  float alibi_c[SEP ? 16 : 1];
  float alibi_lane = 0.f;
  if constexpr (SEP) {
#pragma unroll
    for (int i = 0; i < 16; i++)
      alibi_c[i] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                       __builtin_bit_cast(int, slope2 * (float)acc_row(i, 0))));
    alibi_lane = slope2 * (float)(4 * h - c);
  }
  // Bias: a buffer resource over rows bq0.. of this head's matrix (bytes past row N-1's key N-1
  // read as zeros), this lane's byte offset for each of its wave's DMA pieces (rows past N: an
  // offset past the resource), and the LDS offsets of its reads (row 32 wave + c, chunk j, keys
  // 4h..4h+3 of the chunk). Keys past N within a row are read but masked.
  i32x4v brs;
  unsigned bvo[BIAS ? BT::PER_WAVE : 1];
  int boff[BIAS ? BT::CPR : 1];
  if constexpr (BIAS) {
    const long long rsb = 2LL * a.bias_rs;
    const unsigned long long base = reinterpret_cast<unsigned long long>(
        a.bias + b * a.bias_bs + hq * a.bias_hs) + (unsigned long long)(bq0 * rsb);
    brs[0] = __builtin_amdgcn_readfirstlane((int)(base & 0xffffffffu));
    brs[1] = __builtin_amdgcn_readfirstlane((int)(base >> 32));
    brs[2] = __builtin_amdgcn_readfirstlane((int)(((long long)(N - 1 - bq0) * a.bias_rs + N) * 2));
    brs[3] = 0x00020000;
    const int rin = lane / BT::CPR, slot = lane % BT::CPR;
#pragma unroll
    for (int i = 0; i < BT::PER_WAVE; i++) {
      const int R = BT::RPP * (wave + kExtWaves * i) + rin;
      bvo[i] = bq0 + R < N ? (unsigned)(R * rsb) + 16u * (unsigned)(slot ^ BT::g(R)) : 0x80000000u;
    }
    const int R = 32 * wave + c;
#pragma unroll
    for (int j = 0; j < BT::CPR; j++) boff[j] = R * BT::ROW + 16 * (j ^ BT::g(R)) + 8 * h;
  }
  auto dma_bias = [&](char* tile, int k0) {
    const unsigned soff = __builtin_amdgcn_readfirstlane(2 * k0);
#pragma unroll
    for (int i = 0; i < BT::PER_WAVE; i++)
      dma16(tile + 1024 * (wave + kExtWaves * i), bvo[i], brs, soff);
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; db++) acc[db] = f32x16{};
  float m2 = -INFINITY, l = 0.f;

  const char* kh = reinterpret_cast<const char*>(a.k + kvhead);
  const char* vh = reinterpret_cast<const char*>(a.v + kvhead);
  const int t_first = blo / TK, t_last = bhi / TK;  // tiles with a key some row of the block sees
  // Causal ALiBi (without a bias) walks the tiles from the diagonal down: its term grows by
  // slope * 32 per step towards the diagonal, so in key order the row maximum, hence the lazy
  // reference, would move (and the accumulator be rescaled) on nearly every step of the heads with
  // large slopes; from the diagonal down it is set by the first steps and rarely moves again.
  constexpr bool DESC = CAUSAL && ALIBI && !BIAS;
  if (t_first <= t_last) {
    dma_tile<D, TK, kExtWaves>(sK2[0], kh, rs, (DESC ? t_last : t_first) * TK, N, wave, lane);
    dma_tile<D, TK, kExtWaves>(sV2[0], vh, rs, (DESC ? t_last : t_first) * TK, N, wave, lane);
    if constexpr (BIAS) dma_bias(sB2[0], t_first * TK);
    wait_dma();
    __syncthreads();
  }
  // Tile t sits in stage (t - t_first) % 2 (DESC: (t_last - t) % 2); the stage is a compile-time
  // constant of each copy of the loop body, so every LDS address is a per-lane offset plus an
  // immediate.
  auto tile = [&](auto stage_c, int t) {
    constexpr int st = decltype(stage_c)::value;
    const bool more = DESC ? t > t_first : t < t_last;  // a next tile: t - 1 (DESC) or t + 1
    if (more) {
      dma_tile<D, TK, kExtWaves>(sK2[st ^ 1], kh, rs, (DESC ? t - 1 : t + 1) * TK, N, wave, lane);
      dma_tile<D, TK, kExtWaves>(sV2[st ^ 1], vh, rs, (DESC ? t - 1 : t + 1) * TK, N, wave, lane);
    }
    // bias tile of K/V tiles t.. (if t starts one): stage bst; its first tile requests the next
    // bias tile into the other stage, after K/V so that the wait below can leave it in flight
    const int bst = ((t - t_first) / TPB) & 1;
    constexpr bool bias_first = TPB == 1 || st == 0;
    bool bias_issued = false;
    if constexpr (BIAS && bias_first) {
      if (t + TPB <= t_last) {
        dma_bias(sB2[bst ^ 1], (t + TPB) * TK);
        bias_issued = true;
      }
    }
    race_check_drain();
    const char* sK = sK2[st];
    const char* sV = sV2[st];
    const char* sB = sB2[bst];
    constexpr int bkey0 = TPB == 1 ? 0 : st * TK;  // this tile's first key within the bias tile
#pragma unroll
    for (int sbi = 0; sbi < TK / 32; sbi++) {
      const int sb = DESC ? TK / 32 - 1 - sbi : sbi;  // 32-key steps of the tile, in tile order
      const int k0 = t * TK + 32 * sb;
      // wave-uniform: no key of this step is visible to any row of the wave
      if (wq0 >= N || k0 > whi || k0 + 31 < wlo) continue;  // (continue: next sb)
      bf16x4 bcur[4];
      if constexpr (BIAS) {
#pragma unroll
        for (int j4 = 0; j4 < 4; j4++) bcur[j4] = lds_read_b64(sB + boff[bkey0 / 8 + 4 * sb + j4]);
      }
      f32x16 sc = f32x16{};
      if constexpr (K_AHEAD > 0) {
        // K operands read K_AHEAD MFMAs ahead: reads first, then one read per MFMA, then the last
        // MFMAs (left to itself the compiler waits for each read right before its MFMA)
        bf16x8 kf[DK];
#pragma unroll
        for (int dk = 0; dk < DK; dk++) kf[dk] = tile_row_at<D>(sK, lo_, 32 * sb, dk);
#pragma unroll
        for (int dk = 0; dk < DK; dk++) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[dk], qf[dk], sc, 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, K_AHEAD, 0);  // LDS reads
#pragma unroll
        for (int i = 0; i < DK - K_AHEAD; i++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, K_AHEAD, 0);
      } else {
#pragma unroll
        for (int dk = 0; dk < DK; dk++)
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_row_at<D>(sK, lo_, 32 * sb, dk), qf[dk], sc, 0, 0, 0);
      }
      // mask bounds: keys past N, past the causal diagonal or outside the window (only steps that
      // cross one of those bounds for some row of the wave); register i is key k0 + acc_row(i, h)
      const bool edge = k0 + 31 > min(N - 1, CAUSAL ? wq0 : N - 1) || k0 + 31 > wq0 + a.wr ||
                        k0 < wq1 - a.wl;
      const int lo = qrow - a.wl - k0 - 4 * h;  // visible iff lo <= acc_row(i, 0) <= hi
      const int hi = min(N - 1, min(CAUSAL ? qrow : N - 1, qrow + a.wr)) - k0 - 4 * h;
      float t2;                   // this step's row maximum in log2 units (-inf: nothing visible)
      float alibi_u = 0.f;        // SEP: the per-lane part of the ALiBi term (log2 units)
      float x[16];                // scores in log2 units, or raw scores (PLAIN)
      constexpr bool PLAIN = !ALIBI && !BIAS;
      if constexpr (PLAIN) {
        // raw scores: the maximum commutes with the positive scale, which is fused into the
        // exponent below
#pragma unroll
        for (int i = 0; i < 16; i++) x[i] = sc[i];
        if (edge) {  // wave-uniform: most steps cross no bound and skip the masks
#pragma unroll
          for (int i = 0; i < 16; i++)
            x[i] = (acc_row(i, 0) >= lo && acc_row(i, 0) <= hi) ? x[i] : -INFINITY;
        }
        t2 = half_swap_max(max16_arr(x)) * a.scale_log2;
      } else {
        // x = scale log2(e) s + log2(e) (B - m |i - j|)   (SEP: minus u, see above)
        const float dq = (float)(qrow - k0 - 4 * h);  // qrow - key = dq - acc_row(i, 0)
        if constexpr (SEP) alibi_u = __builtin_fmaf(slope2, (float)(k0 - wq0), alibi_lane);
#pragma unroll
        for (int i = 0; i < 16; i++) {
          float xi = SEP ? __builtin_fmaf(sc[i], a.scale_log2, alibi_c[i]) : sc[i] * a.scale_log2;
          if constexpr (BIAS) xi = __builtin_fmaf((float)bcur[i >> 2][i & 3], kLog2e, xi);
          if constexpr (ALIBI && !SEP) xi = __builtin_fmaf(-slope2, __builtin_fabsf(dq - (float)acc_row(i, 0)), xi);
          x[i] = xi;
        }
        if (edge) {
#pragma unroll
          for (int i = 0; i < 16; i++)
            x[i] = (acc_row(i, 0) >= lo && acc_row(i, 0) <= hi) ? x[i] : -INFINITY;
        }
        t2 = half_swap_max(max16_arr(x) + alibi_u);  // u differs between the row's two halves
      }
      // Running reference, moved only when a score exceeds it by more than kExtSlack (log2 units):
      // any reference gives the same softmax, and the accumulator rescale is skipped wave-wide
      // otherwise (p <= 2^kExtSlack). The -inf guard keeps rows that have seen nothing at 0.
      if (__any(t2 > m2 + kExtSlack)) {
        const float mn = __builtin_fmaxf(m2, t2);
        const float alpha = m2 == -INFINITY ? 0.f : fast_exp2(m2 - mn);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; db++) acc[db] *= alpha;
        m2 = mn;
      }
      const float ref = (m2 == -INFINITY ? 0.f : m2) - alibi_u;
      float p[16];
      bf16x8 pf[2];
#pragma unroll
      for (int i = 0; i < 16; i++) {
        p[i] = PLAIN ? fast_exp2(__builtin_fmaf(x[i], a.scale_log2, -ref)) : fast_exp2(x[i] - ref);
        pf[i >> 3][i & 7] = (bf16)p[i];
      }
      l += sum16(p);
#pragma unroll
      for (int ks = 0; ks < 2; ks++)
#pragma unroll
        for (int db = 0; db < DB; db++)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tile_tr_at<D>(sV, lo_, 32 * sb + 16 * ks, db),
                                                            pf[ks], acc[db], 0, 0, 0);
    }
    if (more) {
      // K/V of tile t + 1 are the oldest loads in flight; a bias tile requested in this tile may
      // stay in flight until the end of the next one (TPB = 2), by which its first tile is due
      if (TPB == 2 && bias_issued)
        wait_dma_but<BT::PER_WAVE>();
      else
        wait_dma();
      __syncthreads();
    }
  };
  if constexpr (DESC) {
    for (int t = t_last; t >= t_first; t -= 2) {
      tile(std::integral_constant<int, 0>{}, t);
      if (t - 1 >= t_first) tile(std::integral_constant<int, 1>{}, t - 1);
    }
  } else {
    for (int t = t_first; t <= t_last; t += 2) {
      tile(std::integral_constant<int, 0>{}, t);
      if (t + 1 <= t_last) tile(std::integral_constant<int, 1>{}, t + 1);
    }
  }

  const float lt = half_swap_sum(l);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if constexpr (ALIBI) {
    // stored straight from the accumulator: the staging below takes the ALiBi kernel past the
    // register count of three waves per SIMD (166 -> 189 at d = 128), which costs more than the
    // stores gain
    if (qrow < N) {
      bf16* orow = a.o + qoff;
#pragma unroll
      for (int db = 0; db < DB; db++)
#pragma unroll
        for (int g4 = 0; g4 < 4; g4++) {
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; e++) ov[e] = (bf16)(acc[db][4 * g4 + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * g4 + 4 * h) = ov;
        }
      if (h == 0) a.lse[(long long)bh * N + qrow] = lt > 0.f ? kLn2 * (m2 + fast_log2(lt)) : -INFINITY;
    }
  } else {
    // O goes out through LDS (the K/V stages, free once every wave is past the last tile): each
    // wave writes its 32 rows of bf16 O into a swizzled region of its own and reads them back as
    // whole rows, so a store instruction writes complete rows instead of 16 bytes of 32 rows.
    __syncthreads();
    constexpr int OREG = 32 * S::ROW;  // one wave's 32 rows
    static_assert(2 * OREG <= (int)sizeof(sK2) && 2 * OREG <= (int)sizeof(sV2), "O staging fits");
    char* const so = (wave < 2 ? &sK2[0][0] : &sV2[0][0]) + (wave & 1) * OREG;
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; e++) ov[e] = (bf16)(acc[db][4 * g4 + e] * inv);
        *(FA_LDS bf16x4*)((FA_LDS char*)so + S::off(c, 4 * db + g4) + 8 * h) = ov;
      }
    if (qrow < N && h == 0)
      a.lse[(long long)bh * N + qrow] = lt > 0.f ? kLn2 * (m2 + fast_log2(lt)) : -INFINITY;
    constexpr int RPI = 64 / S::CPR;  // rows per read instruction
#pragma unroll
    for (int it = 0; it < 32 / RPI; it++) {
      const int r = RPI * it + lane / S::CPR, j = lane % S::CPR;
      const bf16x8 ov = *(const FA_LDS bf16x8*)((FA_LDS char*)so + S::off(r, j));
      const int row = wq0 + r;
      if (row < N)
        *reinterpret_cast<bf16x8*>(a.o + b * a.q_bs + hq * a.q_hs + (long long)row * a.q_rs + 8 * j) = ov;
    }
  }
}

}  // namespace fa
