// Wide-row forward kernel for gfx950, head dim 128: the bench workload (causal Llama-3-8B layer),
// the other large d = 128 grids, and causal sliding windows or causal ALiBi on them (the choice is
// made in fa_api.hip).
//
// The method is the one of the other forward kernels ("FlashAttention-2 -- Deeper Math", Fixes
// 1-5 and "Causal masking: skip the blocks"; "Understanding FlashAttention Pt 1", §2.4 and §3.1):
// per query row a reference maximum m, a running sum l and an unnormalised accumulator a, updated
// key tile by key tile as
//     m' = max(m, rowmax(S)),  alpha = 2^(m - m'),  p = 2^(s - m'),  l' = alpha l + sum p,
//     a' = alpha a + p V,
// with O = a / l and LSE = m + log l (natural-log units on output) written once at the end. The
// reference moves lazily (only when a score exceeds it by more than kWideSlack in log2 units,
// as in the other kernels), with the -inf guard of "Online Softmax & FlashAttention", Listing
// 26.3 for rows that have seen no key yet.
//
// What is different here is the shape of the work per wave and the instruction stream.
//   * A wave owns 64 query rows as two independent 32-row blocks A and B (a workgroup is 4 waves,
//     256 rows, one wave per SIMD: about 370 registers per lane). Every K and V operand fragment
//     read from LDS feeds one MFMA of each block, so a wave reads 0.5 KB of LDS per 32x32x16 MFMA
//     instead of 1 KB, and the workgroup refills its K/V tiles from L2 half as often per query
//     row as a 128-row one.
//   * With one wave per SIMD nothing else fills the matrix core while the wave does vector work,
//     so the two blocks are software-pipelined half a step apart and every phase pairs 8 MFMAs of
//     one block with the vector work of the other. Step j is four phases:
//         P1  S_B(j)   = K(j) Q_B^T         | A, step j: exponentials, bf16 P, pair sums
//         P2  O_A     += V(j)^T P_A(j)^T    | A's row sum; B, step j: shifted scores, maximum
//         P3  S_A(j+1) = K(j+1) Q_A^T       | B, step j: exponentials, bf16 P, pair sums
//         P4  O_B     += V(j)^T P_B(j)^T    | B's row sum; A, step j+1: shifted scores, maximum
//     Each phase is written as 8 groups of one MFMA and the vector instructions that fit in its
//     32 cycles, pinned in place (see pin()). K(j+1) is read from LDS in P2, V(j+1) in P4 (into
//     the second of two V fragment sets, so that no phase waits for V it has just requested).
//   * Exponentials are taken relative to the current reference; the check that moves it (some
//     shifted score above the slack, or the row's first visible score) follows the shift, so the
//     rare rescale of the accumulator is a wave-uniform branch between phases, before the
//     exponentials it affects; so are the masks of the steps that cross the causal diagonal or
//     the end of the sequence.
//   * K/V tiles of 64 keys (two steps) go straight from memory into two swizzled LDS stages by
//     16-byte DMA, one barrier per tile, between P1 and P2 of its second step: the last read of
//     tile t (V of its second step, P4 of its first step) precedes it and the first reads of tile
//     t+1 (K of the next step, P2; V of the next step, P4) follow it. The DMA pieces of tile t+2
//     are issued one per MFMA group of that P2. The epilogue stores O through LDS as whole rows.
//   * With a causal sliding window (row q sees keys q - wl .. q) a workgroup starts at the tile of
//     its first row's first key; the steps before a block's window are masked like those past its
//     diagonal (the waves above the first row run through a few fully masked steps first).
//   * With causal ALiBi the key tiles are walked from the diagonal down (tile n_tiles - 1 first,
//     the steps of a tile from its last to its first, tile t in stage t % 2): the ALiBi term falls
//     away from the diagonal, so the first steps set the lazy reference and it seldom moves again.
//     The waves whose diagonal lies below the workgroup's last tile meet those tiles' barriers
//     first, and each block's step after its last one (keys below 0) is hidden.
//   * Every wave takes part in every tile of its workgroup's key range, so the barrier counts
//     match. The steps past a block's causal diagonal (or past N) are fully masked, which makes
//     their probabilities 0 and leaves the running state unchanged; once a whole tile is past both
//     of a wave's blocks, the wave only meets the tile's barrier and issues its loads.
#pragma once

#include "fa_tiles.h"

namespace fa {

constexpr int kWideWaves = 4;
constexpr int kWideRows = 64 * kWideWaves;  // query rows per workgroup
constexpr int kWideSlack = 2;               // lazy reference: moved when exceeded by > 2 (log2)
constexpr int kWideTK = 64;                 // keys per LDS tile (two 32-key steps)
constexpr int kWideStages = 2;              // LDS stages of the K/V tile ring
constexpr int kWideNoWindow = 1 << 30;      // WideArgs::wl when there is no sliding window

struct WideArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  const float* slopes;  // ALiBi slopes, one per query head (the ALiBi instantiation)
  int wl;  // causal sliding window (the window instantiation): row q sees keys q - wl .. q
  int N, H, group, BH, n_qblk;
  float scale_log2;
  long long q_bs, q_hs, kv_bs, kv_hs;
  int q_rs, kv_rs;
};

// Running state of one 32-row block: lane (c, h) holds query row row0 + c and, per step, 16 of its
// keys (register i: key k0 + acc_row(i, h)).
struct WideBlock {
  bf16x8 q[8];   // Q^T operand, d = 128 in 8 k-steps of 16
  f32x16 o[4];   // O^T accumulator, 4 blocks of 32 columns
  f32x16 x;      // S^T of the step: raw q.k from the MFMAs, then s scale log2(e) - ref
  bf16x8 pb[2];  // probabilities 2^x of the step rounded to bf16: the P^T operand (two k-steps)
  float t[8];    // pair sums of the fp32 probabilities, added into l in the next phase
  float xmax;    // this lane's maximum of x
  float thr;     // x above it moves the reference: the slack, or -inf while m2 is -inf
  float m2;      // reference (log2 units), -inf before any visible key
  float ref;     // exponent reference: m2, or 0 while m2 is -inf
  float l;       // this lane's part of the row sum
};

__device__ __forceinline__ float wide_max16(const f32x16& v) {
  const float a = max3(v[0], v[1], v[2]), b = max3(v[3], v[4], v[5]);
  const float c = max3(v[6], v[7], v[8]), d = max3(v[9], v[10], v[11]);
  const float e = max3(v[12], v[13], v[14]);
  return __builtin_fmaxf(max3(a, b, c), max3(d, e, v[15]));
}

// For a step whose keys (from k0) may pass the last key `last_key` of the lane's row (the causal
// diagonal, the end of the sequence, the padding steps past both) or, with a sliding window, lie
// before its first key: those keys become -inf, and the maximum is taken again. Rare; wave-uniform
// branch.
template <bool WINDOW>
__device__ __forceinline__ void wide_mask(WideBlock& x, int k0, int last_key, int first_key, int h) {
  const int hi = last_key - k0 - 4 * h;
  const int lo = first_key - k0 - 4 * h;  // (window) keys before first_key are hidden as well
#pragma unroll
  for (int i = 0; i < 16; i++)
    x.x[i] = acc_row(i, 0) <= hi && (!WINDOW || acc_row(i, 0) >= lo) ? x.x[i] : -INFINITY;
  x.xmax = wide_max16(x.x);
}

// The reference of the rows moves to their exact maximum (the accumulator and sum rescaled by
// 2^(m_old - m_new)) when some lane of the wave has a score above its threshold: the slack, or any
// visible score while the row has seen none (the -inf guard). Rare; wave-uniform branch, kept out
// of the straight-line step.
__device__ __forceinline__ void wide_fix(WideBlock& x) {
  const float t2 = half_swap_max(x.xmax) + x.ref;  // row maximum in log2 units, -inf if none
  const float mn = __builtin_fmaxf(x.m2, t2);
  const float alpha = x.m2 == -INFINITY ? 0.f : fast_exp2(x.m2 - mn);
  x.l *= alpha;
#pragma unroll
  for (int db = 0; db < 4; db++) x.o[db] *= alpha;
  x.m2 = mn;
  const float nref = mn == -INFINITY ? 0.f : mn;
  const float delta = nref - x.ref;
  x.ref = nref;
  x.thr = mn == -INFINITY ? -INFINITY : (float)kWideSlack;
#pragma unroll
  for (int i = 0; i < 16; i++) x.x[i] -= delta;
}

// The step after a block's last one, when the keys run from the diagonal down (its keys would be
// negative): every score hidden.
__device__ __forceinline__ void wide_mask_all(WideBlock& x) {
#pragma unroll
  for (int i = 0; i < 16; i++) x.x[i] = -INFINITY;
  x.xmax = -INFINITY;
}

__device__ __forceinline__ void wide_check(WideBlock& x) {
  if (__builtin_expect(__any(x.xmax > x.thr), 0)) wide_fix(x);
}

// Instruction order. A wave is alone on its SIMD, so the order of its instructions decides how
// much vector work runs under the matrix core's MFMAs. Each phase is written as 8 groups of one
// MFMA and the vector instructions that fit in its 32 cycles, each value pinned in its group and
// the group closed by a scheduling barrier (pin() and fence(), fa_device.h).

// Exponential phase: S_Y = K Q_Y^T (a chain of 8 MFMAs) with the probabilities of block X: per
// group two exponentials, and the bf16 packing and pair sum of the previous group's two. load(i)
// issues the LDS reads that belong to group i.
template <bool ALIBI, class Load>
__device__ __forceinline__ void phase_exp(WideBlock& Y, const bf16x8 (&kf)[8], WideBlock& X,
                                          const f32x16& s_init, Load&& load) {
  f32x16 s;
  if constexpr (ALIBI) s = s_init;  // the per-register part of the ALiBi term, over the scale
  else s = f32x16{};
  float e[16];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], Y.q[i], s, 0, 0, 0);
    pin(s);
    load(i);
    e[2 * i] = fast_exp2(X.x[2 * i]);
    e[2 * i + 1] = fast_exp2(X.x[2 * i + 1]);
    pin(e[2 * i]);
    pin(e[2 * i + 1]);
    if (i > 0) {
      const int k = 2 * (i - 1);
      X.pb[k >> 3][k & 7] = (bf16)e[k];
      X.pb[k >> 3][(k & 7) + 1] = (bf16)e[k + 1];
      X.t[i - 1] = e[k] + e[k + 1];
      pin(X.pb[k >> 3]);
      pin(X.t[i - 1]);
    }
    fence();
  }
  X.pb[1][6] = (bf16)e[14];
  X.pb[1][7] = (bf16)e[15];
  X.t[7] = e[14] + e[15];
  pin(X.pb[1]);
  pin(X.t[7]);
  Y.x = s;
}

// Shift phase: O_X += V^T P_X^T (8 MFMAs on 4 accumulators) with X's row-sum update and block Y's
// scores moved to log2 units relative to its reference, x = s scale log2(e) - ref, and their
// maximum (the rare reference move and the masks follow the phase).
template <bool ALIBI, class Load>
__device__ __forceinline__ void phase_pv(WideBlock& X, const bf16x8 (&vf)[4][2], WideBlock& Y,
                                         float scale_log2, float yadd, Load&& load) {
  float m1 = 0.f, m2 = 0.f, m3 = 0.f;
  float* t = X.t;
  // ALiBi: yadd = the step's part of the ALiBi term minus the reference
  auto sh = [&](int i) {
    if constexpr (ALIBI) Y.x[i] = __builtin_fmaf(Y.x[i], scale_log2, yadd);
    else Y.x[i] = __builtin_fmaf(Y.x[i], scale_log2, -Y.ref);
    pin(Y.x[i]);
  };
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int ks = i >> 2, db = i & 3;
    X.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][ks], X.pb[ks], X.o[db], 0, 0, 0);
    pin(X.o[db]);
    load(i);
    switch (i) {
      case 0:
        t[0] += t[1]; t[2] += t[3]; t[4] += t[5]; t[6] += t[7];
        pin(t[0]); pin(t[2]); pin(t[4]); pin(t[6]);
        break;
      case 1:
        t[0] += t[2]; t[4] += t[6];
        pin(t[0]); pin(t[4]);
        sh(0); sh(1);
        break;
      case 2:
        X.l += t[0] + t[4];
        pin(X.l);
        sh(2); sh(3);
        break;
      case 3:
        sh(4); sh(5);
        m1 = max3(Y.x[0], Y.x[1], Y.x[2]);
        pin(m1);
        break;
      case 4:
        sh(6); sh(7);
        m2 = max3(Y.x[3], Y.x[4], Y.x[5]);
        pin(m2);
        break;
      case 5:
        sh(8); sh(9);
        m3 = max3(Y.x[6], Y.x[7], Y.x[8]);
        pin(m3);
        break;
      case 6:
        sh(10); sh(11); sh(12);
        m1 = max3(m1, Y.x[9], Y.x[10]);
        pin(m1);
        break;
      default:
        sh(13); sh(14); sh(15);
        m2 = max3(m2, Y.x[11], Y.x[12]);
        m3 = max3(m3, Y.x[13], Y.x[14]);
        pin(m2);
        pin(m3);
        break;
    }
    fence();
  }
  Y.xmax = __builtin_fmaxf(max3(m1, m2, m3), Y.x[15]);
}

// A wave's share of one K or V tile (TK rows of 256 bytes, swizzled as in fa_tiles.h): PW 1 KB
// pieces, piece p = wave + 4 i at LDS offset 1 KB p, each lane fetching the 16-byte chunk that
// belongs at its slot. The per-lane byte offsets within the tile's rows are computed once, and so
// are the pieces' LDS addresses (scalar registers, for M0); per tile only the buffer resource
// moves, in scalar arithmetic. The pieces are issued one per MFMA group of a shift phase.
template <int TK, int NS>
struct WideDma {
  static constexpr int PW = TK * 256 / 1024 / kWideWaves;  // pieces per wave (4 or 8)
  unsigned voff[PW];
  unsigned lds[NS][2][PW];  // M0 of each piece: stage, K or V, piece
  __device__ __forceinline__ void init(int wave, int lane, long long rs, char (*sK)[TK * 256],
                                       char (*sV)[TK * 256]) {
    const int rin = lane / 16, slot = lane % 16;
#pragma unroll
    for (int i = 0; i < PW; i++) {
      const int r = 4 * (wave + kWideWaves * i) + rin;
      voff[i] = (unsigned)(r * rs) + 16u * (unsigned)(slot ^ Swz<128>::f(r));
#pragma unroll
      for (int st = 0; st < NS; st++) {
        lds[st][0][i] = __builtin_amdgcn_readfirstlane(
            (int)(unsigned)(size_t)(FA_LDS char*)(sK[st] + 1024 * (wave + kWideWaves * i)));
        lds[st][1][i] = __builtin_amdgcn_readfirstlane(
            (int)(unsigned)(size_t)(FA_LDS char*)(sV[st] + 1024 * (wave + kWideWaves * i)));
      }
    }
  }
  // piece i of K (kv = 0) or V (kv = 1) into stage st. The s_nop covers the two wait states a VMEM
  // instruction needs after a VALU write of an SGPR it reads, which the compiler does not check
  // inside inline assembly (the operands here are written by scalar instructions in the loop).
  __device__ __forceinline__ void piece(int st, int kv, int i, const i32x4v& rsrc) const {
    asm volatile("s_nop 1\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 ::"v"(voff[i]), "s"(lds[st][kv][i]), "s"(rsrc)
                 : "memory", "m0");
  }
};

template <bool CAUSAL, bool WINDOW, bool ALIBI>
__global__ __launch_bounds__(kWideWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void fa_fwd_wide_kernel(WideArgs a) {
  static_assert(CAUSAL || !WINDOW, "the sliding window is the causal one (keys q - wl .. q)");
  static_assert(!ALIBI || (CAUSAL && !WINDOW), "ALiBi: causal, without a window");
  // ALiBi walks the key tiles from the diagonal down (see the ALiBi note below)
  constexpr bool DESC = ALIBI;
  constexpr int D = 128, DK = 8, DB = 4, TK = kWideTK, SPT = TK / 32;  // steps per tile
  using S = Swz<D>;
  constexpr int TILE = S::template bytes<TK>();
  constexpr int NS = kWideStages;
  __shared__ __attribute__((aligned(1024))) char sK[NS][TILE];
  __shared__ __attribute__((aligned(1024))) char sV[NS][TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h = lane >> 5;
  race_check_poison<NS * TILE>(sK, tid, kWideWaves * 64);
  race_check_poison<NS * TILE>(sV, tid, kWideWaves * 64);
  race_check_barrier();
  int bh, qblk;
  map_block<CAUSAL>(blockIdx.x, gridDim.x, a.BH, a.n_qblk, bh, qblk);
  const int b = bh / a.H, hq = bh - b * a.H, hk = hq / a.group;
  const int N = a.N;
  const float sl2 = a.scale_log2;
  const int bq0 = qblk * kWideRows, bq1 = min(N - 1, bq0 + kWideRows - 1);
  const int ra = bq0 + 64 * wave, rb = ra + 32;  // first rows of blocks A and B
  const long long qh = b * a.q_bs + hq * a.q_hs;
  const long long kvhead = b * a.kv_bs + hk * a.kv_hs;
  const long long rs = 2LL * a.kv_rs;

  WideBlock A, B;
  {
    const int qa = ra + c, qb = rb + c;
#pragma unroll
    for (int dk = 0; dk < DK; dk++) {
      A.q[dk] = qa < N ? *reinterpret_cast<const bf16x8*>(a.q + qh + (long long)qa * a.q_rs + dk * 16 + h * 8) : bf16x8{};
      B.q[dk] = qb < N ? *reinterpret_cast<const bf16x8*>(a.q + qh + (long long)qb * a.q_rs + dk * 16 + h * 8) : bf16x8{};
    }
  }
#pragma unroll
  for (int db = 0; db < DB; db++) A.o[db] = B.o[db] = f32x16{};
  A.m2 = B.m2 = A.thr = B.thr = -INFINITY;
  A.ref = B.ref = 0.f;

  A.l = B.l = 0.f;
  // ALiBi (causal): the score of row r0 + c (block from r0) and key k0 + acc_row(i, h) (register
  // i of a step from k0) gains -slope (q - k) = slope (k0 - r0) - slope c + slope acc_row(i, h).
  // The last part depends only on the register: it seeds the score MFMAs' accumulator, divided by
  // the scale (aini); the rest is added with the reference once per step, in log2 units
  // u = slope log2(e) (k0 - r0) + alane, every term small near the diagonal. The term grows by
  // 32 slope log2(e) per step towards the diagonal, so in key order the row maximum, and with it
  // the lazy reference, would move on nearly every step of the heads with large slopes; the keys
  // are walked from the diagonal down instead, where the first steps set the reference.
  f32x16 aini = f32x16{};
  float slope2 = 0.f, alane = 0.f;
  if constexpr (ALIBI) {
    slope2 = a.slopes[hq] * kLog2e;
    const float per_key = slope2 / sl2;
#pragma unroll
    for (int i = 0; i < 16; i++) aini[i] = per_key * (float)acc_row(i, h);
    alane = -slope2 * (float)c;
  }
  auto yadd = [&](const WideBlock& x, int k0, int r0) __attribute__((always_inline)) {
    return ALIBI ? __builtin_fmaf(slope2, (float)(k0 - r0), alane) - x.ref : 0.f;
  };
  // The last key each lane's row sees; a step whose last key passes the last key of its block's
  // first row needs a mask (wave-uniform): in key order the block's last steps, from the diagonal
  // down its first ones.
  const int lastA = min(N - 1, CAUSAL ? ra + c : N - 1), lastB = min(N - 1, CAUSAL ? rb + c : N - 1);
  const int edgeA = min(N - 1, CAUSAL ? ra : N - 1), edgeB = min(N - 1, CAUSAL ? rb : N - 1);
  // Sliding window: the first key of each lane's row, and the last first key of each block (a step
  // starting before it needs the lower mask). The workgroup starts at the tile of its first row's
  // first key; the waves above it run through a few fully masked steps first.
  const int wl = WINDOW ? a.wl : 0;
  const int firstA = ra + c - wl, firstB = rb + c - wl;
  const int ledgeA = ra + 31 - wl, ledgeB = rb + 31 - wl;

  LaneOffsets<D> lo_;
  lo_.init(lane);
  WideDma<TK, NS> dma;
  dma.init(wave, lane, rs, sK, sV);
  const char* kh = reinterpret_cast<const char*>(a.k + kvhead);
  const char* vh = reinterpret_cast<const char*>(a.v + kvhead);
  const int n_tiles = (CAUSAL ? bq1 : N - 1) / TK + 1;
  const int t_lo = WINDOW ? max(0, bq0 - wl) / TK : 0;  // first tile
  // buffer resources over rows t TK .. min(N, (t + 1) TK) - 1 of K and V (bytes past read as 0;
  // none for tiles past N, whose loads then only write zeros to a stage nothing reads again)
  auto tile_rsrc2 = [&](int t, i32x4v& rk, i32x4v& rv) __attribute__((always_inline)) {
    // (DESC: the tiles "after" tile 0 have negative numbers: empty resources, no memory touched)
    const int row0 = DESC && t < 0 ? 0 : t * TK;
    const int rows = DESC && t < 0 ? 0 : min(N - row0, TK);
    const unsigned long long off = (unsigned long long)row0 * (unsigned long long)rs;
    const unsigned long long bk = reinterpret_cast<unsigned long long>(kh) + off;
    const unsigned long long bv = reinterpret_cast<unsigned long long>(vh) + off;
    rk[0] = (int)(bk & 0xffffffffu);
    rk[1] = (int)(bk >> 32);
    rv[0] = (int)(bv & 0xffffffffu);
    rv[1] = (int)(bv >> 32);
    rk[2] = rv[2] = rows > 0 ? (int)((rows - 1) * rs) + 2 * D : 0;
    rk[3] = rv[3] = 0x00020000;
  };
  auto issue_tile = [&](int t, int st) __attribute__((always_inline)) {
    i32x4v rk, rv;
    tile_rsrc2(t, rk, rv);
#pragma unroll
    for (int i = 0; i < WideDma<TK, NS>::PW; i++) dma.piece(st, 0, i, rk);
#pragma unroll
    for (int i = 0; i < WideDma<TK, NS>::PW; i++) dma.piece(st, 1, i, rv);
  };

  bf16x8 kf[DK];
  bf16x8 vf[DB][2];
  bf16x8 vf2[DB][2];  // V fragments of odd steps (vf: even steps), each read in P4 of the step before
  auto load_k = [&](const char* tile, int r) __attribute__((always_inline)) {
#pragma unroll
    for (int dk = 0; dk < DK; dk++) kf[dk] = tile_row_at<D>(tile, lo_, r, dk);
  };

  // Tiles past the last key any row of this wave sees (the causal diagonal of its block B, or N)
  // are fully masked for both blocks and change nothing: the wave only takes part in their barrier
  // and loads. n_real is wave-uniform; every wave still meets one barrier per tile.
  const int last_seen = min(N - 1, CAUSAL ? rb + 31 : N - 1);
  const int n_real = min(n_tiles, last_seen / TK + 1);

  // prologue: the first two tiles requested, the first awaited. In key order tile t sits in stage
  // (t - t_lo) % 2; from the diagonal down (tiles n_tiles - 1 .. 0) tile t sits in stage t % 2.
  {
    const int t0 = DESC ? n_tiles - 1 : t_lo;
    const bool two = DESC ? t0 >= 1 : t0 + 1 < n_tiles;
    // (the pieces' LDS addresses are scalar operands: one branch per stage)
    auto issue_in = [&](int t, int st) __attribute__((always_inline)) {
      if (st) issue_tile(t, 1);
      else issue_tile(t, 0);
    };
    if constexpr (DESC) issue_in(t0, t0 & 1);
    else issue_tile(t0, 0);
    if (two) {
      if constexpr (DESC) issue_in(t0 - 1, (t0 - 1) & 1);
      else issue_tile(t0 + 1, 1);
      wait_dma_but<2 * WideDma<TK, NS>::PW>();
    } else {
      wait_dma();
    }
  }
  race_check_drain();
  __syncthreads();
  // S_A of the wave's first step (key order: the first step of tile t_lo, in stage 0; from the
  // diagonal down: the last step of its last real tile), shifted and checked
  auto first_step = [&](int st, int k0) __attribute__((always_inline)) {
    const int r0 = DESC ? 32 * (SPT - 1) : 0;
    load_k(sK[st], r0);
    auto& v0 = DESC && (SPT - 1) % 2 ? vf2 : vf;  // the V fragment set of that step's parity
#pragma unroll
    for (int i = 0; i < 8; i++) v0[i & 3][i >> 2] = tile_tr_at<D>(sV[st], lo_, r0 + 16 * (i >> 2), i & 3);
    f32x16 s0 = ALIBI ? aini : f32x16{};
#pragma unroll
    for (int dk = 0; dk < DK; dk++) s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[dk], A.q[dk], s0, 0, 0, 0);
    const float ya = ALIBI ? yadd(A, k0, ra) : -A.ref;
#pragma unroll
    for (int i = 0; i < 16; i++) A.x[i] = __builtin_fmaf(s0[i], sl2, ya);
    A.xmax = wide_max16(A.x);
    if (k0 + 31 > edgeA || (WINDOW && k0 < ledgeA)) wide_mask<WINDOW>(A, k0, lastA, firstA, h);
    wide_check(A);
  };
  if constexpr (!DESC) first_step(0, t_lo * TK);

  // Step j (sub-step sb of tile t, in stage st): the four phases of the header comment.
  auto step = [&](auto st_c, auto sb_c, int t) __attribute__((always_inline)) {
    constexpr int st = decltype(st_c)::value, sb = decltype(sb_c)::value;
    const int k0 = t * TK + 32 * sb;
    const int kn = DESC ? k0 - 32 : k0 + 32;        // first key of step j + 1
    constexpr bool LAST = sb == (DESC ? 0 : SPT - 1);  // last step of tile t
    constexpr int rn = DESC ? 32 * (sb - 1) : 32 * (sb + 1);  // rows of step j + 1 in tile t
    constexpr int rn1 = DESC ? 32 * (SPT - 1) : 0;             // and in the tile after t
    auto& vcur = (sb & 1) ? vf2 : vf;
    auto& vnext = (sb & 1) ? vf : vf2;
    // P1: S_B(j) = K(j) Q_B^T; probabilities of A, step j
    phase_exp<ALIBI>(B, kf, A, aini, [](int) {});
    i32x4v rk, rv;
    if constexpr (LAST) {
      // the next tile in LDS for every wave (each waits for its own pieces, then the barrier)
      wait_dma();
      __syncthreads();  // also: every wave's reads of tile t, whose stage is refilled below, done
      tile_rsrc2(DESC ? t - 2 : t + 2, rk, rv);
    }
    // P2: K(j+1) requested (and, in a tile's last step, the DMA of the tile after the next); O_A
    // += V(j)^T P_A(j)^T, A's sum; B's scores shifted and checked
    const float yb = yadd(B, k0, rb);
    phase_pv<ALIBI>(A, vcur, B, sl2, yb, [&](int i) __attribute__((always_inline)) {
      if constexpr (LAST) kf[i] = tile_row_at<D>(sK[st ^ 1], lo_, rn1, i);
      else kf[i] = tile_row_at<D>(sK[st], lo_, rn, i);
      if constexpr (LAST) {
        constexpr int PW = WideDma<TK, NS>::PW, PG = 2 * PW / 8;  // pieces per group
#pragma unroll
        for (int u = 0; u < PG; u++) {
          const int pc = PG * i + u;
          if (pc < PW) dma.piece(st, 0, pc, rk);
          else dma.piece(st, 1, pc - PW, rv);
        }
      }
    });
    if constexpr (LAST) race_check_drain();
    if (__builtin_expect(k0 + 31 > edgeB || (WINDOW && k0 < ledgeB), 0))
      wide_mask<WINDOW>(B, k0, lastB, firstB, h);
    wide_check(B);
    // P3: S_A(j+1) = K(j+1) Q_A^T; probabilities of B, step j
    phase_exp<ALIBI>(A, kf, B, aini, [](int) {});
    // P4: O_B += V(j)^T P_B(j)^T, B's sum; A's scores of step j + 1 shifted and checked (past the
    // last step: garbage, fully masked)
    const float ya = yadd(A, kn, ra);
    phase_pv<ALIBI>(B, vcur, A, sl2, ya, [&](int i) __attribute__((always_inline)) {
      // V(j+1): the next step of this tile, or the first of the next tile (visible since this
      // step's barrier; past the last tile the reads see a stage nothing uses)
      if constexpr (LAST) vnext[i & 3][i >> 2] = tile_tr_at<D>(sV[st ^ 1], lo_, rn1 + 16 * (i >> 2), i & 3);
      else vnext[i & 3][i >> 2] = tile_tr_at<D>(sV[st], lo_, rn + 16 * (i >> 2), i & 3);
    });
    if (__builtin_expect(kn + 31 > edgeA || (WINDOW && kn < ledgeA), 0))
      wide_mask<WINDOW>(A, kn, lastA, firstA, h);
    // from the diagonal down, the step after a block's last (keys -32 .. -1, read from a stage of
    // zeros) is not past the diagonal: hidden here
    if constexpr (DESC && LAST)
      if (t == 0) wide_mask_all(A);
    wide_check(A);
  };
  auto run_tile = [&](auto st_c, int tt) __attribute__((always_inline)) {
    auto one = [&](auto sb_c) __attribute__((always_inline)) { step(st_c, sb_c, tt); };
    if constexpr (DESC) {
      if constexpr (SPT == 4) {
        one(std::integral_constant<int, 3>{});
        one(std::integral_constant<int, 2>{});
      }
      one(std::integral_constant<int, 1>{});
      one(std::integral_constant<int, 0>{});
    } else {
      one(std::integral_constant<int, 0>{});
      one(std::integral_constant<int, 1>{});
      if constexpr (SPT == 4) {
        one(std::integral_constant<int, 2>{});
        one(std::integral_constant<int, 3>{});
      }
    }
  };
  auto idle_tile = [&](auto st_c, int tt) __attribute__((always_inline)) {
    constexpr int st = decltype(st_c)::value;
    wait_dma();
    __syncthreads();
    i32x4v rk, rv;
    tile_rsrc2(DESC ? tt - 2 : tt + 2, rk, rv);
#pragma unroll
    for (int i = 0; i < WideDma<TK, NS>::PW; i++) dma.piece(st, 0, i, rk);
#pragma unroll
    for (int i = 0; i < WideDma<TK, NS>::PW; i++) dma.piece(st, 1, i, rv);
    race_check_drain();
  };
  if constexpr (DESC) {
    // tiles n_tiles - 1 .. n_real: idle; then the real ones down to tile 0 (in stage 0), in pairs
    // from the bottom
    int t = n_tiles - 1;
    for (; t >= n_real; t--) {
      if (t & 1) idle_tile(std::integral_constant<int, 1>{}, t);
      else idle_tile(std::integral_constant<int, 0>{}, t);
    }
    first_step(t & 1, t * TK + 32 * (SPT - 1));
    if ((t & 1) == 0) {
      run_tile(std::integral_constant<int, 0>{}, t);
      t--;
    }
    for (; t >= 1; t -= 2) {
      run_tile(std::integral_constant<int, 1>{}, t);
      run_tile(std::integral_constant<int, 0>{}, t - 1);
    }
  } else {
    int t = t_lo;  // tile t sits in stage (t - t_lo) % 2
    for (; t + 1 < n_real; t += 2) {
      run_tile(std::integral_constant<int, 0>{}, t);
      run_tile(std::integral_constant<int, 1>{}, t + 1);
    }
    if (t < n_real) {
      run_tile(std::integral_constant<int, 0>{}, t);
      t++;
    }
    for (; t < n_tiles; t++) {
      if ((t - t_lo) & 1) idle_tile(std::integral_constant<int, 1>{}, t);
      else idle_tile(std::integral_constant<int, 0>{}, t);
    }
  }

  // epilogue: O = a / l, LSE = ln 2 (m + log2 l). O goes out through LDS, whose K/V stages are
  // free once every wave is past its last tile: each wave writes its 64 rows of bf16 O into a
  // swizzled 16 KB region (the tile layout of the K/V stages) and reads them back as whole
  // 256-byte rows, so every store instruction writes 4 complete rows instead of 16 bytes of each
  // of 32 rows. The loads of the two tiles past the last one (zero-size: they only write zeros
  // into the stages) may still be in flight; they land before the barrier.
  wait_dma();
  __syncthreads();
  char* const so = (wave < 2 ? &sK[0][0] : &sV[0][0]) + (wave & 1) * (64 * 256);
  auto stage_out = [&](WideBlock& x, int r0) __attribute__((always_inline)) {
    const float lt = half_swap_sum(x.l);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int r = r0 + c;
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; e++) ov[e] = (bf16)(x.o[db][4 * g4 + e] * inv);
        *(FA_LDS bf16x4*)((FA_LDS char*)so + S::off(r, 4 * db + g4) + 8 * h) = ov;
      }
    const int qrow = ra + r;
    if (h == 0 && qrow < N)
      a.lse[(long long)bh * N + qrow] = lt > 0.f ? kLn2 * (x.m2 + fast_log2(lt)) : -INFINITY;
  };
  stage_out(A, 0);
  stage_out(B, 32);
#pragma unroll
  for (int it = 0; it < 16; it++) {
    const int r = 4 * it + (lane >> 4), j = lane & 15;
    const bf16x8 ov = *(const FA_LDS bf16x8*)((FA_LDS char*)so + S::off(r, j));
    const int qrow = ra + r;
    if (qrow < N) *reinterpret_cast<bf16x8*>(a.o + qh + (long long)qrow * a.q_rs + 8 * j) = ov;
  }
}

}  // namespace fa
