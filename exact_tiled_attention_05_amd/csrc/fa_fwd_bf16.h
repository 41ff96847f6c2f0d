// 8-wave bf16 attention forward kernel for gfx950: both contractions on bf16 MFMA, softmax in
// fp32. It runs the small grids (at most 2^16 query rows, non-causal or d = 64); the 4-wave kernel
// of fa_fwd_ext.h runs the rest (the choice is made in fa_api.hip).
//
// The method ("FlashAttention-2 -- Deeper Math", Fixes 1-5 and "Causal masking: skip the blocks";
// "Understanding FlashAttention Pt 1", §2.4 and §3.1): each workgroup owns a block of query rows
// of one head and streams the key/value tiles past it, keeping per row a reference maximum m, a
// running sum l and an unnormalised output accumulator a:
//     m' = max(m, rowmax(S_tile)), alpha = 2^(m - m'), p = 2^(s - m'),
//     l' = alpha l + sum p,        a' = alpha a + p V_tile,
// with O = a / l and LSE = m + log l written once after the last tile. Scores are kept in base 2
// (s = scale * log2(e) * q.k in fp32) and LSE is converted to natural-log units on output.
//
// MI355X mapping.
//   * A workgroup is 8 waves and 256 query rows; each wave owns 32 rows (split-Q: no communication
//     between waves, Fix 5). The wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16, keys on
//     the M axis and queries on the N axis, so every lane holds one query column and 16 of its
//     keys per 32x32 block: the row maximum is an in-lane reduction plus one swap between the two
//     32-lane halves.
//   * The S^T accumulator layout is directly the B operand of O^T += V^T P^T (same MFMA) after a
//     permutation of the keys inside each 16-key k-step: k-slot 8h + e of lane half h holds key
//     8 (e / 4) + 4 h + e % 4. V is read from its row-major LDS tile with transposing reads
//     (ds_read_b64_tr_b16) in that same key order, so P never leaves registers.
//   * Q^T stays in registers for the whole kernel; O^T, m and l too.
//   * Lazy rescaling: the reference maximum only moves when a new score exceeds it by more than
//     kRescaleSlack (log2 units); otherwise p <= 2^kRescaleSlack and the alpha multiply of the
//     accumulator is skipped for the whole wave. Any reference gives the same real-arithmetic
//     result (the rescale identity holds for every reference value). The slack is kept small (a
//     factor 4): a score that arrives without a rescale keeps the key that set the reference at
//     >= 1/5 of their combined weight, so the bf16 rounding of its p cannot dominate a row's
//     output; a large slack (2^8) lets a dominant late key carry a full 2^-9 relative rounding
//     error into O.
//   * Causal: tiles above the diagonal are never loaded or computed; 32-key steps below it run
//     without a mask; only steps crossing the diagonal (or the ragged tail) are masked.
//
// Instruction stream. Step g of a wave consumes 32 keys in two phases:
//     V(g):   request the K fragments of step g+1 and the V^T fragments of step g from LDS, then
//             the softmax of S(g) on the vector ALUs (mask, row maximum, reference update, rare
//             rescale, exponentials, row sums, bf16 packing of P(g));
//     M(g+1): one cluster of 16 MFMAs: S(g+1) = K(g+1) Q^T, then O^T += V^T(g) P^T(g).
// A wave's vector instructions barely overlap its own MFMAs, but the other wave on the same SIMD
// can keep the matrix core busy meanwhile. The 8 waves sit two per SIMD (waves w and w+4, as the
// hardware places them) and form two groups, A = waves 0-3 and B = waves 4-7. The per-tile LDS
// barrier sits at different points of the two groups' streams: group A meets it between M(g) and
// V(g), group B between V(g-1) and M(g). When it releases, A starts a V phase while B starts an M
// phase, so the two waves of every SIMD stay half a step apart (ping-pong) instead of being pulled
// into the same phase at every tile.
//
// LDS protocol. Tiles are 64 keys (steps 2j and 2j+1 of tile j) in three stages, tile j in stage
// j % 3. Crossing j writes the staged tile j+1 (held in registers) into stage (j+1) % 3, meets the
// barrier, and starts the loads of tile j+2 into the staging registers. Group A crosses at the
// start of step 2j+1, group B between V(2j) and M(2j+1). In both groups every read of tile j+1
// (first: K of step 2j+2, requested in V(2j+1)) follows crossing j, and every read of tile j-2
// (last: V^T of step 2j-3, requested in V(2j-3)) precedes crossing j-1, which precedes any write
// of tile j+1. Every wave executes every crossing, also waves whose rows are all past N or whose
// causal rows end early, so barrier counts always match.
#pragma once

#include <type_traits>

#include "fa_device.h"
#include "fa_tiles.h"

namespace fa {

constexpr float kRescaleSlack = 2.0f;

// Shapes and strides. Query head h of batch b reads K/V head h / group ("Understanding
// FlashAttention Pt 1", §4.1: the query heads divide evenly over the K/V heads and each attends
// with its assigned one; MHA is group 1, MQA one K/V head). q and o share one set of element
// strides, k and v another; lse is always [B][H][N].
struct Bf16Args {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  int N;             // sequence length
  int BH;            // batch * query heads
  int H;             // query heads
  int group;         // query heads per K/V head
  int n_qblk;        // query blocks per head
  float scale_log2;  // scale * log2(e)
  long long q_bs, q_hs;    // q/o element strides of a batch and a head
  long long kv_bs, kv_hs;  // k/v element strides of a batch and a head
  int q_rs, kv_rs;         // element strides of a row (one token)
};

constexpr int kNumWaves = 8;                    // waves per workgroup
constexpr int kBlockQ = 32 * kNumWaves;         // query rows per workgroup
constexpr int kBlockK = 64;                     // keys per LDS tile

// LDS layouts: row-major tiles with padded rows, one padding per matrix so that each read pattern
// is bank-conflict free and every address is a per-lane base plus a compile-time offset:
//   K rows are 2*D + 16 bytes: the K operand reads one 16-byte chunk from 16 consecutive rows;
//     a 16-byte row shift walks those 16 reads across all 64 banks.
//   V rows are 2*D + 64 bytes: a transposing read touches 4 consecutive rows x 32 bytes per
//     16-lane group (64 bytes per half-wave); a 64-byte row shift spreads the rows apart.
template <int D>
struct Layout {
  static constexpr int KROW = 2 * D + 16;
  static constexpr int VROW = 2 * D + 64;
  static constexpr int K_BYTES = kBlockK * KROW;
  static constexpr int V_BYTES = kBlockK * VROW;
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Register-staged tile copies. A [64][D] tile is split into 1 KB pieces of 64 16-byte chunks; wave
// w copies pieces w, w+8, ...; lane L of piece i holds chunk 64*i + L of the row-major tile (row
// (64*i + L) / (D/8), column chunk (64*i + L) % (D/8)).
template <int D>
struct TileRegs {
  static constexpr int LOADS = kBlockK * D * 2 / 1024 / kNumWaves;
  static_assert(kBlockK * D * 2 % (1024 * kNumWaves) == 0, "tile must split evenly over the waves");
  u32x4 k[LOADS], v[LOADS];
};

// Loads go through raw buffer resources laid over the tile's rows: a resource starts at the
// tile's first row and ends after its last row below N, so rows at or past N read as zeros
// (their scores are masked) and every offset stays small whatever the row stride. Piece i of
// wave w holds rows (i * 8 + w) * R .. + R - 1 of the tile (R = 64 / (D/8) rows per piece); lane
// L's 16 bytes are chunk L % (D/8) of row L / (D/8). The per-lane offset (voff) is the same for
// every piece and tile and the piece offset is scalar, so a load costs no vector ALU work.
template <int D>
struct TileSrc {
  const char* kbase;  // byte address of row 0 of this head's K (V at the same offsets from vbase)
  const char* vbase;
  long long rs;       // bytes between consecutive rows
  int voff;           // this lane's byte offset inside a piece
};

template <int D>
__device__ __forceinline__ void load_tile(const TileSrc<D>& src, int key0, int N, int wave,
                                          TileRegs<D>& r) {
  constexpr int CPR = D / 8, RPP = 64 / CPR;
  const long long t0 = (long long)key0 * src.rs;
  const int rows = min(N - key0, kBlockK);  // >= 1: only tiles that start below N are loaded
  const int bytes = (int)((rows - 1) * src.rs) + 2 * D;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(src.kbase + t0), 0, bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(src.vbase + t0), 0, bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < TileRegs<D>::LOADS; i++) {
    const int soff = (int)((i * kNumWaves + wave) * RPP * src.rs);
    r.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, src.voff, soff, 0));
    r.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, src.voff, soff, 0));
  }
}

template <int D>
__device__ __forceinline__ void store_tile(char* __restrict__ Kt, char* __restrict__ Vt, int wave,
                                           int lane, const TileRegs<D>& r) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::LOADS; i++) {
    const int slot = (i * kNumWaves + wave) * 64 + lane;
    const int row = slot / CPR, chunk = slot % CPR;
    *(FA_LDS u32x4*)(Kt + row * Layout<D>::KROW + 16 * chunk) = r.k[i];
    *(FA_LDS u32x4*)(Vt + row * Layout<D>::VROW + 16 * chunk) = r.v[i];
  }
}

// Fixed per-lane quantities of a wave, including the per-lane LDS bases:
//   K operand (row 32*sb + c, column 16*dk + 8*h):  kbase + 32*dk + 32*KROW*sb
//   V operand (rows 32*sb + 16*ks + vrow + 8*part, column 32*db + vcol):
//                                                   vbase + 8*VROW*part + 64*db + (32*sb + 16*ks)*VROW
struct Lane {
  int c, h, qrow, qw0, N, last;
  int kbase, vbase;
  float sl2;
};

// K operand of one 32-key step (sub-block sb of the tile at Kt).
template <int D>
__device__ __forceinline__ void read_k(const char* __restrict__ Kt, int sb, const Lane& L,
                                       bf16x8 (&kf)[D / 16]) {
  constexpr int KROW = Layout<D>::KROW;
#pragma unroll
  for (int dk = 0; dk < D / 16; dk++) kf[dk] = lds_read_b128(Kt + L.kbase + 32 * dk + 32 * KROW * sb);
}

// V^T operand of one 32-key step, in the key order of the S^T accumulator.
template <int D>
__device__ __forceinline__ void read_v(const char* __restrict__ Vt, int sb, const Lane& L,
                                       bf16x8 (&vf)[D / 32][2]) {
  constexpr int VROW = Layout<D>::VROW;
#pragma unroll
  for (int db = 0; db < D / 32; db++)
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      const char* p = Vt + L.vbase + 64 * db + (32 * sb + 16 * ks) * VROW;
      const bf16x4 v0 = lds_read_tr16(p);
      const bf16x4 v1 = lds_read_tr16(p + 8 * VROW);
      vf[db][ks] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// Per-wave state.
template <int D>
struct WaveState {
  bf16x8 qf[D / 16];     // Q^T operand (this wave's 32 rows)
  f32x16 acc[D / 32];    // O^T accumulator: register i = d 8*(i/4) + 4*h + i%4 of block db
  f32x16 s;              // S^T of the step whose softmax comes next
  bf16x8 pf[2];          // P^T operand of the step whose PV product comes next
  bf16x8 kf[D / 16];     // K operand of the next QK product
  bf16x8 vf[D / 32][2];  // V^T operand of the next PV product
  float m2, l;           // reference maximum (log2 units) and this lane's part of the row sum
};

// V phase, softmax part: P(g) from S(g). Hidden scores (keys past N, and with a causal mask keys
// past the lane's row) become -inf before the maximum, and exp2(-inf) = 0 removes them from the
// sums.
template <int D, bool CAUSAL>
__device__ __forceinline__ void softmax_step(int g, const Lane& L, WaveState<D>& st) {
  constexpr int DB = D / 32;
  f32x16& s = st.s;
  const int kb0 = g * 32;
  if ((kb0 + 31 >= L.N) || (CAUSAL && kb0 + 31 > L.qw0)) {
    int lim = L.N - 1 - kb0;
    if (CAUSAL) lim = min(lim, L.qrow - kb0);
    lim -= 4 * L.h;
#pragma unroll
    for (int i = 0; i < 16; i++)
      if (8 * (i >> 2) + (i & 3) > lim) s[i] = -INFINITY;
  }
  // Every row of an active step sees at least one key (key 0 at step 0, its own diagonal key in
  // the diagonal step, key kb0 < N in the tail step), so the maximum is finite; scale_log2 > 0
  // (scale 0 runs as FLT_MIN), so t2 and, from the first step on, m2 are finite.
  const float t2 = half_swap_max(max16(s)) * L.sl2;
  if (__any(t2 > st.m2 + kRescaleSlack)) {
    const float mn = __builtin_fmaxf(st.m2, t2);
    const float alpha = fast_exp2(st.m2 - mn);  // 0 at the first step (m2 = -inf)
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; db++) st.acc[db] *= alpha;
    st.m2 = mn;
  }
  const float nref = -st.m2;
  float p[16];
#pragma unroll
  for (int i = 0; i < 16; i++) p[i] = fast_exp2(__builtin_fmaf(s[i], L.sl2, nref));
#pragma unroll
  for (int ks = 0; ks < 2; ks++)
#pragma unroll
    for (int e = 0; e < 8; e++) st.pf[ks][e] = (bf16)p[8 * ks + e];
  st.l += sum16(p);
  // The packed P and the row sum exist here, before any barrier that follows in program order
  // (pure arithmetic would otherwise be free to sink to its first use in the M phase).
  asm volatile("" ::"v"(st.pf[0]), "v"(st.pf[1]), "v"(st.l));
}

// M phase: S(g+1) (when the wave has a step g+1), then O^T += V^T(g) P^T(g).
template <int D>
__device__ __forceinline__ void mfma_step(bool qk, WaveState<D>& st) {
  constexpr int DK = D / 16, DB = D / 32;
  if (qk) {
    st.s = f32x16{};
#pragma unroll
    for (int dk = 0; dk < DK; dk++)
      st.s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(st.kf[dk], st.qf[dk], st.s, 0, 0, 0);
  }
#pragma unroll
  for (int ks = 0; ks < 2; ks++)
#pragma unroll
    for (int db = 0; db < DB; db++)
      st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(st.vf[db][ks], st.pf[ks], st.acc[db], 0, 0, 0);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kNumWaves * 64) void fa_fwd_bf16_kernel(Bf16Args a) {
  constexpr int DK = D / 16;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(1024))) char sK0[Layout<D>::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char sK1[Layout<D>::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char sK2[Layout<D>::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV0[Layout<D>::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[Layout<D>::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV2[Layout<D>::V_BYTES];

  const int lane = threadIdx.x & 63;
  // the wave index is the same for all 64 lanes: keep it (and everything derived from it) scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool group_a = wave < kNumWaves / 2;  // waves w and w + 4 share a SIMD
  const int N = a.N;
  {
    race_check_poison<Layout<D>::K_BYTES>(sK0, threadIdx.x, kNumWaves * 64);
    race_check_poison<Layout<D>::K_BYTES>(sK1, threadIdx.x, kNumWaves * 64);
    race_check_poison<Layout<D>::K_BYTES>(sK2, threadIdx.x, kNumWaves * 64);
    race_check_poison<Layout<D>::V_BYTES>(sV0, threadIdx.x, kNumWaves * 64);
    race_check_poison<Layout<D>::V_BYTES>(sV1, threadIdx.x, kNumWaves * 64);
    race_check_poison<Layout<D>::V_BYTES>(sV2, threadIdx.x, kNumWaves * 64);
    race_check_barrier();
  }

  int bh, qblk;
  map_block<CAUSAL>(blockIdx.x, gridDim.x, a.BH, a.n_qblk, bh, qblk);
  const int b = bh / a.H, h = bh - b * a.H, hk = h / a.group;
  const long long qhead = b * a.q_bs + h * a.q_hs;  // element offset of this head's row 0
  const bf16* __restrict__ Qh = a.q + qhead;
  TileSrc<D> src;
  {
    const long long kvhead = b * a.kv_bs + hk * a.kv_hs;
    src.kbase = reinterpret_cast<const char*>(a.k + kvhead);
    src.vbase = reinterpret_cast<const char*>(a.v + kvhead);
    src.rs = 2LL * a.kv_rs;
    src.voff = (int)((lane / (D / 8)) * src.rs) + 16 * (lane % (D / 8));
  }
  const int q0 = qblk * kBlockQ;

  Lane L;
  L.c = lane & 31;
  L.h = lane >> 5;
  L.N = N;
  L.sl2 = a.scale_log2;
  L.qw0 = q0 + wave * 32;  // the wave's first query row
  L.qrow = L.qw0 + L.c;    // this lane's query row
  {
    // V operand, transposing read: in 16-lane group g = lane/16, lane Lg = lane%16 addresses row
    // vrow = 4*h + Lg/4 (+8 for the second half of the k-slots), column 16*(g&1) + 4*(Lg%4).
    const int Lg = lane & 15;
    const int vrow = 4 * L.h + (Lg >> 2);
    const int vcol = 16 * ((lane >> 4) & 1) + 4 * (Lg & 3);
    L.kbase = L.c * Layout<D>::KROW + 16 * L.h;
    L.vbase = vrow * Layout<D>::VROW + 2 * vcol;
  }

  // Tiles of the workgroup (causal: up to its last row) and 32-key steps of this wave (causal: up
  // to its own diagonal).
  const int n_kt_all = (N + kBlockK - 1) / kBlockK;
  const int n_kt = CAUSAL ? min(n_kt_all, (min(q0 + kBlockQ, N) - 1) / kBlockK + 1) : n_kt_all;
  const int n_steps = 2 * n_kt;
  // last step with a key this wave can see (-1: every row of the wave is past N)
  L.last = L.qw0 >= N ? -1
           : CAUSAL   ? min(n_steps - 1, (min(L.qw0 + 31, N - 1)) / 32)
                      : (N - 1) / 32;

  // Prologue: tile 0 into stage 0, Q into registers, tile 1 into the staging registers, S(0).
  TileRegs<D> stage;
  load_tile<D>(src, 0, N, wave, stage);
  WaveState<D> st;
  {
    // Q of the wave's 32 rows: whole-row loads (4 rows per instruction), through a wave-private
    // swizzled LDS region of stage 1 or 2 (not written before the first crossing, which follows
    // the prologue barrier) into the operand layout
    using SQ = Swz<D>;
    char* const sq = (wave < 2 ? sK1 : wave < 4 ? sK2 : wave < 6 ? sV1 : sV2) + (wave & 1) * (32 * SQ::ROW);
    constexpr int RPI = 64 / SQ::CPR;
    bf16x8 qr[32 / RPI];
#pragma unroll
    for (int it = 0; it < 32 / RPI; it++) {
      const int r = RPI * it + lane / SQ::CPR, j = lane % SQ::CPR;
      qr[it] = L.qw0 + r < N ? *reinterpret_cast<const bf16x8*>(Qh + (long long)(L.qw0 + r) * a.q_rs + 8 * j)
                             : bf16x8{};
    }
#pragma unroll
    for (int it = 0; it < 32 / RPI; it++) {
      const int r = RPI * it + lane / SQ::CPR, j = lane % SQ::CPR;
      *(FA_LDS bf16x8*)((FA_LDS char*)sq + SQ::off(r, j)) = qr[it];
    }
#pragma unroll
    for (int dk = 0; dk < DK; dk++)
      st.qf[dk] = *(const FA_LDS bf16x8*)((FA_LDS char*)sq + SQ::off(L.c, 2 * dk + L.h));
  }
#pragma unroll
  for (int db = 0; db < DB; db++) st.acc[db] = f32x16{};
  st.m2 = -INFINITY;
  st.l = 0.f;
  store_tile<D>(sK0, sV0, wave, lane, stage);
  if (n_kt > 1) load_tile<D>(src, kBlockK, N, wave, stage);
  __syncthreads();
  st.s = f32x16{};
  if (L.last >= 0) {
    read_k<D>(sK0, 0, L, st.kf);
#pragma unroll
    for (int dk = 0; dk < DK; dk++)
      st.s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(st.kf[dk], st.qf[dk], st.s, 0, 0, 0);
  }

  // Crossing j: staged tile j+1 into its stage, barrier, loads of tile j+2.
  auto crossing = [&](char* __restrict__ Kn, char* __restrict__ Vn, int j) {
    race_check_barrier();
    store_tile<D>(Kn, Vn, wave, lane, stage);
    __syncthreads();
    if (j + 2 < n_kt) load_tile<D>(src, (j + 2) * kBlockK, N, wave, stage);
  };

  // Tile j in stage S (a compile-time constant, so every LDS address is a base plus an immediate
  // and the compiler sees which array each access touches).
  auto tile = [&](auto stage_c, int j) {
    constexpr int S = decltype(stage_c)::value;
    constexpr int SN = (S + 1) % 3;
    const char* Kt = S == 0 ? sK0 : S == 1 ? sK1 : sK2;
    const char* Vt = S == 0 ? sV0 : S == 1 ? sV1 : sV2;
    char* Knext = SN == 0 ? sK0 : SN == 1 ? sK1 : sK2;
    char* Vnext = SN == 0 ? sV0 : SN == 1 ? sV1 : sV2;
    const bool has_next_tile = j + 1 < n_kt;
    {  // step 2j
      const int g = 2 * j;
      if (g <= L.last) {
        if (g + 1 <= L.last) read_k<D>(Kt, 1, L, st.kf);
        read_v<D>(Vt, 0, L, st.vf);
        softmax_step<D, CAUSAL>(g, L, st);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (!group_a && has_next_tile) crossing(Knext, Vnext, j);
      __builtin_amdgcn_sched_barrier(0);
      if (g <= L.last) mfma_step<D>(g + 1 <= L.last, st);
      __builtin_amdgcn_sched_barrier(0);
    }
    {  // step 2j+1
      const int g = 2 * j + 1;
      if (group_a && has_next_tile) crossing(Knext, Vnext, j);
      __builtin_amdgcn_sched_barrier(0);
      if (g <= L.last) {
        if (g + 1 <= L.last) read_k<D>(Knext, 0, L, st.kf);
        read_v<D>(Vt, 1, L, st.vf);
        softmax_step<D, CAUSAL>(g, L, st);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (g <= L.last) mfma_step<D>(g + 1 <= L.last, st);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  for (int j = 0; j < n_kt; j += 3) {
    tile(I0{}, j);
    if (j + 1 >= n_kt) break;
    tile(I1{}, j + 1);
    if (j + 2 >= n_kt) break;
    tile(I2{}, j + 2);
  }

  // Epilogue: O = a / l, LSE = ln2 * (m + log2 l). O goes out through LDS (the tile stages, free
  // once every wave is past the last tile): each wave writes its 32 rows of bf16 O into a swizzled
  // region of its own and reads them back as whole rows, so a store instruction writes complete
  // rows instead of 16 bytes of 32 rows.
  const float lt = half_swap_sum(st.l);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  using SO = Swz<D>;
  constexpr int OREG = 32 * SO::ROW;  // one wave's 32 rows
  static_assert(2 * OREG <= Layout<D>::K_BYTES && 2 * OREG <= Layout<D>::V_BYTES, "O staging fits");
  __syncthreads();
  char* const so = (wave < 2 ? sK0 : wave < 4 ? sK1 : wave < 6 ? sK2 : sV0) + (wave & 1) * OREG;
#pragma unroll
  for (int db = 0; db < DB; db++)
#pragma unroll
    for (int g4 = 0; g4 < 4; g4++) {
      bf16x4 ov;
#pragma unroll
      for (int e = 0; e < 4; e++) ov[e] = (bf16)(st.acc[db][4 * g4 + e] * inv);
      *(FA_LDS bf16x4*)((FA_LDS char*)so + SO::off(L.c, 4 * db + g4) + 8 * L.h) = ov;
    }
  if (L.qrow < N && L.h == 0) a.lse[(size_t)bh * N + L.qrow] = kLn2 * (st.m2 + fast_log2(lt));
  constexpr int RPI = 64 / SO::CPR;  // rows per read instruction
#pragma unroll
  for (int it = 0; it < 32 / RPI; it++) {
    const int r = RPI * it + lane / SO::CPR, j = lane % SO::CPR;
    const bf16x8 ov = *(const FA_LDS bf16x8*)((FA_LDS char*)so + SO::off(r, j));
    const int row = L.qw0 + r;
    if (row < N) *reinterpret_cast<bf16x8*>(a.o + qhead + (long long)row * a.q_rs + 8 * j) = ov;
  }
}

}  // namespace fa
