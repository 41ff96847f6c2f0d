// bf16 attention forward kernel for gfx950: both contractions on bf16 MFMA, softmax in fp32.
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
//   * Each wave owns 32*QB query rows (split-Q: no communication between waves, Fix 5). The wave
//     computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16, keys on the M axis and queries on the
//     N axis, so every lane holds one query column and 16 of its keys per 32x32 block: the row
//     maximum is an in-lane reduction plus one swap between the two 32-lane halves.
//   * The S^T accumulator layout is directly the B operand of O^T += V^T P^T (same MFMA) after
//     a permutation of the keys inside each 16-key step; V is read from its row-major LDS tile
//     with transposing reads (ds_read_b64_tr_b16) in that same key order, so P never leaves
//     registers and needs no cross-lane shuffle.
//   * Q^T stays in registers for the whole kernel; O^T, m and l too.
//   * K and V tiles go HBM -> LDS with direct 16-byte-per-lane loads (no VGPR staging), double
//     buffered: tile j+1 is in flight while tile j is consumed; one barrier per tile.
//   * Lazy rescaling: the reference maximum only moves when a new score exceeds it by more than
//     kRescaleSlack (log2 units); otherwise p <= 2^kRescaleSlack and the alpha multiply of the
//     accumulator is skipped for the whole wave. Any reference gives the same real-arithmetic
//     result (the rescale identity holds for every reference value). The slack is kept small (a
//     factor 4): a score that arrives without a rescale keeps the key that set the reference at
//     >= 1/5 of their combined weight, so the bf16 rounding of its p cannot dominate a row's
//     output; a large slack (2^8) lets a dominant late key carry a full 2^-9 relative rounding
//     error into O.
//   * Causal: tiles above the diagonal are never loaded or computed; sub-blocks below it run
//     without a mask; only sub-blocks crossing the diagonal (or the ragged tail) are masked.
#pragma once

#include "fa_device.h"

namespace fa {

constexpr float kRescaleSlack = 2.0f;

// Tuning knob: request all K and V fragments of a 32-key sub-block ahead of their MFMAs.
#ifndef FA_HOIST_LDS
#define FA_HOIST_LDS 0
#endif
// Tuning knob: raise the wave's issue priority while it issues a cluster of MFMAs, so that of two
// waves sharing a SIMD the one feeding the matrix core is issued first and the other's softmax
// instructions fill the gaps.
#ifndef FA_SETPRIO
#define FA_SETPRIO 1
#endif
__device__ __forceinline__ void mfma_prio_begin() {
#if FA_SETPRIO
  __builtin_amdgcn_s_setprio(1);
#endif
}
__device__ __forceinline__ void mfma_prio_end() {
#if FA_SETPRIO
  __builtin_amdgcn_s_setprio(0);
#endif
}

struct Bf16Args {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  int N;             // sequence length
  int BH;            // batch * heads
  int n_qblk;        // query blocks per head
  float scale_log2;  // scale * log2(e)
};

template <int D, int QB, int NW, int BC>
struct Bf16Cfg {
  static constexpr int R = 32 * QB;           // query rows per wave
  static constexpr int BLOCK_Q = R * NW;      // query rows per workgroup
  static constexpr int TILE_BYTES = BC * D * 2;
  static constexpr int NSUB = BC / 32;        // 32-key sub-blocks per tile
  static constexpr int DK = D / 16;           // k-steps of Q K^T
  static constexpr int DB = D / 32;           // 32-row blocks of O^T
  static constexpr int LOADS = TILE_BYTES / 1024 / NW;  // 1 KB direct loads per wave per tile
  static_assert(TILE_BYTES % (1024 * NW) == 0, "tile must split evenly over the waves");
  static_assert(BC % 32 == 0, "key tile is a multiple of 32");
};

// Issue the direct loads of one [BC][D] tile (rows key0..key0+BC-1, clamped to N-1) into `tile`.
template <int D, int BC, int NW>
__device__ inline void issue_tile(const bf16* __restrict__ src, int key0, int N, char* tile,
                                  int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int LOADS = BC * D * 2 / 1024 / NW;
#pragma unroll
  for (int i = 0; i < LOADS; i++) {
    const int blk = i * NW + wave;
    const int slot = blk * 64 + lane;
    const int row = slot / CPR;
    const int pc = slot % CPR;
    const int lc = pc ^ swz<D>(row);
    const int grow = min(key0 + row, N - 1);
    global_to_lds16(src + (size_t)grow * D + lc * 8, tile + blk * 1024);
  }
}

// Per-wave running state of the online softmax.
template <int QB, int DB>
struct RowState {
  f32x16 acc[QB][DB];  // O^T accumulator: register i = d 8*(i/4) + 4*h + i%4 of block db
  float m2[QB];        // reference maximum (log2 units), equal in both lane halves
  float l[QB];         // this lane's part of the running sum (its 16 keys per 32-key block)
};

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
__device__ __forceinline__ float sum16(const float (&p)[16]) {
  float t[8];
#pragma unroll
  for (int i = 0; i < 8; i++) t[i] = p[2 * i] + p[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; i++) t[i] = t[2 * i] + t[2 * i + 1];
  return (t[0] + t[1]) + (t[2] + t[3]);
}

// One 32-key sub-block: S^T = K Q^T, online softmax update, O^T += V^T P^T.
// MASKED sub-blocks cross the causal diagonal or the ragged tail; their hidden scores become -inf
// before the maximum, and exp2(-inf) = 0 removes them from the sums (scale_log2 is never 0 here:
// the host runs scale 0 as the smallest normal float, which gives the same probabilities).
#if FA_HOIST_LDS
template <int D, bool CAUSAL, bool MASKED, int QB, int NW, int BC>
__device__ __forceinline__ void consume_sub(const char* __restrict__ Kt,
                                            const char* __restrict__ Vt, int sb, int kb0, int qw0,
                                            int N, float scale_log2, int c, int h, int vrow,
                                            int vcol, const bf16x8 (&qf)[QB][D / 16],
                                            RowState<QB, D / 32>& st) {
  using C = Bf16Cfg<D, QB, NW, BC>;
  // S^T[key][query] for 32 keys x 32 queries per qb. All K fragments are requested before the
  // first MFMA so that LDS latency overlaps the MFMA chain.
  bf16x8 kf[C::DK];
#pragma unroll
  for (int dk = 0; dk < C::DK; dk++)
    kf[dk] = lds_read_b128(Kt + tile_off<D>(32 * sb + c, 16 * dk + 8 * h));
  f32x16 s[QB];
#pragma unroll
  for (int qb = 0; qb < QB; qb++) s[qb] = f32x16{};
  mfma_prio_begin();
#pragma unroll
  for (int dk = 0; dk < C::DK; dk++) {
#pragma unroll
    for (int qb = 0; qb < QB; qb++)
      s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[dk], qf[qb][dk], s[qb], 0, 0, 0);
  }
  mfma_prio_end();

  // V^T fragments for O^T += V^T P^T, requested now so they arrive during the softmax.
  bf16x8 vf[C::DB][2];
#pragma unroll
  for (int db = 0; db < C::DB; db++) {
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      const int r0 = 32 * sb + 16 * ks + vrow;
      const int col = 32 * db + vcol;
      const bf16x4 v0 = lds_read_tr16(Vt + tile_off<D>(r0, col));
      const bf16x4 v1 = lds_read_tr16(Vt + tile_off<D>(r0 + 8, col));
      vf[db][ks] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }

  // Register i of s holds key kb0 + 8*(i/4) + 4*h + i%4 for query qw0 + 32*qb + c.
  float t2[QB];
  bool grow = false;
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    if (MASKED) {
      // hide key kb0 + off_i when off_i > lim (a future key, or a key >= N)
      int lim = N - 1 - kb0;
      if (CAUSAL) lim = min(lim, qw0 + qb * 32 + c - kb0);
      lim -= 4 * h;
#pragma unroll
      for (int i = 0; i < 16; i++)
        if (8 * (i >> 2) + (i & 3) > lim) s[qb][i] = -INFINITY;
    }
    const float mx = half_swap_max(max16(s[qb]));
    t2[qb] = MASKED && mx == -INFINITY ? -INFINITY : mx * scale_log2;
    grow |= t2[qb] > st.m2[qb] + kRescaleSlack;
  }
  if (__any(grow)) {
#pragma unroll
    for (int qb = 0; qb < QB; qb++) {
      const float mn = __builtin_fmaxf(st.m2[qb], t2[qb]);
      const float ref = (mn == -INFINITY) ? 0.f : mn;
      const float alpha = fast_exp2(st.m2[qb] - ref);  // 0 while nothing was seen yet
      st.l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; db++) st.acc[qb][db] *= alpha;
      st.m2[qb] = mn;
    }
  }

  // P = 2^(s*scale_log2 - m), row sum from fp32 P, bf16 P as the B operand of O^T.
  bf16x8 pf[QB][2];
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    const float nref = (st.m2[qb] == -INFINITY) ? 0.f : -st.m2[qb];
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; i++) p[i] = fast_exp2(__builtin_fmaf(s[qb][i], scale_log2, nref));
    st.l[qb] += sum16(p);
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
      for (int e = 0; e < 8; e++) pf[qb][ks][e] = (bf16)p[8 * ks + e];
  }

  // O^T[d][query] += V^T[d][key] P^T[key][query], 16 keys per MFMA.
  mfma_prio_begin();
#pragma unroll
  for (int db = 0; db < C::DB; db++) {
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
#pragma unroll
      for (int qb = 0; qb < QB; qb++)
        st.acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][ks], pf[qb][ks],
                                                                 st.acc[qb][db], 0, 0, 0);
    }
  }
  mfma_prio_end();
}

#else
template <int D, bool CAUSAL, bool MASKED, int QB, int NW, int BC>
__device__ __forceinline__ void consume_sub(const char* __restrict__ Kt,
                                            const char* __restrict__ Vt, int sb, int kb0, int qw0,
                                            int N, float scale_log2, int c, int h, int vrow,
                                            int vcol, const bf16x8 (&qf)[QB][D / 16],
                                            RowState<QB, D / 32>& st) {
  using C = Bf16Cfg<D, QB, NW, BC>;
  // S^T[key][query] for 32 keys x 32 queries per qb.
  f32x16 s[QB];
#pragma unroll
  for (int qb = 0; qb < QB; qb++) s[qb] = f32x16{};
  mfma_prio_begin();
#pragma unroll
  for (int dk = 0; dk < C::DK; dk++) {
    const bf16x8 kf = lds_read_b128(Kt + tile_off<D>(32 * sb + c, 16 * dk + 8 * h));
#pragma unroll
    for (int qb = 0; qb < QB; qb++)
      s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][dk], s[qb], 0, 0, 0);
  }
  mfma_prio_end();

  // Register i of s holds key kb0 + 8*(i/4) + 4*h + i%4 for query qw0 + 32*qb + c.
  float t2[QB];
  bool grow = false;
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    if (MASKED) {
      // hide key kb0 + off_i when off_i > lim (a future key, or a key >= N)
      int lim = N - 1 - kb0;
      if (CAUSAL) lim = min(lim, qw0 + qb * 32 + c - kb0);
      lim -= 4 * h;
#pragma unroll
      for (int i = 0; i < 16; i++)
        if (8 * (i >> 2) + (i & 3) > lim) s[qb][i] = -INFINITY;
    }
    const float mx = half_swap_max(max16(s[qb]));
    t2[qb] = MASKED && mx == -INFINITY ? -INFINITY : mx * scale_log2;
    grow |= t2[qb] > st.m2[qb] + kRescaleSlack;
  }
  if (__any(grow)) {
#pragma unroll
    for (int qb = 0; qb < QB; qb++) {
      const float mn = __builtin_fmaxf(st.m2[qb], t2[qb]);
      const float ref = (mn == -INFINITY) ? 0.f : mn;
      const float alpha = fast_exp2(st.m2[qb] - ref);  // 0 while nothing was seen yet
      st.l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; db++) st.acc[qb][db] *= alpha;
      st.m2[qb] = mn;
    }
  }

  // P = 2^(s*scale_log2 - m), row sum from fp32 P, bf16 P as the B operand of O^T.
  bf16x8 pf[QB][2];
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    const float nref = (st.m2[qb] == -INFINITY) ? 0.f : -st.m2[qb];
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; i++) p[i] = fast_exp2(__builtin_fmaf(s[qb][i], scale_log2, nref));
    st.l[qb] += sum16(p);
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
      for (int e = 0; e < 8; e++) pf[qb][ks][e] = (bf16)p[8 * ks + e];
  }

  // O^T[d][query] += V^T[d][key] P^T[key][query], 16 keys per MFMA.
  mfma_prio_begin();
#pragma unroll
  for (int db = 0; db < C::DB; db++) {
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      const int r0 = 32 * sb + 16 * ks + vrow;
      const int col = 32 * db + vcol;
      const bf16x4 v0 = lds_read_tr16(Vt + tile_off<D>(r0, col));
      const bf16x4 v1 = lds_read_tr16(Vt + tile_off<D>(r0 + 8, col));
      const bf16x8 vf = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int qb = 0; qb < QB; qb++)
        st.acc[qb][db] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][ks], st.acc[qb][db], 0, 0, 0);
    }
  }
  mfma_prio_end();
}

#endif

// Consume one [BC][D] K/V tile held in LDS, 32 keys at a time.
template <int D, bool CAUSAL, int QB, int NW, int BC>
__device__ __forceinline__ void consume_tile(const char* __restrict__ Kt,
                                             const char* __restrict__ Vt, int j, int qw0, int N,
                                             float scale_log2, int c, int h, int vrow, int vcol,
                                             const bf16x8 (&qf)[QB][D / 16],
                                             RowState<QB, D / 32>& st) {
  using C = Bf16Cfg<D, QB, NW, BC>;
#pragma unroll
  for (int sb = 0; sb < C::NSUB; sb++) {
    const int kb0 = j * BC + sb * 32;  // first key of this 32-key sub-block
    if (CAUSAL && kb0 > qw0 + C::R - 1) break;  // above the diagonal for every row of the wave
    if ((kb0 + 31 >= N) || (CAUSAL && kb0 + 31 > qw0)) {
      consume_sub<D, CAUSAL, true, QB, NW, BC>(Kt, Vt, sb, kb0, qw0, N, scale_log2, c, h, vrow,
                                               vcol, qf, st);
    } else {
      consume_sub<D, CAUSAL, false, QB, NW, BC>(Kt, Vt, sb, kb0, qw0, N, scale_log2, c, h, vrow,
                                                vcol, qf, st);
    }
  }
}

// Minimum waves per SIMD the register allocation must allow (tuning knob; 1 = up to 512 VGPRs).
#ifndef FA_MIN_WAVES_PER_EU
#define FA_MIN_WAVES_PER_EU 1
#endif

template <int D, bool CAUSAL, int QB, int NW, int BC>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(FA_MIN_WAVES_PER_EU)))
void fa_fwd_bf16_kernel(Bf16Args a) {
  using C = Bf16Cfg<D, QB, NW, BC>;
  // Two stages, each with its own K and V array: separate objects let the compiler see that the
  // tile being read and the tile being filled never alias.
  __shared__ __attribute__((aligned(1024))) char sK0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sK1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[C::TILE_BYTES];

  const int lane = threadIdx.x & 63;
  // the wave index is the same for all 64 lanes: keep it (and everything derived from it) scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 31;  // query column (S^T, O^T) / key row (K operand)
  const int h = lane >> 5;  // lane half: selects the k-slot half of MFMA operands
  const int N = a.N;

  int bh, qblk;
  map_block<CAUSAL>(blockIdx.x, gridDim.x, a.BH, a.n_qblk, bh, qblk);
  const size_t head = (size_t)bh * N * D;
  const bf16* __restrict__ Qh = a.q + head;
  const bf16* __restrict__ Kh = a.k + head;
  const bf16* __restrict__ Vh = a.v + head;
  const int q0 = qblk * C::BLOCK_Q;
  const int qw0 = q0 + wave * C::R;  // first query row of this wave

  // Key tiles this workgroup visits (causal: none above its last query row).
  const int n_kt_all = (N + BC - 1) / BC;
  int n_kt = n_kt_all;
  if (CAUSAL) n_kt = min(n_kt_all, (min(q0 + C::BLOCK_Q, N) - 1) / BC + 1);

  // Start streaming tile 0 before touching Q.
  issue_tile<D, BC, NW>(Kh, 0, N, sK0, wave, lane);
  issue_tile<D, BC, NW>(Vh, 0, N, sV0, wave, lane);

  // Q^T as the B operand: lane (h, c) holds Q[row c][16*dk + 8*h .. +7] for each k-step dk.
  bf16x8 qf[QB][C::DK];
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    const int row = qw0 + qb * 32 + c;
#pragma unroll
    for (int dk = 0; dk < C::DK; dk++) {
      if (row < N) {
        qf[qb][dk] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)row * D + dk * 16 + h * 8);
      } else {
        qf[qb][dk] = bf16x8{};
      }
    }
  }

  RowState<QB, C::DB> st;
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    st.m2[qb] = -INFINITY;
    st.l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; db++) st.acc[qb][db] = f32x16{};
  }

  // V operand (A of O^T, transposing read): within the 16-lane group g = lane/16, lane L = lane%16
  // addresses row 32*sb + 16*ks + 8*part + 4*h + L/4, column 32*db + 16*(g&1) + 4*(L%4).
  const int Lg = lane & 15;
  const int vrow = 4 * h + (Lg >> 2);
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (Lg & 3);

  // Tile j lives in stage j%2. At the top of each step: my loads of tile j are done, then the
  // barrier makes everyone's loads visible and guarantees everyone has finished tile j-1, whose
  // stage is refilled with tile j+1 while tile j is consumed.
  for (int j = 0; j < n_kt; j += 2) {
    wait_vmem_all();
    __syncthreads();
    if (j + 1 < n_kt) {
      issue_tile<D, BC, NW>(Kh, (j + 1) * BC, N, sK1, wave, lane);
      issue_tile<D, BC, NW>(Vh, (j + 1) * BC, N, sV1, wave, lane);
    }
    consume_tile<D, CAUSAL, QB, NW, BC>(sK0, sV0, j, qw0, N, a.scale_log2, c, h, vrow, vcol, qf,
                                        st);
    if (j + 1 >= n_kt) break;
    wait_vmem_all();
    __syncthreads();
    if (j + 2 < n_kt) {
      issue_tile<D, BC, NW>(Kh, (j + 2) * BC, N, sK0, wave, lane);
      issue_tile<D, BC, NW>(Vh, (j + 2) * BC, N, sV0, wave, lane);
    }
    consume_tile<D, CAUSAL, QB, NW, BC>(sK1, sV1, j + 1, qw0, N, a.scale_log2, c, h, vrow, vcol,
                                        qf, st);
  }

  // Epilogue: O = a / l, LSE = ln2 * (m + log2 l).
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    const float lt = half_swap_sum(st.l[qb]);
    const int qrow = qw0 + qb * 32 + c;
    if (qrow < N) {
      const float inv = 1.0f / lt;
      bf16* orow = a.o + head + (size_t)qrow * D;
#pragma unroll
      for (int db = 0; db < C::DB; db++) {
#pragma unroll
        for (int g = 0; g < 4; g++) {
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; e++) ov[e] = (bf16)(st.acc[qb][db][4 * g + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * g + 4 * h) = ov;
        }
      }
      if (h == 0) a.lse[(size_t)bh * N + qrow] = kLn2 * (st.m2[qb] + fast_log2(lt));
    }
  }
}

}  // namespace fa
