// bf16 attention forward kernel for gfx950, software-pipelined over 32-key steps.
//
// Same method and MFMA mapping as fa_fwd_bf16.h (the online softmax of "FlashAttention-2 --
// Deeper Math", Fixes 1-5, computed as S^T = K Q^T and O^T += V^T P^T on
// v_mfma_f32_32x32x16_bf16, one wave per 32 query rows, K/V tiles streamed into LDS with direct
// loads). What changes is the order in which one wave issues its work. Step g of a wave consumes
// 32 keys; its instruction stream is
//     1. request the V^T fragments of step g and the K fragments of step g+1 from LDS;
//     2. row maximum of S(g), reference update and (rarely) the rescale of the accumulator;
//     3. S(g+1) = K(g+1) Q^T on the matrix cores, interleaved instruction by instruction with the
//        exponentials, row sums and bf16 conversion of P(g) on the vector ALUs;
//     4. O^T += V^T(g) P^T(g) on the matrix cores.
// so the matrix cores, the vector ALUs and the LDS each have work queued from the same wave, and
// the two waves that share a SIMD fill each other's gaps. The LDS tile barrier sits between 1 and
// 2 of the step that crosses into the next tile: by then every wave has finished reading the tile
// that the next direct load overwrites.
#pragma once

#include <type_traits>

#include "fa_fwd_bf16.h"

namespace fa {

// LDS layouts of the pipelined kernel: row-major tiles with padded rows instead of an XOR
// swizzle, one padding per matrix so that each read pattern is bank-conflict free and every
// address is a per-lane base plus a compile-time offset:
//   K rows are 2*D + 16 bytes: the K operand reads one 16-byte chunk from 16 consecutive rows;
//     a 16-byte row shift walks those 16 reads across all 64 banks.
//   V rows are 2*D + 64 bytes: a transposing read touches 4 consecutive rows x 32 bytes per
//     16-lane group (64 bytes per half-wave); a 64-byte row shift spreads the rows apart.
template <int D>
struct PipeLayout {
  static constexpr int KROW = 2 * D + 16;
  static constexpr int VROW = 2 * D + 64;
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Register-staged tile copies. A [BC][D] tile is split into 1 KB pieces of 64 16-byte chunks;
// wave w copies pieces w, w+NW, ...; lane L of piece i holds chunk (64*i + L) of the row-major
// tile (row (64*i + L) / (D/8), column chunk (64*i + L) % (D/8)). The pieces are loaded from
// global memory one tile ahead and written to LDS when the tile is due; the compiler tracks the
// staging VGPRs exactly, so no LDS read waits for a load it does not depend on.
template <int D, int BC, int NW>
struct TileRegs {
  static constexpr int LOADS = BC * D * 2 / 1024 / NW;
  u32x4 k[LOADS], v[LOADS];
};

template <int D, int BC, int NW>
__device__ __forceinline__ void load_tile_regs(const bf16* __restrict__ Kh,
                                               const bf16* __restrict__ Vh, int key0, int N,
                                               int wave, int lane, TileRegs<D, BC, NW>& r) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < TileRegs<D, BC, NW>::LOADS; i++) {
    const int slot = (i * NW + wave) * 64 + lane;
    const size_t off = (size_t)min(key0 + slot / CPR, N - 1) * D + (slot % CPR) * 8;
    r.k[i] = *reinterpret_cast<const u32x4*>(Kh + off);
    r.v[i] = *reinterpret_cast<const u32x4*>(Vh + off);
  }
}

template <int D, int BC, int NW>
__device__ __forceinline__ void store_tile_regs(char* __restrict__ Kt, char* __restrict__ Vt,
                                                int wave, int lane,
                                                const TileRegs<D, BC, NW>& r) {
  constexpr int CPR = D / 8;
  using Lay = PipeLayout<D>;
#pragma unroll
  for (int i = 0; i < TileRegs<D, BC, NW>::LOADS; i++) {
    const int slot = (i * NW + wave) * 64 + lane;
    const int row = slot / CPR, chunk = slot % CPR;
    *(FA_LDS u32x4*)(Kt + row * Lay::KROW + 16 * chunk) = r.k[i];
    *(FA_LDS u32x4*)(Vt + row * Lay::VROW + 16 * chunk) = r.v[i];
  }
}

// Per-wave state carried from step to step.
template <int D>
struct PipeState {
  bf16x8 qf[D / 16];       // Q^T operand (this wave's 32 rows)
  f32x16 acc[D / 32];      // O^T accumulator
  f32x16 s[2];             // S^T of the current and the next step (steps alternate the roles)
  float m2, l;             // reference maximum (log2 units) and this lane's part of the sum
};

// Fixed per-lane quantities of a wave, including the per-lane LDS bases:
//   K operand (row 32*sb + c, column 16*dk + 8*h):  kbase + 32*dk + 32*KROW*sb
//   V operand (rows 32*sb + 16*ks + vrow + 8*part, column 32*db + vcol):
//                                                   vbase + 8*VROW*part + 64*db + (32*sb + 16*ks)*VROW
struct PipeLane {
  int c, h, qrow, qw0, N, last;
  int kbase, vbase;
  float sl2;
};

template <int D>
__device__ __forceinline__ void pipe_read_k(const char* __restrict__ Kt, int sb, const PipeLane& L,
                                            bf16x8 (&kf)[D / 16]) {
  constexpr int KROW = PipeLayout<D>::KROW;
#pragma unroll
  for (int dk = 0; dk < D / 16; dk++) kf[dk] = lds_read_b128(Kt + L.kbase + 32 * dk + 32 * KROW * sb);
}

template <int D>
__device__ __forceinline__ void pipe_read_v(const char* __restrict__ Vt, int sb, int db0, int db1,
                                            const PipeLane& L, bf16x8 (&vf)[D / 32][2]) {
  constexpr int VROW = PipeLayout<D>::VROW;
#pragma unroll
  for (int db = db0; db < db1; db++)
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      const char* p = Vt + L.vbase + 64 * db + (32 * sb + 16 * ks) * VROW;
      const bf16x4 v0 = lds_read_tr16(p);
      const bf16x4 v1 = lds_read_tr16(p + 8 * VROW);
      vf[db][ks] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// Steps 2-4 of one 32-key step g whose V^T comes from Vt and whose successor's K from Kn
// (the caller has already done step 1's barrier, if any).
template <int D, bool CAUSAL, int CUR>
__device__ __forceinline__ void pipe_compute(const char* __restrict__ Vt, int sb,
                                             const char* __restrict__ Kn, int sbn, bool has_next,
                                             int g, const PipeLane& L, PipeState<D>& st) {
  constexpr int DK = D / 16, DB = D / 32;
  // K of the next step (zeros for the wave's final step: its MFMAs run but are discarded, so the
  // interleaved block below has no branch).
  bf16x8 kf[DK];
  if (has_next) {
    pipe_read_k<D>(Kn, sbn, L, kf);
  } else {
#pragma unroll
    for (int dk = 0; dk < DK; dk++) kf[dk] = bf16x8{};
  }

  // 2. Mask (diagonal or ragged tail), row maximum, reference update.
  f32x16& s = st.s[CUR];
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
  // the diagonal step, key kb0 < N in the tail step), so mx is finite; scale_log2 > 0 (scale 0
  // runs as FLT_MIN), so t2 is finite and m2 is finite from the first step on.
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

  // 3. S(g+1) on the matrix cores interleaved, in program order, with the exponentials of P(g);
  //    the V^T requests of this step go out once half of the K fragments are consumed. The
  //    fences keep the scheduler from regrouping the pieces.
  f32x16& sn = st.s[1 - CUR];
  sn = f32x16{};
  bf16x8 vf[DB][2];
  float p[16];
  constexpr int EPM = 16 / DK;
#pragma unroll
  for (int dk = 0; dk < DK; dk++) {
    sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[dk], st.qf[dk], sn, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < EPM; e++)
      p[EPM * dk + e] = fast_exp2(__builtin_fmaf(s[EPM * dk + e], L.sl2, nref));
    if (dk == DK / 2 - 1) pipe_read_v<D>(Vt, sb, 0, DB / 2, L, vf);
    if (dk == DK - 2) pipe_read_v<D>(Vt, sb, DB / 2, DB, L, vf);
    __builtin_amdgcn_sched_barrier(0);
  }

  // 4. O^T += V^T(g) P^T(g), with the bf16 packing and the row sum in between.
  bf16x8 pf[2];
#pragma unroll
  for (int ks = 0; ks < 2; ks++) {
#pragma unroll
    for (int e = 0; e < 8; e++) pf[ks][e] = (bf16)p[8 * ks + e];
#pragma unroll
    for (int db = 0; db < DB; db++)
      st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][ks], pf[ks], st.acc[db], 0, 0, 0);
  }
  st.l += sum16(p);
}

template <int D, bool CAUSAL, int NW, int BC>
__global__ __launch_bounds__(NW * 64) void fa_fwd_bf16_pipe_kernel(Bf16Args a) {
  constexpr int NSUB = BC / 32;  // 32-key steps per tile
  static_assert(NSUB % 2 == 0, "an even number of steps per tile keeps the S buffers aligned");
  constexpr int DK = D / 16;     // k-steps of Q K^T
  constexpr int DB = D / 32;     // 32-row blocks of O^T
  constexpr int BLOCK_Q = 32 * NW;
  constexpr int KT_BYTES = BC * PipeLayout<D>::KROW;
  constexpr int VT_BYTES = BC * PipeLayout<D>::VROW;
  static_assert((BC * D * 2) % (1024 * NW) == 0, "tile must split evenly over the waves");
  // Three stages, each a separate K and V array. Tile j lives in stage j % 3; while tile j is
  // consumed, tile j+1 is already visible and tile j+2 is in flight into staging registers.
  __shared__ __attribute__((aligned(1024))) char sK0[KT_BYTES];
  __shared__ __attribute__((aligned(1024))) char sK1[KT_BYTES];
  __shared__ __attribute__((aligned(1024))) char sK2[KT_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV0[VT_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[VT_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV2[VT_BYTES];

  const int lane = threadIdx.x & 63;
  // the wave index is the same for all 64 lanes: keep it (and everything derived from it) scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int N = a.N;

  int bh, qblk;
  map_block<CAUSAL>(blockIdx.x, gridDim.x, a.BH, a.n_qblk, bh, qblk);
  const size_t head = (size_t)bh * N * D;
  const bf16* __restrict__ Qh = a.q + head;
  const bf16* __restrict__ Kh = a.k + head;
  const bf16* __restrict__ Vh = a.v + head;
  const int q0 = qblk * BLOCK_Q;

  PipeLane L;
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
    L.kbase = L.c * PipeLayout<D>::KROW + 16 * L.h;
    L.vbase = vrow * PipeLayout<D>::VROW + 2 * vcol;
  }

  // Tiles of the workgroup and 32-key steps of this wave (causal: up to its own diagonal).
  const int n_kt_all = (N + BC - 1) / BC;
  const int n_kt = CAUSAL ? min(n_kt_all, (min(q0 + BLOCK_Q, N) - 1) / BC + 1) : n_kt_all;
  const int n_steps = n_kt * NSUB;  // workgroup-uniform
  // last step with a key this wave can see (-1: every row of the wave is past N)
  L.last = L.qw0 >= N ? -1
           : CAUSAL   ? min(n_steps - 1, (min(L.qw0 + 31, N - 1)) / 32)
                      : (N - 1) / 32;

  // Tile 0 into stage 0, Q into registers, tile 1 into staging registers.
  TileRegs<D, BC, NW> stage;
  load_tile_regs<D, BC, NW>(Kh, Vh, 0, N, wave, lane, stage);
  PipeState<D> st;
#pragma unroll
  for (int dk = 0; dk < DK; dk++)
    st.qf[dk] = (L.qrow < N)
                    ? *reinterpret_cast<const bf16x8*>(Qh + (size_t)L.qrow * D + dk * 16 + L.h * 8)
                    : bf16x8{};
#pragma unroll
  for (int db = 0; db < DB; db++) st.acc[db] = f32x16{};
  st.m2 = -INFINITY;
  st.l = 0.f;
  store_tile_regs<D, BC, NW>(sK0, sV0, wave, lane, stage);
  if (n_kt > 1) load_tile_regs<D, BC, NW>(Kh, Vh, BC, N, wave, lane, stage);
  __syncthreads();

  // S(0).
  st.s[0] = f32x16{};
  if (L.last >= 0) {
    bf16x8 kf[DK];
    pipe_read_k<D>(sK0, 0, L, kf);
#pragma unroll
    for (int dk = 0; dk < DK; dk++)
      st.s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[dk], st.qf[dk], st.s[0], 0, 0, 0);
  }

  // Tile j (in stage S): steps 0..NSUB-1. The last step of the tile writes the staged tile j+1
  // into stage (j+1) % 3 (its previous tile, j-2, was finished by every wave before the last
  // barrier), waits at the barrier until every wave has done the same, and starts loading tile
  // j+2 into the staging registers.
  auto tile = [&](auto stage_c, int j) {
    constexpr int S = decltype(stage_c)::value;
    constexpr int SN = (S + 1) % 3;  // stage of tile j+1
    const char* Kt = S == 0 ? sK0 : S == 1 ? sK1 : sK2;
    const char* Vt = S == 0 ? sV0 : S == 1 ? sV1 : sV2;
    char* Knext = SN == 0 ? sK0 : SN == 1 ? sK1 : sK2;
    char* Vnext = SN == 0 ? sV0 : SN == 1 ? sV1 : sV2;
#pragma unroll
    for (int sb = 0; sb < NSUB; sb++) {
      const int g = j * NSUB + sb;
      const bool cross = sb == NSUB - 1;
      if (cross && g + 1 < n_steps) {
        store_tile_regs<D, BC, NW>(Knext, Vnext, wave, lane, stage);
        __syncthreads();  // tile j+1 visible to every wave
        if (j + 2 < n_kt) load_tile_regs<D, BC, NW>(Kh, Vh, (j + 2) * BC, N, wave, lane, stage);
      }
      if (g <= L.last) {
        // step g reads S from st.s[g % 2] (NSUB is even, so g % 2 == sb % 2)
        if (sb % 2 == 0) {
          pipe_compute<D, CAUSAL, 0>(Vt, sb, cross ? Knext : Kt, cross ? 0 : sb + 1,
                                     g + 1 <= L.last, g, L, st);
        } else {
          pipe_compute<D, CAUSAL, 1>(Vt, sb, cross ? Knext : Kt, cross ? 0 : sb + 1,
                                     g + 1 <= L.last, g, L, st);
        }
      }
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

  // Epilogue: O = a / l, LSE = ln2 * (m + log2 l).
  const float lt = half_swap_sum(st.l);
  if (L.qrow < N) {
    const float inv = 1.0f / lt;
    bf16* orow = a.o + head + (size_t)L.qrow * D;
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; e++) ov[e] = (bf16)(st.acc[db][4 * g4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * g4 + 4 * L.h) = ov;
      }
    if (L.h == 0) a.lse[(size_t)bh * N + L.qrow] = kLn2 * (st.m2 + fast_log2(lt));
  }
}

}  // namespace fa
