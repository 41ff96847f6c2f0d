// fp32 attention forward kernel: every step in fp32 on the vector ALUs (no bf16 anywhere).
//
// Sixteen lanes own one query row: lane g of the group holds dims D/16 g .. D/16 (g + 1) - 1 of
// q and of the unnormalised output a, so a wave works on 4 rows and a workgroup of 4 waves on 16
// consecutive rows of one head. Keys arrive in blocks of 8 and each block is folded into the
// row's running state with the blockwise recurrence of "Understanding FlashAttention Pt 1", §2.4
// (m' = max(m, max_j s_j), alpha = e^(m - m'), l' = alpha l + sum_j e^(s_j - m'),
// a' = alpha a + sum_j e^(s_j - m') v_j, o = a / l after the last block): every lane forms the
// partial dot products of its dims with the block's 8 keys, the group adds its 16 partials with
// four cross-lane steps inside its 16-lane DPP row, and then every lane of the group holds the
// same 8 scores and updates its own share of a. K and V rows are read straight from memory (each
// lane 16 or 32 bytes of a row per key; the four groups of a wave read the same rows), one block
// ahead of the arithmetic. Causal: a wave stops after the key of its last row, and keys past a
// row are -inf for it; keys past N are -inf for every row. A row that sees no key keeps m = -inf,
// and the exponent reference is 0 then ("Online Softmax & FlashAttention", Listing 26.3's guard).
// Scores are kept in base 2 and the logsumexp is written in natural-log units.
#pragma once

#include "fa_device.h"

namespace fa {

// Same shapes, head grouping and strides as Bf16Args (fa_fwd_bf16.h).
struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int N;
  int BH;
  int H;
  int group;
  float scale_log2;
  long long q_bs, q_hs;
  long long kv_bs, kv_hs;
  int q_rs, kv_rs;
};

constexpr int kF32Lanes = 16;    // lanes per query row (one DPP row)
constexpr int kF32Rows = 16;     // query rows per workgroup: 4 waves x 4 rows
constexpr int kF32Threads = 256;
constexpr int kF32KeyBlock = 8;  // keys per step of the recurrence

// Sum over the 16 lanes of a DPP row: after the four steps every lane holds the total.
// quad_perm [1,0,3,2] and [2,3,0,1] add within each quad; row_half_mirror (lane i <- 7 - i within
// 8) adds the other quad of the half row; row_mirror (lane i <- 15 - i) adds the other half.
__device__ __forceinline__ float row16_sum(float x) {
  auto step = [](float v, auto ctrl_c) {
    constexpr int ctrl = decltype(ctrl_c)::value;
    const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false);
    return v + __int_as_float(o);
  };
  x = step(x, std::integral_constant<int, 0xB1>{});
  x = step(x, std::integral_constant<int, 0x4E>{});
  x = step(x, std::integral_constant<int, 0x141>{});
  x = step(x, std::integral_constant<int, 0x140>{});
  return x;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF32Threads) void fa_fwd_f32_kernel(F32Args a) {
  constexpr int DPL = D / kF32Lanes;  // dims per lane: 4 (d = 64) or 8 (d = 128)
  constexpr int KB = kF32KeyBlock;
  typedef float vec __attribute__((ext_vector_type(DPL)));
  const int N = a.N;
  const int bh = blockIdx.y;
  // causal: heaviest query blocks first
  const int qblk = CAUSAL ? (gridDim.x - 1 - blockIdx.x) : blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane & (kF32Lanes - 1);
  const int wrow0 = qblk * kF32Rows + 4 * wave;  // the wave's first row
  const int qrow = wrow0 + (lane >> 4);
  const int b = bh / a.H, h = bh - b * a.H, hk = h / a.group;
  const long long qhead = b * a.q_bs + h * a.q_hs;
  const long long kvhead = b * a.kv_bs + hk * a.kv_hs;
  const float* Kh = a.k + kvhead + DPL * g;
  const float* Vh = a.v + kvhead + DPL * g;

  const vec q = qrow < N ? *reinterpret_cast<const vec*>(a.q + qhead + (long long)qrow * a.q_rs + DPL * g)
                         : vec{};
  vec acc = vec{};
  float m2 = -INFINITY, l = 0.f;

  // keys the wave needs (wave-uniform): all N, or (causal) up to its last row; none past N
  const int n_keys = wrow0 >= N ? 0 : CAUSAL ? min(N, wrow0 + 4) : N;
  const int last = CAUSAL ? min(qrow, N - 1) : N - 1;  // the row's last visible key
  vec kr[KB], vr[KB];
  auto load = [&](int k0) {
#pragma unroll
    for (int j = 0; j < KB; j++) {
      const int key = min(k0 + j, N - 1);  // past N: a valid row, masked below
      kr[j] = *reinterpret_cast<const vec*>(Kh + (long long)key * a.kv_rs);
      vr[j] = *reinterpret_cast<const vec*>(Vh + (long long)key * a.kv_rs);
    }
  };
  if (n_keys > 0) load(0);
  for (int k0 = 0; k0 < n_keys; k0 += KB) {
    float s[KB];
#pragma unroll
    for (int j = 0; j < KB; j++) {
      float part = 0.f;
#pragma unroll
      for (int t = 0; t < DPL; t++) part = __builtin_fmaf(q[t], kr[j][t], part);
      s[j] = part;
    }
    vec vb[KB];
#pragma unroll
    for (int j = 0; j < KB; j++) vb[j] = vr[j];
    if (k0 + KB < n_keys) load(k0 + KB);  // next block in flight during this one
    float mb = -INFINITY;
#pragma unroll
    for (int j = 0; j < KB; j++) {
      // the cross-lane sum runs in every lane (a lane it reads must be active); then the mask
      const float tot = row16_sum(s[j]) * a.scale_log2;
      s[j] = k0 + j <= last ? tot : -INFINITY;
      mb = fmaxf(mb, s[j]);
    }
    const float mn = fmaxf(m2, mb);
    const float ref = mn == -INFINITY ? 0.f : mn;
    if (mn > m2) {  // the maximum moves: rescale what was accumulated under the old one
      const float alpha = m2 == -INFINITY ? 0.f : exp2f(m2 - ref);
      l *= alpha;
      acc *= alpha;
      m2 = mn;
    }
#pragma unroll
    for (int j = 0; j < KB; j++) {
      const float p = exp2f(s[j] - ref);
      l += p;
#pragma unroll
      for (int t = 0; t < DPL; t++) acc[t] = __builtin_fmaf(p, vb[j][t], acc[t]);
    }
  }

  if (qrow < N) {
    const float inv = 1.0f / l;
    *reinterpret_cast<vec*>(a.o + qhead + (long long)qrow * a.q_rs + DPL * g) = acc * inv;
    if (g == 0) a.lse[(long long)bh * N + qrow] = kLn2 * (m2 + log2f(l));
  }
}

}  // namespace fa
