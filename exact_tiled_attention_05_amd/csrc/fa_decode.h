// Split-KV attention for few queries against a long key/value sequence (decoding), gfx950.
//
// "FlashAttention-2 -- Deeper Math" ("What FA-2 does not fix"): with one query (or a handful)
// against a long K/V sequence the query-block axis collapses and the work is bound by reading K and
// V from memory; it needs the opposite split, over the keys, with the partial softmaxes merged
// afterwards. The merge is the blockwise recurrence of "Understanding FlashAttention Pt 1", §2.4:
// a split s with row maximum m_s, row sum l_s and normalised output O_s = a_s / l_s is carried as
// (O_s, LSE_s = m_s + ln l_s), and
//     LSE = M + ln sum_s e^{LSE_s - M},   O = sum_s e^{LSE_s - LSE} O_s      (M = max_s LSE_s).
//
// Two kernels.
//   fa_decode_partial_kernel: one wave per (batch, K/V head, key split, 32-row tile). The G =
//     H / H_kv query heads of that K/V head and their N_q query rows are stacked into R = G N_q
//     rows (row r = g * N_q + i), cut into 32-row MFMA tiles; with R <= 32 one wave reads every
//     K/V byte of its split once for all of them. With more rows the waves of one split's tiles
//     are numbered so that they run on the same XCD one after another, and all but the first find
//     the split's K/V in that XCD's L2. Per 32-key step: K and V come from memory in whole rows (non-temporal buffer loads)
//     into wave-private LDS tiles, laid out as in the prefill kernel, and are read back as MFMA
//     operands (V with the transposing read); S^T = K Q^T and O^T += V^T P^T on
//     v_mfma_f32_32x32x16_bf16, the online softmax with an exact running maximum. The next step's
//     K and V loads are issued while the current step computes. The wave writes, for its valid rows,
//     O_s (fp32) and LSE_s to the workspace; a row with no visible key in the split writes O_s = 0
//     and LSE_s = -inf (the -inf guard of "Online Softmax & FlashAttention", Listing 26.3: the
//     exponent reference is 0 while a row has seen no key).
//   fa_decode_combine_kernel: one workgroup of 256 threads per (batch, K/V head, stacked row):
//     the recurrence above over the splits, in fp32, with all of the row's partials loaded at
//     once; O rounded to bf16, LSE written.
//
// Masking with N_q < N_kv: query i is token N_kv - N_q + i of the sequence, and with a causal mask
// it sees keys j <= N_kv - N_q + i (the queries are the last N_q tokens); without one it sees every
// key.
#pragma once

#include "fa_fwd_bf16.h"

namespace fa {

constexpr int kDecodeRows = 32;       // stacked query rows per wave (one MFMA tile)
constexpr int kDecodeMaxRows = 512;   // stacked query rows per K/V head, 16 tiles
// Cache-policy operand of the decode kernel's K/V loads: bit 1 is the non-temporal hint (each K/V
// byte is read once per call, so its lines go first when L2 needs room).
constexpr int kStreamLoad = 2;

struct DecodeArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  float* ws_o;    // [B * H_kv][n_splits][R][D] fp32 partial outputs
  float* ws_lse;  // [B * H_kv][n_splits][R] fp32 partial logsumexps
  int Nq, Nkv;
  int B, H, Hkv, group;  // batch, query heads, K/V heads, query heads per K/V head
  int R;                 // stacked rows = group * Nq (<= kDecodeMaxRows)
  int row_tiles;         // ceil(R / 32)
  int n_splits, keys_per_split;
  int causal, causal_off;  // causal_off = Nkv - Nq
  float scale_log2;
  long long q_bs, q_hs;
  long long kv_bs, kv_hs;
  int q_rs, kv_rs;
  __host__ __device__ int B_Hkv() const { return B * Hkv; }
};

// Element offset of stacked row r (query head hk * group + r / Nq, query r % Nq) of batch b.
__device__ __forceinline__ long long decode_q_offset(const DecodeArgs& a, int b, int hk, int r) {
  const int g = r / a.Nq, i = r - g * a.Nq;
  return b * a.q_bs + (long long)(hk * a.group + g) * a.q_hs + (long long)i * a.q_rs;
}

template <int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void fa_decode_partial_kernel(DecodeArgs a) {
  constexpr int DK = D / 16, DB = D / 32, CPR = D / 8;
  constexpr int KROW = Layout<D>::KROW, VROW = Layout<D>::VROW;
  constexpr int LOADS = 32 * D * 2 / 1024;  // 1 KB pieces of a 32-key K or V tile
  constexpr int RPP = 64 / CPR;             // rows per piece
  __shared__ __attribute__((aligned(1024))) char sK[32 * KROW];
  __shared__ __attribute__((aligned(1024))) char sV[32 * VROW];

  const int lane = threadIdx.x;
  const int bk = blockIdx.y;
  // (split, row tile) of this wave. One tile: x is the split. Several: x = 8 (T (s / 8) + t) +
  // s mod 8 for split s and tile t of T, so that (with the grid's x extent a multiple of 8 and
  // workgroups dealt to the 8 XCDs in turn) every tile of a split runs on XCD s mod 8, the T of
  // them consecutively there. x past the last split exits (the whole one-wave workgroup).
  int s = blockIdx.x, rt = 0;
  if (a.row_tiles > 1) {
    const int T = a.row_tiles, u = blockIdx.x >> 3;
    rt = u % T;
    s = (u / T) * 8 + (blockIdx.x & 7);
    if (s >= a.n_splits) return;
  }
  const int b = bk / a.Hkv, hk = bk - b * a.Hkv;
  const int key_begin = s * a.keys_per_split;
  const int key_end = min(a.Nkv, key_begin + a.keys_per_split);
  const int n_steps = (key_end - key_begin + 31) / 32;

  Lane L;
  L.c = lane & 31;
  L.h = lane >> 5;
  L.sl2 = a.scale_log2;
  {
    const int Lg = lane & 15;
    L.kbase = L.c * KROW + 16 * L.h;
    L.vbase = (4 * L.h + (Lg >> 2)) * VROW + 2 * (16 * ((lane >> 4) & 1) + 4 * (Lg & 3));
  }
  const int row = 32 * rt + L.c;  // this lane's stacked row
  const bool row_ok = row < a.R;
  // query index of this lane's stacked row (for the causal limit)
  const int qi = row_ok ? row % a.Nq : 0;
  const int key_limit = a.causal ? min(key_end - 1, qi + a.causal_off) : key_end - 1;

  bf16x8 qf[DK];
  {
    const bf16* qrow = a.q + (row_ok ? decode_q_offset(a, b, hk, row) : 0);
#pragma unroll
    for (int dk = 0; dk < DK; dk++)
      qf[dk] = row_ok ? *reinterpret_cast<const bf16x8*>(qrow + dk * 16 + L.h * 8) : bf16x8{};
  }

  // K and V of each 32-key step: whole rows, one 16-byte chunk per lane and 1 KB piece, through
  // buffer resources that start at the step's first key and end at the split's last key (keys
  // past it read as zeros and are masked), so offsets stay below 32 rows whatever the row stride.
  // Whole-row loads matter: loading K straight into the MFMA operand layout (32 rows x 32 bytes
  // per instruction) fetches each 128-byte line four times, and with the non-temporal hint those
  // lines are gone before the next request.
  const long long rs = 2LL * a.kv_rs;
  const long long kvhead = b * a.kv_bs + hk * a.kv_hs;
  const char* kb = reinterpret_cast<const char*>(a.k + kvhead) + key_begin * rs;
  const char* vb = reinterpret_cast<const char*>(a.v + kvhead) + key_begin * rs;
  const int voff = (int)((lane / CPR) * rs) + 16 * (lane % CPR);  // row lane / CPR of a piece
  auto load_step = [&](int step, u32x4 (&kr)[LOADS], u32x4 (&vr)[LOADS]) {
    const int rows = min(32, key_end - key_begin - 32 * step);  // >= 1 for every step taken
    const int bytes = (int)((rows - 1) * rs) + 2 * D;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kb + step * 32 * rs), 0, bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vb + step * 32 * rs), 0, bytes, 0x00020000);
#pragma unroll
    for (int p = 0; p < LOADS; p++) {
      const int soff = (int)(p * RPP * rs);
      kr[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, voff, soff, kStreamLoad));
      vr[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, soff, kStreamLoad));
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; db++) acc[db] = f32x16{};
  float m2 = -INFINITY, l = 0.f;
  u32x4 kr[LOADS], vr[LOADS];
  if (n_steps > 0) load_step(0, kr, vr);
  for (int t = 0; t < n_steps; t++) {
    // K(t), V(t) into the wave's LDS tiles (the previous step's reads of them are complete: this
    // wave issued them and waited for them before its products), then step t+1 from memory.
#pragma unroll
    for (int p = 0; p < LOADS; p++) {
      const int slot = p * 64 + lane;
      *(FA_LDS u32x4*)(sK + (slot / CPR) * KROW + 16 * (slot % CPR)) = kr[p];
      *(FA_LDS u32x4*)(sV + (slot / CPR) * VROW + 16 * (slot % CPR)) = vr[p];
    }
    if (t + 1 < n_steps) load_step(t + 1, kr, vr);
    bf16x8 kf[DK];
    bf16x8 vf[DB][2];
    read_k<D>(sK, 0, L, kf);
    read_v<D>(sV, 0, L, vf);

    // S^T(t) = K Q^T
    f32x16 sc = f32x16{};
#pragma unroll
    for (int dk = 0; dk < DK; dk++) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[dk], qf[dk], sc, 0, 0, 0);

    // Mask keys past the split or the row's causal limit; exact running maximum with the -inf
    // reference guard.
    const int kb0 = key_begin + 32 * t;
    const int lim = key_limit - kb0 - 4 * L.h;
#pragma unroll
    for (int i = 0; i < 16; i++)
      if (8 * (i >> 2) + (i & 3) > lim) sc[i] = -INFINITY;
    const float t2 = half_swap_max(max16(sc)) * L.sl2;
    const float mn = __builtin_fmaxf(m2, t2);
    const float ref = mn == -INFINITY ? 0.f : mn;
    if (__any(mn > m2)) {
      const float alpha = m2 == -INFINITY ? 0.f : fast_exp2(m2 - ref);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; db++) acc[db] *= alpha;
    }
    m2 = mn;
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; i++) p[i] = fast_exp2(__builtin_fmaf(sc[i], L.sl2, -ref));
    bf16x8 pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
      for (int e = 0; e < 8; e++) pf[ks][e] = (bf16)p[8 * ks + e];
    l += sum16(p);
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
      for (int db = 0; db < DB; db++)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][ks], pf[ks], acc[db], 0, 0, 0);
  }

  // Partial of this split for the valid rows: O_s = a / l, LSE_s = ln2 * (m + log2 l), or
  // (0, -inf) if the row saw no key here.
  const float lt = half_swap_sum(l);
  if (row_ok) {
    const long long slot = ((long long)bk * a.n_splits + s) * a.R + row;
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    float* orow = a.ws_o + slot * D;
#pragma unroll
    for (int db = 0; db < DB; db++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        float4 ov;
        ov.x = acc[db][4 * g4 + 0] * inv;
        ov.y = acc[db][4 * g4 + 1] * inv;
        ov.z = acc[db][4 * g4 + 2] * inv;
        ov.w = acc[db][4 * g4 + 3] * inv;
        *reinterpret_cast<float4*>(orow + 32 * db + 8 * g4 + 4 * L.h) = ov;
      }
    if (L.h == 0) a.ws_lse[slot] = lt > 0.f ? kLn2 * (m2 + fast_log2(lt)) : -INFINITY;
  }
}

// Merge of the splits' partials for one (batch, K/V head, stacked row) by 256 threads: thread
// (sg, cg) owns columns 4 cg .. 4 cg + 3 of the splits s = sg, sg + SG, ... (SG = 256 / (D / 4)
// split groups), so every partial of the row is loaded at once; the split groups' sums are then
// added through LDS. M is the largest LSE_s (finite: split 0 holds key 0, which every query sees).
constexpr int kCombineThreads = 256;

template <int D>
__global__ __launch_bounds__(kCombineThreads) void fa_decode_combine_kernel(DecodeArgs a) {
  constexpr int CG = D / 4, SG = kCombineThreads / CG;
  const int r = blockIdx.x, bk = blockIdx.y;
  const int b = bk / a.Hkv, hk = bk - b * a.Hkv;
  const int tid = threadIdx.x, cg = tid % CG, sg = tid / CG;
  const long long base = (long long)bk * a.n_splits * a.R + r;  // slot of split 0
  __shared__ float red[kCombineThreads / 64];
  __shared__ float4 part[SG][CG];
  __shared__ float wpart[SG];

  float mx = -INFINITY;
  for (int s = tid; s < a.n_splits; s += kCombineThreads)
    mx = fmaxf(mx, a.ws_lse[base + (long long)s * a.R]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / 64; w++) M = fmaxf(M, red[w]);

  float4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  constexpr int U = 4;  // splits per batch of independent loads
  for (int s0 = sg; s0 < a.n_splits; s0 += U * SG) {
    float ls[U];
    float4 ov[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int s = s0 + u * SG;
      const long long slot = base + (long long)min(s, a.n_splits - 1) * a.R;
      ls[u] = s < a.n_splits ? a.ws_lse[slot] : -INFINITY;
      ov[u] = *reinterpret_cast<const float4*>(a.ws_o + slot * D + 4 * cg);
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const float w = ls[u] == -INFINITY ? 0.f : expf(ls[u] - M);
      wsum += w;
      acc.x += w * ov[u].x;
      acc.y += w * ov[u].y;
      acc.z += w * ov[u].z;
      acc.w += w * ov[u].w;
    }
  }
  part[sg][cg] = acc;
  if (cg == 0) wpart[sg] = wsum;
  __syncthreads();
  if (sg == 0) {
    float wt = wpart[0];
    for (int g = 1; g < SG; g++) {
      const float4 p = part[g][cg];
      acc.x += p.x;
      acc.y += p.y;
      acc.z += p.z;
      acc.w += p.w;
      wt += wpart[g];
    }
    const float inv = 1.0f / wt;
    const bf16x4 ob = {(bf16)(acc.x * inv), (bf16)(acc.y * inv), (bf16)(acc.z * inv),
                       (bf16)(acc.w * inv)};
    *reinterpret_cast<bf16x4*>(a.o + decode_q_offset(a, b, hk, r) + 4 * cg) = ob;
    if (cg == 0) {
      const int g = r / a.Nq, i = r - g * a.Nq;
      a.lse[((long long)b * a.H + hk * a.group + g) * a.Nq + i] = M + logf(wt);
    }
  }
}

}  // namespace fa
