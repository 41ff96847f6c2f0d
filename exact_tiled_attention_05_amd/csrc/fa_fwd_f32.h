// fp32 attention forward kernel: every step in fp32 on the vector ALUs (no bf16 anywhere).
//
// Laid out for precision rather than speed. One thread owns one query row: its q, its running
// maximum m, running sum l and unnormalised output a stay in registers, and the keys are folded in
// one at a time with the scalar online recurrence ("Understanding FlashAttention Pt 1", §2.3:
// m_j = max(m_{j-1}, x_j), l_j = l_{j-1} e^{m_{j-1} - m_j} + e^{x_j - m_j}, with a rescaled the
// same way and o = a / l at the end). A workgroup owns 128 consecutive query rows of one head;
// K/V tiles are staged through LDS and read as broadcasts; causal tiles above the workgroup's last
// row are never loaded ("FlashAttention-2 -- Deeper Math", causal tile skipping). Scores are kept
// in base 2 and the logsumexp is written in natural-log units.
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

constexpr int kF32BlockQ = 128;
constexpr int kF32BlockK = 32;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF32BlockQ) void fa_fwd_f32_kernel(F32Args a) {
  __shared__ float Ks[kF32BlockK][D];
  __shared__ float Vs[kF32BlockK][D];
  const int N = a.N;
  const int bh = blockIdx.y;
  // causal: heaviest query blocks first
  const int qblk = CAUSAL ? (gridDim.x - 1 - blockIdx.x) : blockIdx.x;
  const int q0 = qblk * kF32BlockQ;
  const int qrow = q0 + threadIdx.x;
  const int b = bh / a.H, h = bh - b * a.H, hk = h / a.group;
  const long long qhead = b * a.q_bs + h * a.q_hs;
  const long long kvhead = b * a.kv_bs + hk * a.kv_hs;
  const float* Qh = a.q + qhead;
  const float* Kh = a.k + kvhead;
  const float* Vh = a.v + kvhead;

  float qr[D], o[D];
#pragma unroll
  for (int t = 0; t < D; t++) {
    qr[t] = (qrow < N) ? Qh[(long long)qrow * a.q_rs + t] : 0.f;
    o[t] = 0.f;
  }
  float m2 = -INFINITY, l = 0.f;

  // keys this workgroup needs: all N, or (causal) up to its last row
  const int n_keys = CAUSAL ? min(N, q0 + kF32BlockQ) : N;
  for (int k0 = 0; k0 < n_keys; k0 += kF32BlockK) {
    __syncthreads();
    for (int e = threadIdx.x; e < kF32BlockK * D; e += kF32BlockQ) {
      const int r = e / D, t = e % D;
      const bool in = k0 + r < N;
      Ks[r][t] = in ? Kh[(long long)(k0 + r) * a.kv_rs + t] : 0.f;
      Vs[r][t] = in ? Vh[(long long)(k0 + r) * a.kv_rs + t] : 0.f;
    }
    __syncthreads();
    const int kend = min(kF32BlockK, n_keys - k0);
#pragma unroll 1
    for (int r = 0; r < kend; r++) {
      if (CAUSAL && k0 + r > qrow) break;  // later keys of this tile are in the future too
      float dot = 0.f;
#pragma unroll
      for (int t = 0; t < D; t++) dot = __builtin_fmaf(qr[t], Ks[r][t], dot);
      const float s2 = dot * a.scale_log2;
      if (s2 > m2) {  // the maximum moves: rescale what was accumulated under the old one
        const float alpha = exp2f(m2 - s2);  // 0 for the first key (m2 = -inf)
        l *= alpha;
#pragma unroll
        for (int t = 0; t < D; t++) o[t] *= alpha;
        m2 = s2;
      }
      const float p = exp2f(s2 - m2);
      l += p;
#pragma unroll
      for (int t = 0; t < D; t++) o[t] = __builtin_fmaf(p, Vs[r][t], o[t]);
    }
  }

  if (qrow < N) {
    const float inv = 1.0f / l;
    float* orow = a.o + qhead + (long long)qrow * a.q_rs;
#pragma unroll
    for (int t = 0; t < D; t++) orow[t] = o[t] * inv;
    a.lse[(long long)bh * N + qrow] = kLn2 * (m2 + log2f(l));
  }
}

}  // namespace fa
