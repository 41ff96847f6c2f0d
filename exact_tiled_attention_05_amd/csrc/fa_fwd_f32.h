// fp32 attention forward kernel: every step in fp32 on the vector ALUs (no bf16 anywhere).
//
// Same method as the bf16 kernel ("Understanding FlashAttention Pt 1", §2.4 and §3.1;
// "FlashAttention-2 -- Deeper Math", Fixes 1-4 and causal tile skipping), laid out for
// precision rather than speed: one thread owns one query row (its q, its running maximum, sum and
// unnormalised output stay in registers), a workgroup owns 128 consecutive rows of one head, and
// 32-key K/V tiles are staged through LDS and read as broadcasts. The reference maximum is the
// exact running maximum (rescale whenever it moves).
#pragma once

#include "fa_device.h"

namespace fa {

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int N;
  int BH;
  float scale_log2;
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
  const size_t head = (size_t)bh * N * D;
  const float* Qh = a.q + head;
  const float* Kh = a.k + head;
  const float* Vh = a.v + head;

  float qr[D], o[D];
#pragma unroll
  for (int t = 0; t < D; t++) {
    qr[t] = (qrow < N) ? Qh[(size_t)qrow * D + t] : 0.f;
    o[t] = 0.f;
  }
  float m2 = -INFINITY, l = 0.f;

  const int n_kt_all = (N + kF32BlockK - 1) / kF32BlockK;
  const int n_kt = CAUSAL ? min(n_kt_all, (min(q0 + kF32BlockQ, N) - 1) / kF32BlockK + 1)
                          : n_kt_all;
  for (int j = 0; j < n_kt; j++) {
    const int k0 = j * kF32BlockK;
    __syncthreads();
    for (int e = threadIdx.x; e < kF32BlockK * D; e += kF32BlockQ) {
      const int r = e / D, t = e % D;
      const bool in = k0 + r < N;
      Ks[r][t] = in ? Kh[(size_t)(k0 + r) * D + t] : 0.f;
      Vs[r][t] = in ? Vh[(size_t)(k0 + r) * D + t] : 0.f;
    }
    __syncthreads();

    float s[kF32BlockK];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < kF32BlockK; r++) {
      float dot = 0.f;
#pragma unroll
      for (int t = 0; t < D; t++) dot = __builtin_fmaf(qr[t], Ks[r][t], dot);
      const int key = k0 + r;
      const bool vis = key < N && (!CAUSAL || key <= qrow);
      s[r] = vis ? dot * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    const float mn = fmaxf(m2, mx);
    const float ref = (mn == -INFINITY) ? 0.f : mn;  // no visible key yet: any finite reference
    const float alpha = exp2f(m2 - ref);
    l *= alpha;
#pragma unroll
    for (int t = 0; t < D; t++) o[t] *= alpha;
#pragma unroll
    for (int r = 0; r < kF32BlockK; r++) {
      const float p = (s[r] == -INFINITY) ? 0.f : exp2f(s[r] - ref);
      l += p;
#pragma unroll
      for (int t = 0; t < D; t++) o[t] = __builtin_fmaf(p, Vs[r][t], o[t]);
    }
    m2 = mn;
  }

  if (qrow < N) {
    const float inv = 1.0f / l;
    float* orow = a.o + head + (size_t)qrow * D;
#pragma unroll
    for (int t = 0; t < D; t++) orow[t] = o[t] * inv;
    a.lse[(size_t)bh * N + qrow] = kLn2 * (m2 + log2f(l));
  }
}

}  // namespace fa
