// C-ABI entry points of libfa.so: argument checks, kernel selection and launch.
// Declared (with their contract) in include/fa.h.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>

#include "fa.h"
#include "fa_fwd_bf16.h"
#include "fa_fwd_f32.h"

namespace {

constexpr int kVersion = 200;  // 0.2.0: grouped K/V heads and the [B][N][H][d] layout
constexpr int kMaxN = 1 << 22;
constexpr int kMaxBH = 65535;  // grid y of the fp32 kernel; also keeps bf16 grids < 2^31

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Shared argument checks; elem is the byte size of one q/k/v/o element.
int check_args(const void* q, const void* k, const void* v, const void* o, const void* lse,
               int B, int H, int H_kv, int N, int d, float scale, int causal, int layout,
               size_t elem) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || N > kMaxN) return FA_ERR_INVALID_ARG;
  if ((int64_t)B * H > kMaxBH) return FA_ERR_INVALID_ARG;
  if (H_kv < 1 || H_kv > H || H % H_kv != 0) return FA_ERR_INVALID_ARG;
  if (layout != FA_LAYOUT_BHND && layout != FA_LAYOUT_BNHD) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                        reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o) |
                        reinterpret_cast<uintptr_t>(lse);
  if (mis & 15) return FA_ERR_ALIGNMENT;
  const size_t qb = (size_t)B * H * N * d * elem;     // q and o
  const size_t kb = (size_t)B * H_kv * N * d * elem;  // k and v
  const size_t lb = (size_t)B * H * N * sizeof(float);
  if (ranges_overlap(o, qb, q, qb) || ranges_overlap(o, qb, k, kb) ||
      ranges_overlap(o, qb, v, kb) || ranges_overlap(o, qb, lse, lb) ||
      ranges_overlap(lse, lb, q, qb) || ranges_overlap(lse, lb, k, kb) ||
      ranges_overlap(lse, lb, v, kb))
    return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// Element strides (batch, head, row) of a [B][heads][N][d] or [B][N][heads][d] tensor.
struct Strides {
  long long bs, hs;
  int rs;
};
Strides strides_of(int layout, int heads, int N, int d) {
  if (layout == FA_LAYOUT_BHND) return {(long long)heads * N * d, (long long)N * d, d};
  return {(long long)N * heads * d, (long long)d, heads * d};
}

template <class Args>
void fill_shape(Args& a, int B, int H, int H_kv, int N, int d, int layout) {
  a.N = N;
  a.BH = B * H;
  a.H = H;
  a.group = H / H_kv;
  const Strides sq = strides_of(layout, H, N, d), sk = strides_of(layout, H_kv, N, d);
  a.q_bs = sq.bs;
  a.q_hs = sq.hs;
  a.q_rs = sq.rs;
  a.kv_bs = sk.bs;
  a.kv_hs = sk.hs;
  a.kv_rs = sk.rs;
}

template <int D, bool CAUSAL>
hipError_t launch_bf16(fa::Bf16Args a, hipStream_t s) {
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fa::fa_fwd_bf16_kernel<D, CAUSAL>),
                         dim3(a.n_qblk * a.BH), dim3(fa::kNumWaves * 64), args, 0, s);
}

template <int D, bool CAUSAL>
hipError_t launch_f32(fa::F32Args a, int n_qblk, hipStream_t s) {
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fa::fa_fwd_f32_kernel<D, CAUSAL>),
                         dim3(n_qblk, a.BH), dim3(fa::kF32BlockQ), args, 0, s);
}

int run_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int H_kv, int N, int d, float scale, int causal, int layout, void* stream) {
  const int rc = check_args(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout, 2);
  if (rc != FA_OK) return rc;
  fa::Bf16Args a;
  a.q = static_cast<const fa::bf16*>(q);
  a.k = static_cast<const fa::bf16*>(k);
  a.v = static_cast<const fa::bf16*>(v);
  a.o = static_cast<fa::bf16*>(o);
  a.lse = lse;
  fill_shape(a, B, H, H_kv, N, d, layout);
  // scale 0 runs as the smallest normal float: every probability still rounds to exactly 1 (the
  // scaled scores are below 2^-24 in magnitude), while hidden keys stay at -inf instead of 0*inf.
  a.scale_log2 = scale > 0.f ? scale * fa::kLog2e : FLT_MIN;
  a.n_qblk = (N + fa::kBlockQ - 1) / fa::kBlockQ;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (d == 128)
    e = causal ? launch_bf16<128, true>(a, s) : launch_bf16<128, false>(a, s);
  else
    e = causal ? launch_bf16<64, true>(a, s) : launch_bf16<64, false>(a, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int run_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
            int H_kv, int N, int d, float scale, int causal, int layout, void* stream) {
  const int rc = check_args(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout, 4);
  if (rc != FA_OK) return rc;
  fa::F32Args a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  fill_shape(a, B, H, H_kv, N, d, layout);
  a.scale_log2 = scale * fa::kLog2e;
  const int n_qblk = (N + fa::kF32BlockQ - 1) / fa::kF32BlockQ;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (d == 128)
    e = causal ? launch_f32<128, true>(a, n_qblk, s) : launch_f32<128, false>(a, n_qblk, s);
  else
    e = causal ? launch_f32<64, true>(a, n_qblk, s) : launch_f32<64, false>(a, n_qblk, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int causal, void* stream) {
  return run_bf16(q, k, v, o, lse, B, H, H, N, d, scale, causal, FA_LAYOUT_BHND, stream);
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, void* stream) {
  return run_f32(q, k, v, o, lse, B, H, H, N, d, scale, causal, FA_LAYOUT_BHND, stream);
}

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int H_kv, int N, int d, float scale, int causal, int layout, void* stream) {
  return run_bf16(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout, stream);
}

int fa_fwd_gqa_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                   int H, int H_kv, int N, int d, float scale, int causal, int layout,
                   void* stream) {
  return run_f32(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout, stream);
}

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK:
      return "success";
    case FA_ERR_INVALID_ARG:
      return "invalid argument (null or overlapping pointer, B/H/N out of range, H not a multiple "
             "of H_kv, layout not 0/1, causal not 0/1, or scale negative or not finite)";
    case FA_ERR_UNSUPPORTED:
      return "unsupported head dimension (supported: 64, 128)";
    case FA_ERR_ALIGNMENT:
      return "pointer not 16-byte aligned";
    case FA_ERR_LAUNCH:
      return "kernel launch failed";
    default:
      return "unknown error code";
  }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
