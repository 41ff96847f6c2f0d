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

constexpr int kVersion = 100;  // 0.1.0
constexpr int kMaxN = 1 << 22;
constexpr int kMaxBH = 65535;  // grid y of the fp32 kernel; also keeps bf16 grids < 2^31

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Shared argument checks; elem is the byte size of one q/k/v/o element.
int check_args(const void* q, const void* k, const void* v, const void* o, const void* lse,
               int B, int H, int N, int d, float scale, int causal, size_t elem) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || N > kMaxN) return FA_ERR_INVALID_ARG;
  if ((int64_t)B * H > kMaxBH) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                        reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o) |
                        reinterpret_cast<uintptr_t>(lse);
  if (mis & 15) return FA_ERR_ALIGNMENT;
  const size_t nel = (size_t)B * H * N * d;
  const size_t tb = nel * elem, lb = (size_t)B * H * N * sizeof(float);
  if (ranges_overlap(o, tb, q, tb) || ranges_overlap(o, tb, k, tb) ||
      ranges_overlap(o, tb, v, tb) || ranges_overlap(o, tb, lse, lb) ||
      ranges_overlap(lse, lb, q, tb) || ranges_overlap(lse, lb, k, tb) ||
      ranges_overlap(lse, lb, v, tb))
    return FA_ERR_INVALID_ARG;
  return FA_OK;
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

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int causal, void* stream) {
  const int rc = check_args(q, k, v, o, lse, B, H, N, d, scale, causal, 2);
  if (rc != FA_OK) return rc;
  fa::Bf16Args a;
  a.q = static_cast<const fa::bf16*>(q);
  a.k = static_cast<const fa::bf16*>(k);
  a.v = static_cast<const fa::bf16*>(v);
  a.o = static_cast<fa::bf16*>(o);
  a.lse = lse;
  a.N = N;
  a.BH = B * H;
  // scale 0 runs as the smallest normal float: every probability still rounds to exactly 1 (the
  // scaled scores are below 2^-24 in magnitude), while hidden keys stay at -inf instead of 0*inf.
  a.scale_log2 = scale > 0.f ? scale * fa::kLog2e : FLT_MIN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  a.n_qblk = (N + fa::kBlockQ - 1) / fa::kBlockQ;
  if (d == 128)
    e = causal ? launch_bf16<128, true>(a, s) : launch_bf16<128, false>(a, s);
  else
    e = causal ? launch_bf16<64, true>(a, s) : launch_bf16<64, false>(a, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, void* stream) {
  const int rc = check_args(q, k, v, o, lse, B, H, N, d, scale, causal, 4);
  if (rc != FA_OK) return rc;
  fa::F32Args a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.N = N;
  a.BH = B * H;
  a.scale_log2 = scale * fa::kLog2e;
  const int n_qblk = (N + fa::kF32BlockQ - 1) / fa::kF32BlockQ;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (d == 128) {
    e = causal ? launch_f32<128, true>(a, n_qblk, s) : launch_f32<128, false>(a, n_qblk, s);
  } else {
    e = causal ? launch_f32<64, true>(a, n_qblk, s) : launch_f32<64, false>(a, n_qblk, s);
  }
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK:
      return "success";
    case FA_ERR_INVALID_ARG:
      return "invalid argument (null or overlapping pointer, B/H/N out of range, causal not 0/1, "
             "or scale negative or not finite)";
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
