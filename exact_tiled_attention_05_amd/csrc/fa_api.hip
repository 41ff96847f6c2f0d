// C-ABI entry points of libfa.so: argument checks, kernel selection and launch.
// Declared (with their contract) in include/fa.h.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <algorithm>
#include <cstdint>
#include <mutex>

#include "fa.h"
#include "fa_bwd.h"
#include "fa_decode.h"
#include "fa_fwd_bf16.h"
#include "fa_fwd_ext.h"
#include "fa_fwd_f32.h"
#include "fa_fwd_wide.h"

namespace fa {
// fa_wide.hip and fa_bwd_wide.hip (compiled separately, see there)
hipError_t launch_wide(const WideArgs& args, bool causal, hipStream_t stream);
hipError_t launch_bwd_dkdv_wide(const BwdArgs& args, bool causal, hipStream_t stream);
}  // namespace fa

namespace {

constexpr int kVersion = 600;  // 0.6.0: bias rows 16-byte aligned; forward kernel chosen by shape
constexpr int kMaxN = 1 << 22;
constexpr int kMaxBH = 65535;  // grid y of the fp32 kernel; also keeps bf16 grids < 2^31

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Shared argument checks; elem is the byte size of one q/k/v/o element; d256: whether d = 256 is
// accepted (by the bf16 forward only).
int check_args(const void* q, const void* k, const void* v, const void* o, const void* lse,
               int B, int H, int H_kv, int N, int d, float scale, int causal, int layout,
               size_t elem, bool d256 = false) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || N > kMaxN) return FA_ERR_INVALID_ARG;
  if ((int64_t)B * H > kMaxBH) return FA_ERR_INVALID_ARG;
  if (H_kv < 1 || H_kv > H || H % H_kv != 0) return FA_ERR_INVALID_ARG;
  if (layout != FA_LAYOUT_BHND && layout != FA_LAYOUT_BNHD) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128 && !(d256 && d == 256)) return FA_ERR_UNSUPPORTED;
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
                         dim3(n_qblk, a.BH), dim3(fa::kF32Threads), args, 0, s);
}

// ---- score variants and d = 256 ------------------------------------------------------------------

template <int D, bool CAUSAL, bool ALIBI, bool BIAS>
hipError_t launch_ext_t(fa::ExtArgs a, hipStream_t s) {
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fa::fa_fwd_ext_kernel<D, CAUSAL, ALIBI, BIAS>),
                         dim3(a.n_qblk * a.BH), dim3(fa::kExtWaves * 64), args, 0, s);
}
template <int D, bool CAUSAL>
hipError_t launch_ext_c(fa::ExtArgs a, hipStream_t s) {
  const bool al = a.slopes != nullptr, bi = a.bias != nullptr;
  if (al) return bi ? launch_ext_t<D, CAUSAL, true, true>(a, s) : launch_ext_t<D, CAUSAL, true, false>(a, s);
  return bi ? launch_ext_t<D, CAUSAL, false, true>(a, s) : launch_ext_t<D, CAUSAL, false, false>(a, s);
}
template <int D>
hipError_t launch_ext_d(fa::ExtArgs a, int causal, hipStream_t s) {
  return causal ? launch_ext_c<D, true>(a, s) : launch_ext_c<D, false>(a, s);
}

int run_wide(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int H_kv, int N, float scale, int causal, int layout, int window_left,
             const float* slopes, void* stream);

int run_ext(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
            int H_kv, int N, int d, float scale, int causal, int layout, int window_left,
            int window_right, const float* slopes, const void* bias, long long bias_bs,
            long long bias_hs, long long bias_rs, void* stream) {
  const int rc = check_args(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout, 2, true);
  if (rc != FA_OK) return rc;
  if (window_left < -1 || window_right < -1) return FA_ERR_INVALID_ARG;
  // A causal sliding window alone at d = 128 and N >= 4096 (the right bound changes nothing under
  // the causal rule): the wide-row kernel, which starts each workgroup at its first row's first
  // key tile and masks keys before a row's window. Grouped Llama layer with a 4095-key window
  // (one box, alternating runs): see the measurement notes.
  if (causal && !slopes && !bias && d == 128 && N >= 4096 && window_left >= 0)
    return run_wide(q, k, v, o, lse, B, H, H_kv, N, scale, causal, layout, window_left, nullptr,
                    stream);
  const size_t qb = (size_t)B * H * N * d * 2, lb = (size_t)B * H * N * sizeof(float);
  if (slopes) {
    if (reinterpret_cast<uintptr_t>(slopes) & 3) return FA_ERR_ALIGNMENT;
    if (ranges_overlap(slopes, H * sizeof(float), o, qb) ||
        ranges_overlap(slopes, H * sizeof(float), lse, lb))
      return FA_ERR_INVALID_ARG;
    // Causal ALiBi alone at d = 128 and N >= 4096: the wide-row kernel, which walks the key tiles
    // from the diagonal down for it (its ALiBi term divides by the scale: scales below 1e-6 stay
    // on the 4-wave kernel).
    if (causal && !bias && d == 128 && N >= 4096 && window_left < 0 && scale >= 1e-6f)
      return run_wide(q, k, v, o, lse, B, H, H_kv, N, scale, causal, layout, -1, slopes, stream);
  }
  if (bias) {
    if (bias_bs < 0 || bias_hs < 0 || bias_rs < N) return FA_ERR_INVALID_ARG;
    // 16-byte chunks of the bias rows go straight into LDS: every row starts 16-byte aligned
    if ((reinterpret_cast<uintptr_t>(bias) & 15) || (bias_rs & 7) || (bias_bs & 7) || (bias_hs & 7))
      return FA_ERR_ALIGNMENT;
    // one head's matrix is addressed with 32-bit byte offsets
    if (((int64_t)(N - 1) * bias_rs + N) * 2 >= ((int64_t)1 << 31)) return FA_ERR_UNSUPPORTED;
    const size_t bb = (size_t)(((int64_t)(B - 1) * bias_bs + (int64_t)(H - 1) * bias_hs +
                                (int64_t)(N - 1) * bias_rs + N) * 2);
    if (ranges_overlap(bias, bb, o, qb) || ranges_overlap(bias, bb, lse, lb))
      return FA_ERR_INVALID_ARG;
  }
  fa::ExtArgs a;
  a.q = static_cast<const fa::bf16*>(q);
  a.k = static_cast<const fa::bf16*>(k);
  a.v = static_cast<const fa::bf16*>(v);
  a.o = static_cast<fa::bf16*>(o);
  a.lse = lse;
  a.bias = static_cast<const fa::bf16*>(bias);
  a.slopes = slopes;
  a.bias_bs = bias_bs;
  a.bias_hs = bias_hs;
  a.bias_rs = (int)bias_rs;
  a.N = N;
  a.H = H;
  a.Hkv = H_kv;
  a.group = H / H_kv;
  a.BH = B * H;
  a.n_qblk = (N + fa::kExtRows - 1) / fa::kExtRows;
  a.wl = window_left < 0 ? fa::kExtNoWindow : std::min(window_left, N);
  a.wr = window_right < 0 ? fa::kExtNoWindow : std::min(window_right, N);
  // scale 0 runs as the smallest normal float (as in run_bf16): the raw-score maximum of a masked
  // step stays -inf instead of 0 * inf
  a.scale_log2 = scale > 0.f ? scale * fa::kLog2e : FLT_MIN;
  const Strides sq = strides_of(layout, H, N, d), sk = strides_of(layout, H_kv, N, d);
  a.q_bs = sq.bs;
  a.q_hs = sq.hs;
  a.q_rs = sq.rs;
  a.kv_bs = sk.bs;
  a.kv_hs = sk.hs;
  a.kv_rs = sk.rs;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = d == 256 ? launch_ext_d<256>(a, causal, st)
               : d == 128 ? launch_ext_d<128>(a, causal, st)
                          : launch_ext_d<64>(a, causal, st);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int run_wide(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int H_kv, int N, float scale, int causal, int layout, int window_left,
             const float* slopes, void* stream) {
  const int rc = check_args(q, k, v, o, lse, B, H, H_kv, N, 128, scale, causal, layout, 2);
  if (rc != FA_OK) return rc;
  fa::WideArgs a;
  a.wl = window_left < 0 ? fa::kWideNoWindow : std::min(window_left, N);
  a.slopes = slopes;
  a.q = static_cast<const fa::bf16*>(q);
  a.k = static_cast<const fa::bf16*>(k);
  a.v = static_cast<const fa::bf16*>(v);
  a.o = static_cast<fa::bf16*>(o);
  a.lse = lse;
  fill_shape(a, B, H, H_kv, N, 128, layout);
  a.scale_log2 = scale > 0.f ? scale * fa::kLog2e : FLT_MIN;
  a.n_qblk = (N + fa::kWideRows - 1) / fa::kWideRows;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = fa::launch_wide(a, causal == 1, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int run_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int H_kv, int N, int d, float scale, int causal, int layout, void* stream) {
  // d = 128 and N >= 4096: the wide-row kernel (fa_fwd_wide.h). Measured on one box against the
  // 4-wave kernel, TFLOP/s: causal B=1 H=32 N=8192 1150 / 1080, N=32768 1205 / 1105, 8 K/V heads
  // N=8192 1155 / 1082, N=4096 988 / 955; non-causal B=1 H=32 N=4096 1146 / 1024, B=4 H=16
  // N=4096 1166 / 1070. Below N = 4096 its 256-row workgroups leave too few (and, causal, too
  // unequal) blocks: causal N=2048 561 / 628, N=1024 251 / 322.
  if (d == 128 && N >= 4096)
    return run_wide(q, k, v, o, lse, B, H, H_kv, N, scale, causal, layout, -1, nullptr, stream);
  // Which forward kernel: the 4-wave kernel of the variants (no variant enabled) for d = 256, for
  // causal d = 128 and for every grid of more than 2^16 query rows; the 8-wave kernel for the
  // remaining small grids. Measured on one box (alternating runs): the 4-wave kernel is 2.7-4.2%
  // faster on the causal Llama layer (32 and 8 K/V heads, N = 32768), 1-7% non-causal at d = 128
  // (N 2048-32768, B up to 16), 5-20% at d = 64 on grids past 2^16 rows, and 14-21% on causal
  // d = 128 grids as small as B=1 H=32 N=1024-2048, whose causal imbalance its 128-row blocks even
  // out; on grids of at most 2^16 rows the 8-wave kernel is 3-5% faster non-causal and at d = 64.
  if (d == 256 || (d == 128 && causal == 1) || (int64_t)B * H * N > (1 << 16))
    return run_ext(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout, -1, -1, nullptr,
                   nullptr, 0, 0, 0, stream);
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
  const int n_qblk = (N + fa::kF32Rows - 1) / fa::kF32Rows;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (d == 128)
    e = causal ? launch_f32<128, true>(a, n_qblk, s) : launch_f32<128, false>(a, n_qblk, s);
  else
    e = causal ? launch_f32<64, true>(a, n_qblk, s) : launch_f32<64, false>(a, n_qblk, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// ---- split-KV decoding ------------------------------------------------------------------------

// Splits: about 768 (batch, K/V head, split, row tile) waves in all, three per CU, but at least
// 128 keys per split; a caller's count is honoured up to one split per 32 keys. Fewer, longer K/V streams read
// faster than a full 8 waves per CU: on the Llama-3-8B decoding batch (64 K/V heads, 32768 keys)
// 12 splits take 163 us where 32 take 180 us, and 512-768 waves were best on every shape measured.
struct SplitPlan {
  int n_splits, keys_per_split;
};
SplitPlan plan_splits(int B, int H_kv, int N_kv, int R, int n_splits) {
  int n = n_splits;
  if (n <= 0) {
    const int tiles = (R + fa::kDecodeRows - 1) / fa::kDecodeRows;
    const int want = (768 + B * H_kv * tiles - 1) / (B * H_kv * tiles);
    n = std::max(1, std::min(want, (N_kv + 127) / 128));
  }
  n = std::min(n, (N_kv + 31) / 32);
  const int kps = ((N_kv + n - 1) / n + 31) / 32 * 32;
  return {(N_kv + kps - 1) / kps, kps};
}

size_t ws_lse_offset(int B, int H_kv, int R, int d, int splits) {
  return ((size_t)B * H_kv * splits * R * d * sizeof(float) + 255) / 256 * 256;
}
size_t ws_bytes(int B, int H_kv, int R, int d, int splits) {
  return ws_lse_offset(B, H_kv, R, d, splits) + (size_t)B * H_kv * splits * R * sizeof(float);
}

// Shape checks shared by the workspace query and the call; 0 when the shape is usable.
int check_decode_shape(int B, int H, int H_kv, int N_q, int N_kv, int d, int causal, int n_splits) {
  if (B < 1 || H < 1 || N_q < 1 || N_kv < 1 || N_kv > kMaxN) return FA_ERR_INVALID_ARG;
  if (H_kv < 1 || H_kv > H || H % H_kv != 0) return FA_ERR_INVALID_ARG;
  if ((int64_t)B * H > kMaxBH) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (causal && N_q > N_kv) return FA_ERR_INVALID_ARG;
  if (n_splits < 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((int64_t)(H / H_kv) * N_q > fa::kDecodeMaxRows) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

template <int D>
hipError_t launch_decode(fa::DecodeArgs a, hipStream_t s) {
  void* args[] = {&a};
  // one row tile: a wave per split; several: the splits padded to a multiple of 8 (the kernel's
  // XCD-grouped numbering), T waves each
  const int gx = a.row_tiles == 1 ? a.n_splits : (a.n_splits + 7) / 8 * 8 * a.row_tiles;
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fa::fa_decode_partial_kernel<D>),
                                 dim3(gx, a.B_Hkv()), dim3(64), args, 0, s);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&fa::fa_decode_combine_kernel<D>),
                         dim3(a.R, a.B_Hkv()), dim3(fa::kCombineThreads), args, 0, s);
}

// ---- the allocation-free split-KV entry point's scratch ---------------------------------------

// Device memory for the split partials of fa_fwd_splitkv_noalloc, for callers that cannot
// allocate. Each GPU the library runs on holds its own copy until the process ends; in host code
// the name is only a stand-in, so kernels get the per-device address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the device `stream` runs on, looked up once per device with that device
// current (which the stream's device must be). FA_ERR_INVALID_ARG for a stream of another device.
int static_scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return FA_ERR_LAUNCH;
    if (sdev != dev) return FA_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

// Shared by fa_fwd_splitkv (caller workspace) and fa_fwd_splitkv_noalloc (the library's static
// scratch): checks, split plan, launches. ws = NULL asks for the static scratch, whose size is
// checked right after the shape (before the pointers), and whose device address is looked up only
// once every argument has passed.
int run_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int H_kv, int N_q, int N_kv, int d, float scale, int causal, int layout,
                int n_splits, void* workspace, size_t workspace_bytes, bool static_scratch,
                void* stream) {
  if (!q || !k || !v || !o || !lse || (!static_scratch && !workspace)) return FA_ERR_INVALID_ARG;
  int rc = check_decode_shape(B, H, H_kv, N_q, N_kv, d, causal, n_splits);
  if (rc != FA_OK) return rc;
  const int R = (H / H_kv) * N_q;
  const SplitPlan sp = plan_splits(B, H_kv, N_kv, R, n_splits);
  const size_t need = ws_bytes(B, H_kv, R, d, sp.n_splits);
  if (static_scratch && need > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_TOO_LARGE;
  if (layout != FA_LAYOUT_BHND && layout != FA_LAYOUT_BNHD) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                        reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o) |
                        reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(workspace);
  if (mis & 15) return FA_ERR_ALIGNMENT;
  if (!static_scratch && workspace_bytes < need) return FA_ERR_INVALID_ARG;
  const size_t qb = (size_t)B * H * N_q * d * 2, kb = (size_t)B * H_kv * N_kv * d * 2;
  const size_t lb = (size_t)B * H * N_q * sizeof(float);
  const void* ins[3] = {q, k, v};
  const size_t insz[3] = {qb, kb, kb};
  for (int i = 0; i < 3; i++)
    if (ranges_overlap(o, qb, ins[i], insz[i]) || ranges_overlap(lse, lb, ins[i], insz[i]) ||
        (!static_scratch && ranges_overlap(workspace, need, ins[i], insz[i])))
      return FA_ERR_INVALID_ARG;
  if (ranges_overlap(o, qb, lse, lb) ||
      (!static_scratch && (ranges_overlap(workspace, need, o, qb) ||
                           ranges_overlap(workspace, need, lse, lb))))
    return FA_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (static_scratch) {
    rc = static_scratch_address(s, &workspace);
    if (rc != FA_OK) return rc;
  }

  fa::DecodeArgs a;
  a.q = static_cast<const fa::bf16*>(q);
  a.k = static_cast<const fa::bf16*>(k);
  a.v = static_cast<const fa::bf16*>(v);
  a.o = static_cast<fa::bf16*>(o);
  a.lse = lse;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      ws_lse_offset(B, H_kv, R, d, sp.n_splits));
  a.Nq = N_q;
  a.Nkv = N_kv;
  a.H = H;
  a.Hkv = H_kv;
  a.group = H / H_kv;
  a.B = B;
  a.R = R;
  a.row_tiles = (R + fa::kDecodeRows - 1) / fa::kDecodeRows;
  a.n_splits = sp.n_splits;
  a.keys_per_split = sp.keys_per_split;
  a.causal = causal;
  a.causal_off = N_kv - N_q;
  a.scale_log2 = scale > 0.f ? scale * fa::kLog2e : FLT_MIN;
  const Strides sq = strides_of(layout, H, N_q, d), sk = strides_of(layout, H_kv, N_kv, d);
  a.q_bs = sq.bs;
  a.q_hs = sq.hs;
  a.q_rs = sq.rs;
  a.kv_bs = sk.bs;
  a.kv_hs = sk.hs;
  a.kv_rs = sk.rs;
  const hipError_t e = d == 128 ? launch_decode<128>(a, s) : launch_decode<64>(a, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// ---- backward ----------------------------------------------------------------------------------

// Query-head splits of the dK/dV kernel: enough (K/V head, key block, split) workgroups for about
// four per CU with the 8-wave kernel (d = 64), two per CU with the wide one (d = 128: fewer,
// longer workgroups balance as well, and every split adds a partial dK/dV to write and add up), a
// divisor of the group size. MHA, and grouped heads with many K/V heads or long sequences, need
// none; the grouped Llama-3-8B layer (8 K/V heads, 32 key blocks) takes 2 (measured against 4:
// 1680 against 1715 us per backward call).
int bwd_hsplit(int B, int H, int H_kv, int N, int d) {
  const int group = H / H_kv;
  const int n_kblk = (N + fa::kBwdKvRows - 1) / fa::kBwdKvRows;
  const int64_t wgs = (int64_t)n_kblk * B * H_kv;
  const int64_t target = d == 128 ? 512 : 1024;
  int want = (int)std::min<int64_t>(group, (target + wgs - 1) / wgs);
  while (group % want) want--;
  return std::max(want, 1);
}
size_t bwd_dsum_bytes(int B, int H, int N) {
  return ((size_t)B * H * N * sizeof(float) + 255) / 256 * 256;
}
size_t bwd_ws_bytes(int B, int H, int H_kv, int N, int d) {
  const int hs = bwd_hsplit(B, H, H_kv, N, d);
  return bwd_dsum_bytes(B, H, N) + (hs > 1 ? 2 * (size_t)hs * B * H_kv * N * d * sizeof(float) : 0);
}

template <int D, bool CAUSAL>
hipError_t launch_bwd(fa::BwdArgs a, hipStream_t s) {
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fa::fa_bwd_dq_kernel<D, CAUSAL>),
                                 dim3(a.n_qblk * a.BH), dim3(fa::kBwdQWaves * 64), args, 0, s);
  if (e != hipSuccess) return e;
  // dK/dV: at d = 128 the wide kernel (fa_bwd_wide.h: 4 waves of 64 keys, bit-identical results),
  // at d = 64 the 8-wave one
  if constexpr (D == 128)
    e = fa::launch_bwd_dkdv_wide(a, CAUSAL, s);
  else
    e = hipLaunchKernel(reinterpret_cast<const void*>(&fa::fa_bwd_dkdv_kernel<D, CAUSAL>),
                        dim3(a.n_kblk * a.BHkv * a.hsplit), dim3(fa::kBwdKvWaves * 64), args, 0, s);
  if (e != hipSuccess || a.hsplit == 1) return e;
  const long long n4 = (long long)a.BHkv * a.N * (D / 4);
  return hipLaunchKernel(reinterpret_cast<const void*>(&fa::fa_bwd_combine_kernel<D>),
                         dim3((unsigned)((n4 + 255) / 256)), dim3(256), args, 0, s);
}

}  // namespace

extern "C" {

int fa_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int H_kv, int N, int d, float scale, int causal, int layout, int window_left,
               int window_right, const float* alibi_slopes, const void* bias,
               long long bias_batch_stride, long long bias_head_stride, long long bias_row_stride,
               void* stream) {
  return run_ext(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout, window_left,
                 window_right, alibi_slopes, bias, bias_batch_stride, bias_head_stride,
                 bias_row_stride, stream);
}

size_t fa_bwd_workspace_bytes(int B, int H, int H_kv, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || N > kMaxN || (int64_t)B * H > kMaxBH) return 0;
  if (H_kv < 1 || H_kv > H || H % H_kv != 0 || (d != 64 && d != 128)) return 0;
  return bwd_ws_bytes(B, H, H_kv, N, d);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d,
           float scale, int causal, int layout, void* workspace, size_t workspace_bytes,
           void* stream) {
  if (!dout || !dq || !dk || !dv || !workspace) return FA_ERR_INVALID_ARG;
  int rc = check_args(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout, 2);
  if (rc != FA_OK) return rc;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(dout) | reinterpret_cast<uintptr_t>(dq) |
                        reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv) |
                        reinterpret_cast<uintptr_t>(workspace);
  if (mis & 15) return FA_ERR_ALIGNMENT;
  const size_t wb = bwd_ws_bytes(B, H, H_kv, N, d);
  if (workspace_bytes < wb) return FA_ERR_INVALID_ARG;
  const size_t qb = (size_t)B * H * N * d * 2, kb = (size_t)B * H_kv * N * d * 2;
  const size_t lb = (size_t)B * H * N * sizeof(float);
  const void* ins[6] = {q, k, v, o, dout, lse};
  const size_t insz[6] = {qb, kb, kb, qb, qb, lb};
  const void* outs[4] = {dq, dk, dv, workspace};
  const size_t outsz[4] = {qb, kb, kb, wb};
  for (int i = 0; i < 4; i++) {
    for (int j = 0; j < 6; j++)
      if (ranges_overlap(outs[i], outsz[i], ins[j], insz[j])) return FA_ERR_INVALID_ARG;
    for (int j = i + 1; j < 4; j++)
      if (ranges_overlap(outs[i], outsz[i], outs[j], outsz[j])) return FA_ERR_INVALID_ARG;
  }

  fa::BwdArgs a;
  a.q = static_cast<const fa::bf16*>(q);
  a.k = static_cast<const fa::bf16*>(k);
  a.v = static_cast<const fa::bf16*>(v);
  a.o = static_cast<const fa::bf16*>(o);
  a.dout = static_cast<const fa::bf16*>(dout);
  a.lse = lse;
  a.dq = static_cast<fa::bf16*>(dq);
  a.dk = static_cast<fa::bf16*>(dk);
  a.dv = static_cast<fa::bf16*>(dv);
  a.dsum = static_cast<float*>(workspace);
  a.hsplit = bwd_hsplit(B, H, H_kv, N, d);
  a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_dsum_bytes(B, H, N));
  a.N = N;
  a.H = H;
  a.Hkv = H_kv;
  a.group = H / H_kv;
  a.BH = B * H;
  a.BHkv = B * H_kv;
  a.n_qblk = (N + fa::kBwdQRows - 1) / fa::kBwdQRows;
  a.n_kblk = (N + fa::kBwdKvRows - 1) / fa::kBwdKvRows;
  a.scale = scale;
  a.scale_log2 = scale * fa::kLog2e;
  const Strides sq = strides_of(layout, H, N, d), sk = strides_of(layout, H_kv, N, d);
  a.q_bs = sq.bs;
  a.q_hs = sq.hs;
  a.q_rs = sq.rs;
  a.kv_bs = sk.bs;
  a.kv_hs = sk.hs;
  a.kv_rs = sk.rs;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (d == 128)
    e = causal ? launch_bwd<128, true>(a, s) : launch_bwd<128, false>(a, s);
  else
    e = causal ? launch_bwd<64, true>(a, s) : launch_bwd<64, false>(a, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_splitkv_workspace_bytes(int B, int H, int H_kv, int N_q, int N_kv, int d, int causal,
                                  int n_splits) {
  if (check_decode_shape(B, H, H_kv, N_q, N_kv, d, causal, n_splits) != FA_OK) return 0;
  const int R = (H / H_kv) * N_q;
  const SplitPlan sp = plan_splits(B, H_kv, N_kv, R, n_splits);
  return ws_bytes(B, H_kv, R, d, sp.n_splits);
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int H_kv, int N_q, int N_kv, int d, float scale, int causal, int layout,
                   int n_splits, void* workspace, size_t workspace_bytes, void* stream) {
  return run_splitkv(q, k, v, o, lse, B, H, H_kv, N_q, N_kv, d, scale, causal, layout, n_splits,
                     workspace, workspace_bytes, false, stream);
}

int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int H_kv, int N_q, int N_kv, int d, float scale, int causal,
                           int layout, int n_splits, void* stream) {
  return run_splitkv(q, k, v, o, lse, B, H, H_kv, N_q, N_kv, d, scale, causal, layout, n_splits,
                     nullptr, 0, true, stream);
}

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
             "of H_kv, layout not 0/1, causal not 0/1, scale negative or not finite, or a "
             "workspace that is too small)";
    case FA_ERR_UNSUPPORTED:
      return "unsupported shape (head dimension not 64 or 128 -- or 256 on the bf16 forward "
             "entry points --, or more than 512 query rows per K/V head in split-KV decoding)";
    case FA_ERR_ALIGNMENT:
      return "pointer not 16-byte aligned";
    case FA_ERR_LAUNCH:
      return "kernel launch failed (or a HIP runtime query it needed failed)";
    case FA_ERR_TOO_LARGE:
      return "shape too large for the static scratch of fa_fwd_splitkv_noalloc "
             "(FA_NOALLOC_SCRATCH_BYTES); use fa_fwd_splitkv with a workspace";
    default:
      return "unknown error code";
  }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
