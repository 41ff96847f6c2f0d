// Launcher of the wide-row forward kernel (fa_fwd_wide.h). This file is compiled on its own, with
// the MFMA results kept in VGPRs (build.py: -amdgpu-mfma-vgpr-form): the kernel needs about 360
// registers per lane (one wave per SIMD), and with that form the allocator puts the Q operands in
// AGPRs, which MFMAs read directly, instead of the score and output accumulators, which the vector
// instructions of the softmax read and rescale (an AGPR accumulator would cost a copy each way).
#include <hip/hip_runtime.h>

#include "fa_fwd_wide.h"

namespace fa {

__attribute__((visibility("hidden"))) hipError_t launch_wide(const WideArgs& args, bool causal,
                                                           hipStream_t stream) {
  WideArgs a = args;
  void* argv[] = {&a};
  const bool window = causal && a.wl < kWideNoWindow;
  const bool alibi = causal && !window && a.slopes != nullptr;
  const void* fn = alibi    ? reinterpret_cast<const void*>(&fa_fwd_wide_kernel<true, false, true>)
                 : window ? reinterpret_cast<const void*>(&fa_fwd_wide_kernel<true, true, false>)
                 : causal ? reinterpret_cast<const void*>(&fa_fwd_wide_kernel<true, false, false>)
                          : reinterpret_cast<const void*>(&fa_fwd_wide_kernel<false, false, false>);
  return hipLaunchKernel(fn, dim3(a.n_qblk * a.BH), dim3(kWideWaves * 64), argv, 0, stream);
}

}  // namespace fa
