// Launcher of the wide dK/dV kernel of the backward pass (fa_bwd_wide.h). Compiled on its own with
// the compiler's default MFMA form: the kernel's 256 accumulator registers go to AGPRs, which only
// the MFMAs touch, and the scores, probabilities and operands stay in VGPRs.
#include <hip/hip_runtime.h>

#include "fa_bwd_wide.h"

namespace fa {

__attribute__((visibility("hidden"))) hipError_t launch_bwd_dkdv_wide(const BwdArgs& args,
                                                                    bool causal,
                                                                    hipStream_t stream) {
  BwdArgs a = args;
  void* argv[] = {&a};
  const void* fn = causal ? reinterpret_cast<const void*>(&fa_bwd_dkdv_wide_kernel<true>)
                          : reinterpret_cast<const void*>(&fa_bwd_dkdv_wide_kernel<false>);
  return hipLaunchKernel(fn, dim3(a.n_kblk * a.BHkv * a.hsplit), dim3(kBwdWideWaves * 64), argv, 0,
                         stream);
}

}  // namespace fa
