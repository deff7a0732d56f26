// Instances of the fused RMSNorm + q/k/v projection + RoPE kernels for head_dim 128.
#include "launch.h"
#include "qkv_kernel.h"

namespace cgr {
hipError_t launch_qkv_d128(const QkvArgs& a, int style, hipStream_t stream) {
  return launch_qkv_d<128>(a, style, stream);
}
}  // namespace cgr
