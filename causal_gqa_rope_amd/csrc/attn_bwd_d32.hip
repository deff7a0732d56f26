// Instances of the attention backward for head_dim 32.
#include "attn_bwd_kernel.h"
#include "launch.h"

namespace cgr {
hipError_t launch_attn_bwd_d32(const BwdArgs& a, int qk_bf16, int style, int causal, hipStream_t stream) {
  return launch_attn_bwd_d<32>(a, qk_bf16, style, causal, stream);
}
}  // namespace cgr
