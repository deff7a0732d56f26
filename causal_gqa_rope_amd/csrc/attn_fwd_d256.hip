// Instances of the fused attention forward for head_dim 256 (bf16 I/O).
#include "attn_fwd_kernel.h"
#include "launch.h"

namespace cgr {
hipError_t launch_attn_d256(const AttnArgs& a, int f32_io, int qk_bf16, int style, int causal,
                           bool varlen, int grid, hipStream_t stream, int phases, bool small) {
  return launch_attn_d<256>(a, f32_io, qk_bf16, style, causal, varlen, grid, stream, phases, small);
}
}  // namespace cgr
