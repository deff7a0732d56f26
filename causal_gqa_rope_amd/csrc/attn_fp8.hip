// Instances of the fp8-operand attention forward (head_dim 128).
#include "attn_fp8_kernel.h"
#include "launch.h"

namespace cgr {
hipError_t launch_attn_fp8(const Fp8Args& a, int style, int causal, hipStream_t stream) {
  if (causal) {
    if (style == STYLE_HALF) return launch_fp8_inst<true, STYLE_HALF>(a, stream);
    return launch_fp8_inst<true, STYLE_INTERLEAVED>(a, stream);
  }
  if (style == STYLE_HALF) return launch_fp8_inst<false, STYLE_HALF>(a, stream);
  return launch_fp8_inst<false, STYLE_INTERLEAVED>(a, stream);
}
}  // namespace cgr
