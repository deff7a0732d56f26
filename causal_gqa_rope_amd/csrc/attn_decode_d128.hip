// Instances of the decode and row-rotation kernels for head_dim 128.
#include "attn_decode_kernel.h"
#include "launch.h"

namespace cgr {
hipError_t launch_decode_d128(const DecodeArgs& a, int style, hipStream_t stream) {
  return launch_decode_d<128>(a, style, stream);
}
hipError_t launch_rope_rotate_d128(const void* x, void* out, const int32_t* positions, long n_rows, int nh,
                                 int f32_io, const float* cs, const float* sn, int P, int style,
                                 int32_t* status, hipStream_t stream) {
  return launch_rope_rotate_d<128>(x, out, positions, n_rows, nh, f32_io, cs, sn, P, style, status, stream);
}
}  // namespace cgr
