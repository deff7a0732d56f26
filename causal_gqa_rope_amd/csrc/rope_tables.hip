// RoPE cos/sin tables ("Embeddings & the Residual Stream", section
// "Positional information: RoPE"): for position p and pair i < d/2, the angle
// is p * base^(-2i/d). Angle, cosine and sine are evaluated in float64 and
// rounded once to float32. One thread per table entry.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace cgr {

__global__ void rope_tables_kernel(long n, int half, int head_dim, double base, float* cos_out,
                                   float* sin_out) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const long p = idx / half;
  const int i = (int)(idx - p * half);
  const double inv_freq = pow(base, -(2.0 * i) / (double)head_dim);
  const double ang = (double)p * inv_freq;
  double s, c;
  sincos(ang, &s, &c);
  cos_out[idx] = (float)c;
  sin_out[idx] = (float)s;
}

hipError_t launch_rope_tables(int max_pos, int head_dim, double base, float* cos_out,
                              float* sin_out, hipStream_t stream) {
  const int half = head_dim / 2;
  const long n = (long)max_pos * half;
  const int threads = 256;
  const long blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(rope_tables_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, n, half,
                     head_dim, base, cos_out, sin_out);
  return hipGetLastError();
}

}  // namespace cgr
