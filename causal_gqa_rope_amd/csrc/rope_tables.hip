// RoPE cos/sin tables ("Embeddings & the Residual Stream", section
// "Positional information: RoPE"): for position p and pair i < d/2, the angle
// is p * base^(-2i/d). Angle, cosine and sine are evaluated in float64 and
// rounded once to float32. A thread owns pair i for kPosPerThread consecutive
// positions, so base^(-2i/d) is evaluated once for all of them (the same
// float64 value for every position, as before); consecutive threads take
// consecutive pairs, so each position's row is written contiguously.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace cgr {

constexpr int kPosPerThread = 4;

__global__ void rope_tables_kernel(long max_pos, int half, int head_dim, double base, float* cos_out,
                                   float* sin_out) {
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long group = t / half;
  const int i = (int)(t - group * half);
  const long p0 = group * kPosPerThread;
  if (p0 >= max_pos) return;
  const double inv_freq = pow(base, -(2.0 * i) / (double)head_dim);
#pragma unroll
  for (int k = 0; k < kPosPerThread; ++k) {
    const long p = p0 + k;
    if (p < max_pos) {
      const double ang = (double)p * inv_freq;
      double s, c;
      sincos(ang, &s, &c);
      cos_out[p * half + i] = (float)c;
      sin_out[p * half + i] = (float)s;
    }
  }
}

hipError_t launch_rope_tables(int max_pos, int head_dim, double base, float* cos_out,
                              float* sin_out, hipStream_t stream) {
  const int half = head_dim / 2;
  const long n = ((long)max_pos + kPosPerThread - 1) / kPosPerThread * half;
  const int threads = 256;
  const long blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(rope_tables_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, (long)max_pos, half,
                     head_dim, base, cos_out, sin_out);
  return hipGetLastError();
}

}  // namespace cgr
