// The schedule-only prepass of a packed variable-length batch (see
// varlen_schedule.h), for calls that rotate the keys on every tile.
#include <hip/hip_runtime.h>

#include "attn_fwd_kernel.h"
#include "launch.h"
#include "varlen_schedule.h"

namespace cgr {

__global__ __launch_bounds__(kSchedThreads) void varlen_schedule_kernel(
    const int32_t* cu, int nseq, int total, int max_seqlen, int lbm, int lbn, int causal,
    int32_t* sched, int max_items, int32_t* status_out) {
  schedule_body(cu, nseq, total, max_seqlen, lbm, lbn, causal, sched, max_items, status_out);
}

hipError_t launch_varlen_schedule(const int32_t* cu_seqlens, int num_seqs, int total_tokens,
                                  int max_seqlen, int bm, int bn, int causal, int32_t* sched,
                                  int max_items, int32_t* status_out, hipStream_t stream) {
  // Query blocks and key tiles are powers of two: the kernel shifts.
  if (bm <= 0 || bn <= 0 || (bm & (bm - 1)) != 0 || (bn & (bn - 1)) != 0) return hipErrorInvalidValue;
  const int lbm = __builtin_ctz(bm), lbn = __builtin_ctz(bn);
  hipLaunchKernelGGL(varlen_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, cu_seqlens,
                     num_seqs, total_tokens, max_seqlen, lbm, lbn, causal, sched, max_items, status_out);
  return hipGetLastError();
}

}  // namespace cgr
