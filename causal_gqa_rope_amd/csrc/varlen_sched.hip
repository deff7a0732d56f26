// Work schedule of a packed variable-length batch (the kohakutt page,
// Highlights: flash attention over "packed variable-length batches").
//
// A single workgroup reads cu_seqlens on the device, checks it, and writes
// the list of (sequence, query block) items sorted by cost, most expensive
// first, where cost = number of key tiles the item visits (under the causal
// mask, query block qb of a sequence of length L sees ceil(min((qb+1)*BM, L)
// / BN) tiles). A counting sort over cost bins keeps this one pass. The
// attention kernel's persistent workgroups then pull items in that order
// (longest-processing-time-first), which balances the causal triangle of
// every sequence over the compute units.
//
// Layout of `sched` (int32): [0] number of items, [1] queue counter (reset to
// 0 here), [2] error word (0 = well formed), [3] unused, then items as
// (sequence, query block) int pairs.
//
// status_out (optional): a second copy of the error word, for callers that
// pass no workspace of their own.
//
// When the call rotates the keys once (kimg_base non-null), the prepass also
// writes kimg_base[s] = sum over s' < s of ceil(L_s' / bn), s = 0 .. num_seqs:
// the first K tile image slot of every sequence.
#include <hip/hip_runtime.h>

#include "attn_fwd_kernel.h"
#include "launch.h"

namespace cgr {

constexpr int kSchedThreads = 1024;
constexpr int kBins = 2048;  // costs >= kBins - 1 share the last bin

__device__ __forceinline__ int cost_bin(int qb, int L, int bm, int bn, int causal) {
  const int keys = causal ? min((qb + 1) * bm, L) : L;
  return min((keys + bn - 1) / bn, kBins - 1);
}

__global__ __launch_bounds__(kSchedThreads) void varlen_schedule_kernel(
    const int32_t* cu, int nseq, int total, int max_seqlen, int bm, int bn, int causal,
    int32_t* sched, int max_items, int32_t* kimg_base, int32_t* status_out) {
  __shared__ int hist[kBins];
  __shared__ int part[kSchedThreads];
  __shared__ int err;
  const int tid = threadIdx.x;
  for (int b = tid; b < kBins; b += kSchedThreads) hist[b] = 0;
  if (tid == 0) err = 0;
  __syncthreads();

  // 1. Check every sequence boundary and count items per cost bin.
  for (int s = tid; s < nseq; s += kSchedThreads) {
    const int c0 = cu[s], c1 = cu[s + 1];
    int e = 0;
    if (s == 0 && c0 != 0) e = 1;
    else if (c1 < c0) e = 2;
    else if (c1 - c0 > max_seqlen) e = 3;
    else if (s == nseq - 1 && c1 != total) e = 4;
    if (e) {
      atomicCAS(&err, 0, e);
      continue;
    }
    const int L = c1 - c0;
    const int nq = (L + bm - 1) / bm;
    for (int qb = 0; qb < nq; ++qb) atomicAdd(&hist[cost_bin(qb, L, bm, bn, causal)], 1);
  }
  __syncthreads();
  if (err != 0) {
    if (tid == 0) {
      sched[0] = 0;
      sched[1] = 0;
      sched[2] = err;
      if (status_out != nullptr) *status_out = err;
    }
    return;
  }

  // 2. Exclusive scan over the bins from the most expensive down: each thread
  //    owns kBins / kSchedThreads consecutive bins of that order.
  constexpr int per = kBins / kSchedThreads;
  int local = 0;
#pragma unroll
  for (int k = 0; k < per; ++k) local += hist[kBins - 1 - (tid * per + k)];
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {
    const int add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  int run = part[tid] - local;
#pragma unroll
  for (int k = 0; k < per; ++k) {
    const int b = kBins - 1 - (tid * per + k);
    const int c = hist[b];
    hist[b] = run;
    run += c;
  }
  const int n_items = part[kSchedThreads - 1];
  __syncthreads();

  // 3. Scatter the items to their slots (order inside a bin is arbitrary).
  int2* items = (int2*)(sched + kSchedHeaderInts);
  for (int s = tid; s < nseq; s += kSchedThreads) {
    const int c0 = cu[s];
    const int L = cu[s + 1] - c0;
    const int nq = (L + bm - 1) / bm;
    for (int qb = 0; qb < nq; ++qb) {
      const int pos = atomicAdd(&hist[cost_bin(qb, L, bm, bn, causal)], 1);
      if (pos < max_items) items[pos] = make_int2(s, qb);
    }
  }
  // 4. First image slot of every sequence: each thread sums the tiles of a
  //    run of consecutive sequences, a scan over the threads gives the runs'
  //    starts.
  if (kimg_base != nullptr) {
    const int chunk = (nseq + kSchedThreads - 1) / kSchedThreads;
    const int s0 = min(tid * chunk, nseq), s1 = min(s0 + chunk, nseq);
    int own = 0;
    for (int s = s0; s < s1; ++s) own += (cu[s + 1] - cu[s] + bn - 1) / bn;
    __syncthreads();  // every thread is done with part[] above
    part[tid] = own;
    __syncthreads();
    for (int off = 1; off < kSchedThreads; off <<= 1) {
      const int add = tid >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    int at = part[tid] - own;
    for (int s = s0; s < s1; ++s) {
      kimg_base[s] = at;
      at += (cu[s + 1] - cu[s] + bn - 1) / bn;
    }
    if (tid == kSchedThreads - 1) kimg_base[nseq] = part[tid];
  }
  if (tid == 0) {
    sched[0] = min(n_items, max_items);
    sched[1] = 0;
    sched[2] = 0;
    if (status_out != nullptr) *status_out = 0;
  }
}

hipError_t launch_varlen_schedule(const int32_t* cu_seqlens, int num_seqs, int total_tokens,
                                  int max_seqlen, int bm, int bn, int causal, int32_t* sched,
                                  int max_items, int32_t* kimg_base, int32_t* status_out, hipStream_t stream) {
  hipLaunchKernelGGL(varlen_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, cu_seqlens,
                     num_seqs, total_tokens, max_seqlen, bm, bn, causal, sched, max_items, kimg_base,
                     status_out);
  return hipGetLastError();
}

}  // namespace cgr
