// Work schedule of a packed variable-length batch (the kohakutt page,
// Highlights: flash attention over "packed variable-length batches"): the
// prepass that one workgroup runs, shared by the schedule-only kernel
// (varlen_sched.hip) and the kernel that also rotates the keys once
// (varlen_prep_kernel).
//
// It reads cu_seqlens on the device, checks it, and writes the list of
// (sequence, query block) items sorted by cost, most expensive first, where
// cost = number of key tiles the item visits (under the causal mask, query
// block qb of a sequence of length L sees ceil(min((qb+1)*BM, L) / BN)
// tiles). A counting sort over cost bins keeps this to two passes over the
// items, each spread evenly over the workgroup's threads. The attention
// kernel's workgroups take the items in that order (the device hands them out
// by index as compute units free up: longest-processing-time-first), which
// balances the causal triangle of every sequence over the compute units.
//
// Layout of `sched` (int32): [0] number of items, [1] set to 0 (unused),
// [2] error word (0 = well formed), [3] unused, then items as (sequence,
// query block) int pairs. status_out (optional): a second copy of the error
// word, for callers that pass no workspace of their own.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cgr {

constexpr int kSchedHeaderInts = 4;  // ints before the items in `sched`
constexpr int kSchedThreads = 512;
constexpr int kSchedWaves = kSchedThreads / 64;
constexpr int kBins = 2048;  // costs >= kBins - 1 share the last bin

// Key tiles (of 1 << lbn keys) that query block qb (rows qb << lbm ..) of a
// sequence of L tokens visits.
__device__ __forceinline__ int cost_bin(int qb, int L, int lbm, int lbn, int causal) {
  const int keys = causal ? min((qb + 1) << lbm, L) : L;
  return min((keys + (1 << lbn) - 1) >> lbn, kBins - 1);
}

// Inclusive sum of v over the workgroup (wave shuffles, then the wave totals
// through LDS); *total receives the sum over all threads. Every thread calls it.
__device__ __forceinline__ int block_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kSchedWaves; ++i) {
    const int x = wsum[i];
    before += i < w ? x : 0;
    all += x;
  }
  __syncthreads();
  *total = all;
  return v + before;
}

// The prepass itself, run by one workgroup of kSchedThreads threads.
__device__ __forceinline__ void schedule_body(const int32_t* cu, int nseq, int total, int max_seqlen, int lbm,
                                              int lbn, int causal, int32_t* sched, int max_items,
                                              int32_t* status_out) {
  __shared__ int hist[kBins];
  __shared__ int incl[kSchedThreads];  // a round's items per sequence, inclusive sums
  __shared__ int lens[kSchedThreads];
  __shared__ int wsum[kSchedWaves];
  __shared__ int err;
  const int tid = threadIdx.x;
  for (int b = tid; b < kBins; b += kSchedThreads) hist[b] = 0;
  if (tid == 0) err = 0;
  __syncthreads();

  // The items of kSchedThreads sequences at a time, spread evenly over the
  // threads whatever the lengths: one thread per sequence counts its query
  // blocks, a scan numbers the round's items, and thread tid takes items tid,
  // tid + kSchedThreads, ..., finding each one's sequence by a binary search
  // over the inclusive counts. With check set, the round also checks every
  // sequence boundary (a bad sequence contributes no items). act(s, qb, L)
  // runs once per item.
  auto for_items = [&](bool check, auto&& act) {
    for (int s0 = 0; s0 < nseq; s0 += kSchedThreads) {
      const int s = s0 + tid;
      int L = 0;
      if (s < nseq) {
        const int c0 = cu[s], c1 = cu[s + 1];
        int e = 0;
        if (check) {
          if (s == 0 && c0 != 0) e = 1;
          else if (c1 < c0) e = 2;
          else if (c1 - c0 > max_seqlen) e = 3;
          else if (s == nseq - 1 && c1 != total) e = 4;
          if (e) atomicCAS(&err, 0, e);
        }
        L = e ? 0 : c1 - c0;
      }
      const int nq = (L + (1 << lbm) - 1) >> lbm;
      int n_round;
      const int inc = block_scan(nq, wsum, &n_round);
      incl[tid] = inc;
      lens[tid] = L;
      __syncthreads();
      for (int g = tid; g < n_round; g += kSchedThreads) {
        // i = the first entry with incl[i] > g (the number of entries <= g).
        int i = 0;
#pragma unroll
        for (int step = kSchedThreads / 2; step > 0; step >>= 1)
          if (incl[i + step - 1] <= g) i += step;
        const int Li = lens[i];
        const int qb = g - (incl[i] - ((Li + (1 << lbm) - 1) >> lbm));
        act(s0 + i, qb, Li);
      }
      __syncthreads();  // incl and lens are rewritten by the next round
    }
  };

  // 1. Check the boundaries and count items per cost bin.
  for_items(true, [&](int, int qb, int L) { atomicAdd(&hist[cost_bin(qb, L, lbm, lbn, causal)], 1); });
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
  int n_items;
  int run = block_scan(local, wsum, &n_items) - local;
#pragma unroll
  for (int k = 0; k < per; ++k) {
    const int b = kBins - 1 - (tid * per + k);
    const int c = hist[b];
    hist[b] = run;
    run += c;
  }
  __syncthreads();

  // 3. Scatter the items to their slots (order inside a bin is arbitrary).
  int2* items = (int2*)(sched + kSchedHeaderInts);
  for_items(false, [&](int s, int qb, int L) {
    const int pos = atomicAdd(&hist[cost_bin(qb, L, lbm, lbn, causal)], 1);
    if (pos < max_items) items[pos] = make_int2(s, qb);
  });

  if (tid == 0) {
    sched[0] = min(n_items, max_items);
    sched[1] = 0;
    sched[2] = 0;
    if (status_out != nullptr) *status_out = 0;
  }
}

}  // namespace cgr
