// cgr_gqa_rope_attn_fwd_varlen_noalloc: the packed-batch forward for callers
// that cannot allocate device memory (code under graph capture, tight serving
// loops). Its schedule lives in `scratch`, a file-scope device array of
// kNoAllocScratchBytes that every GPU the library runs on holds until the
// process ends; the caller passes only inputs and outputs.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <mutex>

#include "cgr.h"
#include "launch.h"

namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)1 << 20;  // 1 MiB

// In host code `scratch` names a host-side stand-in, not the device array:
// everything the host hands to a kernel uses the address scratch_on_device()
// looked up for the current device.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch`: looked up with hipGetSymbolAddress
// on the first call on that device (with it current), then cached.
hipError_t scratch_on_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

CGR_API cgr_status cgr_gqa_rope_attn_fwd_varlen_noalloc(
    const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens, int num_seqs,
    int total_tokens, int max_seqlen, int n_head, int n_kv_head, int head_dim, cgr_dtype dtype,
    const float* rope_cos, const float* rope_sin, int rope_max_pos, cgr_rope_style style, cgr_mask mask,
    int window, float softmax_scale, cgr_qk_operand qk_operand, int32_t* device_status, void* stream) {
  char msg[256];
  const cgr_status st = cgr::varlen_check(q, k, v, o, lse, cu_seqlens, num_seqs, total_tokens, max_seqlen, n_head,
                                          n_kv_head, head_dim, dtype, rope_cos, rope_sin, rope_max_pos, style, mask,
                                          window, softmax_scale, qk_operand);
  if (st != CGR_OK) return st;
  const size_t need = cgr_attn_fwd_varlen_workspace_size(num_seqs, total_tokens);
  if (need > kNoAllocScratchBytes) {
    snprintf(msg, sizeof(msg),
             "the schedule of %d sequences / %d tokens needs %zu bytes; the no-alloc scratch holds %zu "
             "(about 4 million tokens): use cgr_gqa_rope_attn_fwd_varlen with a workspace",
             num_seqs, total_tokens, need, kNoAllocScratchBytes);
    return cgr::report_error(CGR_ERR_WORKSPACE, msg);
  }
  if ((reinterpret_cast<uintptr_t>(device_status) & 3) != 0)
    return cgr::report_error(CGR_ERR_ALIGNMENT, "device_status must be 4-byte aligned");
  void* ws = nullptr;
  const hipError_t e = scratch_on_device(&ws);
  if (e != hipSuccess) {
    snprintf(msg, sizeof(msg), "no-alloc scratch address: %s", hipGetErrorString(e));
    return cgr::report_error(CGR_ERR_HIP, msg);
  }
  return cgr::varlen_fwd(q, k, v, o, lse, cu_seqlens, num_seqs, total_tokens, max_seqlen, n_head, n_kv_head,
                         head_dim, dtype, rope_cos, rope_sin, rope_max_pos, style, mask, window, softmax_scale,
                         qk_operand, ws, kNoAllocScratchBytes, device_status, stream);
}

}  // extern "C"
