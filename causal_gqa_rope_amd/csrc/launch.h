// Host-side launchers shared by the C-ABI entry points (internal to libcgr).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cgr {

struct AttnArgs;
struct BwdArgs;
struct DecodeArgs;
struct QkvArgs;
struct Fp8Args;

hipError_t launch_attn_d32(const AttnArgs& a, int f32_io, int qk_bf16, int style, int causal,
                           bool varlen, int grid, hipStream_t stream, int phases);
hipError_t launch_attn_d64(const AttnArgs& a, int f32_io, int qk_bf16, int style, int causal,
                           bool varlen, int grid, hipStream_t stream, int phases);
hipError_t launch_attn_d128(const AttnArgs& a, int f32_io, int qk_bf16, int style, int causal,
                            bool varlen, int grid, hipStream_t stream, int phases);
hipError_t launch_attn_d256(const AttnArgs& a, int f32_io, int qk_bf16, int style, int causal,
                            bool varlen, int grid, hipStream_t stream, int phases);
hipError_t launch_attn_fp8(const Fp8Args& a, int style, int causal, hipStream_t stream);

hipError_t launch_attn_bwd_d32(const BwdArgs& a, int qk_bf16, int style, int causal, hipStream_t stream);
hipError_t launch_attn_bwd_d64(const BwdArgs& a, int qk_bf16, int style, int causal, hipStream_t stream);
hipError_t launch_attn_bwd_d128(const BwdArgs& a, int qk_bf16, int style, int causal, hipStream_t stream);

hipError_t launch_decode_d32(const DecodeArgs& a, int style, hipStream_t stream);
hipError_t launch_decode_d64(const DecodeArgs& a, int style, hipStream_t stream);
hipError_t launch_decode_d128(const DecodeArgs& a, int style, hipStream_t stream);
hipError_t launch_rope_rotate_d32(const void* x, void* out, const int32_t* positions, long n_rows, int nh,
                                  int f32_io, const float* cs, const float* sn, int P, int style,
                                  int32_t* status, hipStream_t stream);
hipError_t launch_rope_rotate_d64(const void* x, void* out, const int32_t* positions, long n_rows, int nh,
                                  int f32_io, const float* cs, const float* sn, int P, int style,
                                  int32_t* status, hipStream_t stream);
hipError_t launch_rope_rotate_d128(const void* x, void* out, const int32_t* positions, long n_rows, int nh,
                                   int f32_io, const float* cs, const float* sn, int P, int style,
                                   int32_t* status, hipStream_t stream);

hipError_t launch_qkv_d32(const QkvArgs& a, int style, hipStream_t stream);
hipError_t launch_qkv_d64(const QkvArgs& a, int style, hipStream_t stream);
hipError_t launch_qkv_d128(const QkvArgs& a, int style, hipStream_t stream);

hipError_t launch_rope_tables(int max_pos, int head_dim, double base, float* cos_out,
                              float* sin_out, hipStream_t stream);

// Builds the work list of a packed batch into `sched` and, if kimg_base is
// non-null, the first K image slot of every sequence (see varlen_sched.hip).
hipError_t launch_varlen_schedule(const int32_t* cu_seqlens, int num_seqs, int total_tokens,
                                  int max_seqlen, int bm, int bn, int causal, int32_t* sched,
                                  int max_items, int32_t* kimg_base, hipStream_t stream);

}  // namespace cgr
