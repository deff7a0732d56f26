// Host-side launchers shared by the C-ABI entry points (internal to libcgr).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cgr.h"

namespace cgr {

struct AttnArgs;
struct BwdArgs;
struct DecodeArgs;
struct QkvArgs;
struct Fp8Args;

hipError_t launch_attn_d32(const AttnArgs& a, int f32_io, int qk_bf16, int style, int causal,
                           bool varlen, int grid, hipStream_t stream, int phases, bool small);
hipError_t launch_attn_d64(const AttnArgs& a, int f32_io, int qk_bf16, int style, int causal,
                           bool varlen, int grid, hipStream_t stream, int phases, bool small);
hipError_t launch_attn_d128(const AttnArgs& a, int f32_io, int qk_bf16, int style, int causal,
                            bool varlen, int grid, hipStream_t stream, int phases, bool small);
hipError_t launch_attn_d256(const AttnArgs& a, int f32_io, int qk_bf16, int style, int causal,
                            bool varlen, int grid, hipStream_t stream, int phases, bool small);
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

// Builds the work list of a packed batch into `sched` (see varlen_schedule.h).
hipError_t launch_varlen_schedule(const int32_t* cu_seqlens, int num_seqs, int total_tokens,
                                  int max_seqlen, int bm, int bn, int causal, int32_t* sched,
                                  int max_items, int32_t* status_out, hipStream_t stream);

// Records `msg` as cgr_last_error() and returns st.
cgr_status report_error(cgr_status st, const char* msg);

// Every host check of a packed-batch forward call except the workspace's (cgr_api.hip).
cgr_status varlen_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const int32_t* cu_seqlens, int num_seqs, int total_tokens, int max_seqlen, int n_head,
                        int n_kv_head, int head_dim, cgr_dtype dtype, const float* rope_cos,
                        const float* rope_sin, int rope_max_pos, cgr_rope_style style, cgr_mask mask,
                        int window, float softmax_scale, cgr_qk_operand qk_operand);

// The packed-batch forward of cgr_gqa_rope_attn_fwd_varlen on a given
// workspace (cgr_api.hip); status_out, if non-null, receives the schedule's
// error word as well.
cgr_status varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int32_t* cu_seqlens, int num_seqs, int total_tokens, int max_seqlen, int n_head,
                      int n_kv_head, int head_dim, cgr_dtype dtype, const float* rope_cos,
                      const float* rope_sin, int rope_max_pos, cgr_rope_style style, cgr_mask mask, int window,
                      float softmax_scale, cgr_qk_operand qk_operand, void* workspace, size_t workspace_bytes,
                      int32_t* status_out, void* stream);

}  // namespace cgr
