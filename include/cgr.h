/*
 * cgr.h -- fused causal grouped-query attention with rotary position
 * embedding (RoPE) for AMD Instinct MI355X (gfx950): forward (dense and packed
 * batches), backward, decode against a KV cache, and the fused RMSNorm + q/k/v
 * projection + RoPE step that feeds them.
 *
 * The operation, as the pages define it:
 *   - RoPE tables: "Embeddings & the Residual Stream", section "Positional
 *     information: RoPE" -- inv_freq[i] = base^(-2i/d) for i < d/2, angle at
 *     position p = p * inv_freq[i], rotation applied to Q and K only.
 *   - Attention: "Attention from Scratch", section "Attention, the math" --
 *     n_head query heads share n_kv_head K/V heads (query head h reads K/V
 *     head h / (n_head / n_kv_head)), scores q.k / sqrt(d), causal mask
 *     (no token attends to a later one) or none, softmax over keys, weighted
 *     sum of V, output laid out [B, T, n_head, d].
 *   - Computed tile by tile with an online softmax so the T x T score matrix
 *     never reaches memory: same page, section "Coming from CUDA:
 *     FlashAttention".
 *   - Packed variable-length batches with MHA/GQA/MQA: "kohakutt" (PyPI
 *     page), Highlights.
 * Both forward entry points also return, per query row, the natural
 * log-sum-exp of that row's scaled, masked scores (the softmax denominator in
 * log form), so that partial results over disjoint key sets can be merged.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are device memory of the current HIP device;
 *     the caller allocates and owns all of them. The library allocates no
 *     device memory and keeps no per-call state.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). Work is
 *     enqueued on it and the call returns without synchronising.
 *   - Errors: a host-checkable problem returns a non-zero cgr_status and
 *     enqueues nothing; cgr_last_error() then describes it (thread-local).
 *     A failed kernel launch returns CGR_ERR_HIP. No C++ exception crosses
 *     this interface.
 *   - Tensors are contiguous, row-major, and every pointer is 16-byte aligned.
 *   - Linking: the library leaves the HIP runtime's symbols to the process
 *     (link the program with -lamdhip64, or load the runtime first), so that
 *     it always runs on the same runtime instance as its caller.
 */
#ifndef CGR_H
#define CGR_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define CGR_API __attribute__((visibility("default")))
#else
#define CGR_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CGR_OK = 0,
  CGR_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, n_head % n_kv_head != 0, ... */
  CGR_ERR_UNSUPPORTED = 2, /* head_dim not in {32, 64, 128}, unknown dtype/style/mask */
  CGR_ERR_ALIGNMENT = 3,   /* a tensor pointer is not 16-byte aligned */
  CGR_ERR_WORKSPACE = 4,   /* workspace missing or too small */
  CGR_ERR_HIP = 5          /* a HIP call failed; cgr_last_error() holds its message */
} cgr_status;

/* I/O element type of q, k, v and o. */
typedef enum { CGR_F32 = 0, CGR_BF16 = 1 } cgr_dtype;

/* Which features rotate together.
 *   CGR_ROPE_INTERLEAVED: pair i is (2i, 2i+1) -- "rotate each adjacent pair of
 *     features" in the RoPE prose of "Embeddings & the Residual Stream".
 *   CGR_ROPE_HALF: pair i is (i, i + d/2) -- the x*cos + rotate_half(x)*sin
 *     form of the helper printed on the same page. */
typedef enum { CGR_ROPE_INTERLEAVED = 0, CGR_ROPE_HALF = 1 } cgr_rope_style;

/* CGR_MASK_CAUSAL: key j is visible to query i iff j <= i (positions within
 * the sequence). CGR_MASK_NONE: every key of the sequence is visible.
 * The entry points that take a `window` argument add a sliding window to the
 * causal mask: window W > 0 keeps only keys with 0 <= i - j < W (each query
 * sees itself and the W - 1 tokens before it); 0 means no window. A window
 * requires CGR_MASK_CAUSAL. */
typedef enum { CGR_MASK_NONE = 0, CGR_MASK_CAUSAL = 1 } cgr_mask;

/* Operand type of the Q.K^T matrix product (bf16 I/O only; f32 I/O always
 * multiplies in f32). RoPE is applied in f32 and rounded once to this type.
 *   CGR_QK_F16 (default): 3 more mantissa bits than bf16, range +-65504. A
 *     work unit (the rows of one query block) in which a rotated query times
 *     softmax_scale * log2(e), or a rotated key it can see, reaches 65520 or
 *     more (which f16 cannot hold) is found by the forward and recomputed with
 *     the scores taken from bf16 hi + lo parts of the rotated operands (16
 *     significant bits, f32's range): the result is never NaN or infinite
 *     from that cause, at the cost of a slower unit. The backward has no such
 *     path: there the rotated values must stay below 65504.
 *   CGR_QK_BF16: bf16's full range, coarser rounding.
 * The P.V product always multiplies bf16 P by bf16 V, accumulating in f32. */
typedef enum { CGR_QK_F16 = 0, CGR_QK_BF16 = 1 } cgr_qk_operand;

/*
 * RoPE tables ("Embeddings & the Residual Stream", "Positional information:
 * RoPE"). For p < max_pos and i < head_dim/2:
 *   cos_out[p * (head_dim/2) + i] = cos(p * base^(-2i/head_dim))
 *   sin_out[p * (head_dim/2) + i] = sin(p * base^(-2i/head_dim))
 * The angle and its cosine and sine are evaluated in float64 and stored as
 * float32.
 *   max_pos >= 1; head_dim even and >= 2; base > 0 (and finite).
 *   cos_out, sin_out: device float32 [max_pos, head_dim/2], caller-owned.
 */
CGR_API cgr_status cgr_rope_tables(int max_pos, int head_dim, double base, float* cos_out,
                           float* sin_out, void* stream);

/*
 * Bytes of the optional workspace of cgr_gqa_rope_attn_fwd (bf16 I/O): the
 * rotated keys in the Q.K^T operand type as tiles of BN keys (BN = 64, 32 for
 * head_dim 256) in the layout the kernel's LDS holds them, then 256 bytes for
 * the attention kernel's work counter (zero between calls):
 * B * n_kv_head * ceil(T / BN) * BN * head_dim * 2 + 256. Returns 0 for
 * invalid sizes.
 */
CGR_API size_t cgr_attn_fwd_workspace_size(int B, int T, int n_kv_head, int head_dim);

/*
 * Dense batch forward.
 *   q: device [B, T, n_head, head_dim]      (dtype)
 *   k, v: device [B, T, n_kv_head, head_dim] (dtype)
 *   o: device [B, T, n_head, head_dim]      (dtype), written in full
 *     (without seqlens)
 *   lse: device float32 [B, n_head, T], or NULL to skip it
 *   B, T, n_head, n_kv_head >= 1; n_head % n_kv_head == 0;
 *   head_dim in {32, 64, 128}.
 *   rope_cos, rope_sin: device float32 [rope_max_pos, head_dim/2] as written by
 *     cgr_rope_tables; rope_max_pos >= T (token t of every batch entry is at
 *     position t).
 *   window: sliding window (see cgr_mask), 0 for none.
 *   softmax_scale <= 0 selects 1/sqrt(head_dim).
 *   qk_operand: see cgr_qk_operand (ignored for CGR_F32).
 *   seqlens: NULL (every entry holds T tokens), or device int32 [B], 4-byte
 *     aligned: entry b holds L_b valid tokens followed by T - L_b padding
 *     tokens (right padding; a padding mask, one of the masks of the
 *     Kohaku-TT feature list). Keys at or past L_b are hidden from every
 *     query on top of `mask`, and rows at or past L_b of o and lse are left
 *     as they were. The kernel clamps each L_b to [0, T]; no error is
 *     reported for values outside it.
 *   workspace: NULL, or (bf16 I/O) device memory of at least
 *     cgr_attn_fwd_workspace_size(B, T, n_kv_head, head_dim) bytes, 16-byte
 *     aligned, scratch for this call only. With it the keys are rotated
 *     once, before the attention kernel, instead of on every tile that reads
 *     them (the results are the same bits either way). Ignored for CGR_F32,
 *     and left untouched by a call without window whose default grid of
 *     work units would leave compute units idle: such a call runs units half
 *     as tall (twice as many) and rotates the keys per tile, since at that
 *     size a separate rotation pass costs more than it saves (same bits).
 * o and lse must not overlap the inputs.
 */
CGR_API cgr_status cgr_gqa_rope_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int B, int T, int n_head, int n_kv_head, int head_dim,
                                 cgr_dtype dtype, const float* rope_cos, const float* rope_sin,
                                 int rope_max_pos, cgr_rope_style style, cgr_mask mask, int window,
                                 float softmax_scale, cgr_qk_operand qk_operand,
                                 const int32_t* seqlens, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * The two halves of cgr_gqa_rope_attn_fwd with a workspace (bf16 I/O), for a
 * caller that attends several times to the same keys, or that times the
 * attention kernel on its own. Enqueued back to back with the same
 * arguments they give the bits of the one call.
 *
 * cgr_attn_fwd_rotate_keys: rotates every key of k (device [B, T, n_kv_head,
 *   head_dim], bf16) at its position ("Embeddings & the Residual Stream",
 *   "Positional information: RoPE") and writes it, rounded once to the
 *   qk_operand type, into `workspace` (cgr_attn_fwd_workspace_size(B, T,
 *   n_kv_head, head_dim) bytes, 16-byte aligned). seqlens as for the forward
 *   (keys past an entry's length become zeros). Reads nothing else.
 *   dtype must be CGR_BF16 and workspace non-NULL (else CGR_ERR_UNSUPPORTED /
 *   CGR_ERR_WORKSPACE); the other checks are those of the forward.
 *
 * cgr_gqa_rope_attn_fwd_rotated: the attention of cgr_gqa_rope_attn_fwd over
 *   the keys cgr_attn_fwd_rotate_keys left in `workspace`. The call reads the
 *   keys and uses the workspace's last 256 bytes for a work counter, which
 *   cgr_attn_fwd_rotate_keys zeroes and every call leaves at zero: calls
 *   that share a workspace may follow one another but must not overlap
 *   (they would race on the counter). Every argument means what it means for the forward; k,
 *   rope_cos/rope_sin, rope_style, qk_operand and seqlens must be those the
 *   keys were rotated with (the kernel cannot tell, and other values give a
 *   wrong result, not an error). k is still read where a unit recomputes its
 *   scores from the raw keys.
 */
CGR_API cgr_status cgr_attn_fwd_rotate_keys(const void* k, int B, int T, int n_kv_head, int head_dim,
                                    cgr_dtype dtype, const float* rope_cos, const float* rope_sin,
                                    int rope_max_pos, cgr_rope_style style, cgr_qk_operand qk_operand,
                                    const int32_t* seqlens, void* workspace, size_t workspace_bytes,
                                    void* stream);
CGR_API cgr_status cgr_gqa_rope_attn_fwd_rotated(const void* q, const void* k, const void* v, void* o,
                                         float* lse, int B, int T, int n_head, int n_kv_head,
                                         int head_dim, cgr_dtype dtype, const float* rope_cos,
                                         const float* rope_sin, int rope_max_pos, cgr_rope_style style,
                                         cgr_mask mask, int window, float softmax_scale,
                                         cgr_qk_operand qk_operand, const int32_t* seqlens,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of the workspace of cgr_gqa_rope_attn_fwd_fp8: the rotated keys and
 * the transposed values as 64-key tile images, 2 * B * n_kv_head *
 * ceil(T / 64) * 64 * head_dim. Returns 0 for invalid sizes (head_dim must be
 * 128).
 */
CGR_API size_t cgr_attn_fwd_fp8_workspace_size(int B, int T, int n_kv_head, int head_dim);

/*
 * Dense batch forward with fp8 operands ("fp8 operands" of the masks/GQA/
 * packed-batch flash attention listed in the Kohaku-TT feature list; the
 * attention itself as in "Attention from Scratch", "Attention, the math").
 *   q: device [B, T, n_head, 128], k, v: device [B, T, n_kv_head, 128], all
 *     OCP fp8 e4m3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 *     0x7f / 0xff are NaN; largest finite 448). The real inputs are the
 *     codes times q_descale, k_descale, v_descale (finite, > 0).
 *   o: device bf16 [B, T, n_head, 128], written in full (without seqlens).
 *   lse: device float32 [B, n_head, T], or NULL.
 *   head_dim must be 128; mask CGR_MASK_CAUSAL or CGR_MASK_NONE; RoPE tables
 *     as for cgr_gqa_rope_attn_fwd (rope_max_pos >= T).
 *   seqlens: NULL, or device int32 [B] valid tokens per entry (right padding),
 *     exactly as for cgr_gqa_rope_attn_fwd: keys at or past L_b are hidden,
 *     rows at or past L_b of o and lse are left as they were, each L_b is
 *     clamped to [0, T].
 *   workspace: device memory of cgr_attn_fwd_fp8_workspace_size(...) bytes,
 *     16-byte aligned, scratch for this call only (required).
 * Arithmetic: q and k are rotated in f32 and rounded back to e4m3 (q scaled
 * into [1/4, 1/2) of its range, k halved, so no rotated value overflows);
 * both products run on the e4m3 matrix cores with f32 accumulation, the
 * probabilities rounded to e4m3. Expect errors of a few 1e-2 relative to the
 * exact attention of the dequantized inputs (about 10x those of the bf16
 * path). If the softmax scale times the descales is outside 2^-127 .. 2^127
 * the call returns CGR_ERR_INVALID_ARG.
 */
CGR_API cgr_status cgr_gqa_rope_attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                                     int B, int T, int n_head, int n_kv_head, int head_dim,
                                     float q_descale, float k_descale, float v_descale,
                                     const float* rope_cos, const float* rope_sin, int rope_max_pos,
                                     cgr_rope_style style, cgr_mask mask, float softmax_scale,
                                     const int32_t* seqlens, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * Bytes of device workspace cgr_gqa_rope_attn_fwd_varlen needs for a packed
 * batch of num_seqs sequences holding total_tokens tokens. Returns 0 for
 * invalid sizes (num_seqs < 1 or total_tokens < 0).
 */
CGR_API size_t cgr_attn_fwd_varlen_workspace_size(int num_seqs, int total_tokens);

/*
 * Bytes of device workspace with which cgr_gqa_rope_attn_fwd_varlen (bf16
 * I/O) also rotates every key once up front: the schedule above, then, on a
 * 256-byte boundary, the rotated keys as tile images (per K/V head,
 * ceil(total_tokens / BN) + num_seqs tiles of BN keys x head_dim, BN = 64, or
 * 32 at head_dim 256, in the Q.K^T operand type). The rotation is the same
 * arithmetic as the per-tile one, so the results are bit-identical. Returns 0 for invalid
 * sizes (num_seqs < 1, total_tokens < 0, n_kv_head < 1, or a head_dim other
 * than 32, 64, 128, 256).
 */
CGR_API size_t cgr_attn_fwd_varlen_rotated_workspace_size(int num_seqs, int total_tokens, int n_kv_head,
                                                          int head_dim);

/*
 * Packed variable-length batch forward. Sequence s holds tokens
 * cu_seqlens[s] .. cu_seqlens[s+1]-1; RoPE positions restart at 0 in every
 * sequence and the mask never crosses a sequence boundary.
 *   q: device [total_tokens, n_head, head_dim]; k, v: device [total_tokens,
 *     n_kv_head, head_dim]; o: device [total_tokens, n_head, head_dim].
 *   lse: device float32 [n_head, total_tokens], or NULL.
 *   cu_seqlens: device int32 [num_seqs + 1] with cu_seqlens[0] = 0,
 *     non-decreasing, cu_seqlens[num_seqs] = total_tokens, and no sequence
 *     longer than max_seqlen. Zero-length sequences are allowed.
 *   rope_max_pos >= max_seqlen. Other arguments as for the dense call.
 *   workspace: device memory of at least
 *     cgr_attn_fwd_varlen_workspace_size(num_seqs, total_tokens) bytes,
 *     16-byte aligned, used as scratch by this call only (it holds the
 *     work schedule); calls that overlap in time need separate workspaces.
 *     With bf16 I/O and at least cgr_attn_fwd_varlen_rotated_workspace_size(
 *     num_seqs, total_tokens, n_kv_head, head_dim) bytes, the keys are
 *     rotated once into it before the attention kernel (same results).
 * cu_seqlens lives on the device, so its contents are checked there: a
 * malformed array schedules no work (o and lse are left unwritten) and sets
 * an error word that cgr_varlen_device_status() reports.
 */
CGR_API cgr_status cgr_gqa_rope_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                                        float* lse, const int32_t* cu_seqlens, int num_seqs,
                                        int total_tokens, int max_seqlen, int n_head,
                                        int n_kv_head, int head_dim, cgr_dtype dtype,
                                        const float* rope_cos, const float* rope_sin,
                                        int rope_max_pos, cgr_rope_style style, cgr_mask mask,
                                        int window, float softmax_scale, cgr_qk_operand qk_operand,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace cgr_gqa_rope_attn_bwd needs for these sizes
 * (0 for invalid sizes): the rotated q and k in the Q.K^T operand type plus
 * two floats per query row and head; with more than 4 query heads per K/V
 * head, also f32 partial sums of dk and dv, 2 * ceil(G / 4) * B * T *
 * n_kv_head * head_dim floats (G = n_head / n_kv_head); then 256 bytes for
 * the gradient kernels' work counters.
 */
CGR_API size_t cgr_attn_bwd_workspace_size(int B, int T, int n_head, int n_kv_head, int head_dim);

/*
 * Dense batch backward: the gradients of a loss L with respect to q, k and v,
 * given dL/dO, by the chain rule through the forward above ("Train It & Run
 * for Real", section "Coming from CUDA: where's .backward()?": RoPE and
 * attention each carry their backward). With q~ = R q and k~ = R k rotated at
 * their positions, P the forward's softmax weights and D_i = dO_i . O_i:
 *   dv_j = sum_i P_ij dO_i;   dS_ij = P_ij (dO_i . v_j - D_i)
 *   dq_i = R_i^T scale sum_j dS_ij k~_j;   dk_j = R_j^T scale sum_i dS_ij q~_i
 * where dk and dv sum over the n_head / n_kv_head query heads sharing the K/V
 * head.
 *   q, k, v, rope tables, sizes, style, mask, window, softmax_scale,
 *     qk_operand: as given to cgr_gqa_rope_attn_fwd.
 *   o: device [B, T, n_head, head_dim], lse: device float32 [B, n_head, T] --
 *     the forward's outputs for these inputs (P is recomputed from q, k and
 *     lse; D from o).
 *   dout: device [B, T, n_head, head_dim], dL/dO.
 *   dq: device [B, T, n_head, head_dim]; dk, dv: device [B, T, n_kv_head,
 *     head_dim]; all written in full, none may overlap an input.
 *   dtype: CGR_BF16 only (CGR_F32 returns CGR_ERR_UNSUPPORTED). The products
 *     that involve q~ or k~ use the qk_operand type (dS is rounded to it), the
 *     ones that involve dO use bf16 (P is rounded to bf16); all accumulate in
 *     f32, and each gradient is rounded once to bf16.
 *   workspace: device memory of at least cgr_attn_bwd_workspace_size(...)
 *     bytes, 256-byte aligned, scratch for this call only.
 * Every output element is written once, in a fixed order: repeated calls give
 * identical bits.
 */
CGR_API cgr_status cgr_gqa_rope_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                 const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                 int B, int T, int n_head, int n_kv_head, int head_dim,
                                 cgr_dtype dtype, const float* rope_cos, const float* rope_sin,
                                 int rope_max_pos, cgr_rope_style style, cgr_mask mask, int window,
                                 float softmax_scale, cgr_qk_operand qk_operand, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace cgr_gqa_rope_attn_bwd_varlen needs (0 for invalid
 * sizes): the rotated q and k of the total_tokens rows in the Q.K^T operand
 * type plus two floats per head for every row of ceil(total_tokens / 32) +
 * num_seqs slots of 32 rows (each sequence starts a slot of its own); with
 * more than 4 query heads per K/V head, also 2 * ceil(G / 4) * total_tokens *
 * n_kv_head * head_dim floats of partial sums, and 256 bytes of counters,
 * as for the dense call.
 */
CGR_API size_t cgr_attn_bwd_varlen_workspace_size(int num_seqs, int total_tokens, int n_head, int n_kv_head,
                                                  int head_dim);

/*
 * Packed variable-length batch backward: for every sequence of the batch,
 * the gradients that cgr_gqa_rope_attn_bwd gives for it alone (same chain
 * rule through RoPE and attention, "Train It & Run for Real", section
 * "Coming from CUDA: where's .backward()?"; positions restart at 0 in every
 * sequence and no row sees another sequence's keys).
 *   q, k, v, cu_seqlens, num_seqs, total_tokens, max_seqlen, rope tables,
 *     sizes, style, mask, window, softmax_scale, qk_operand: as given to
 *     cgr_gqa_rope_attn_fwd_varlen.
 *   o: device [total_tokens, n_head, head_dim], lse: device float32 [n_head,
 *     total_tokens] -- that forward's outputs.
 *   dout: device [total_tokens, n_head, head_dim], dL/dO.
 *   dq: device [total_tokens, n_head, head_dim]; dk, dv: device
 *     [total_tokens, n_kv_head, head_dim]; every row is written once, none
 *     may overlap an input.
 *   dtype: CGR_BF16 only; the arithmetic is that of cgr_gqa_rope_attn_bwd
 *     (the same bits as that call on each sequence alone).
 *   workspace: device memory of at least cgr_attn_bwd_varlen_workspace_size(
 *     ...) bytes, 256-byte aligned, scratch for this call only.
 * cu_seqlens must be an array that the forward accepted (its checks run on the
 * device there); the kernels read it but do not check it again. With any
 * contents no access leaves the tensors, but rows outside every well-formed
 * sequence are then left unwritten.
 */
CGR_API cgr_status cgr_gqa_rope_attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                                const int32_t* cu_seqlens, int num_seqs, int total_tokens,
                                                int max_seqlen, int n_head, int n_kv_head, int head_dim,
                                                cgr_dtype dtype, const float* rope_cos, const float* rope_sin,
                                                int rope_max_pos, cgr_rope_style style, cgr_mask mask, int window,
                                                float softmax_scale, cgr_qk_operand qk_operand, void* workspace,
                                                size_t workspace_bytes, void* stream);

/*
 * RoPE on rows at given positions ("Embeddings & the Residual Stream",
 * "Positional information: RoPE"): out[t, h, :] = R(positions[t]) x[t, h, :]
 * for x, out device [n_tokens, n_heads, head_dim] (dtype; out may equal x).
 * The step that appends new keys to a KV cache for cgr_gqa_rope_attn_decode,
 * which expects keys already rotated at their positions.
 *   positions: device int32 [n_tokens]; a row whose position is outside
 *     [0, rope_max_pos) is left unwritten and sets *device_status to 1 (when
 *     device_status, a device int32, is non-null; it is never cleared here).
 *   head_dim in {32, 64, 128}; tables as for the forward.
 */
CGR_API cgr_status cgr_rope_rotate(const void* x, void* out, const int32_t* positions, int n_tokens,
                           int n_heads, int head_dim, cgr_dtype dtype, const float* rope_cos,
                           const float* rope_sin, int rope_max_pos, cgr_rope_style style,
                           int32_t* device_status, void* stream);

/*
 * Bytes of device workspace cgr_gqa_rope_attn_decode needs (0 for invalid
 * sizes): a 256-byte header, then one partial output and log-sum-exp per
 * (batch entry, head, query, key chunk); the chunking depends on the sizes
 * only.
 */
CGR_API size_t cgr_attn_decode_workspace_size(int B, int Tq, int max_seqlen, int n_head, int n_kv_head,
                                      int head_dim);

/*
 * Decode: the Tq newest tokens of each of B sequences attend to that
 * sequence's KV cache ("Attention from Scratch", "Attention, the math": GQA
 * lets n_head / n_kv_head query heads share one cached K/V head).
 * Batch entry b has L_b = cache_seqlens[b] cached tokens at positions
 * 0 .. L_b - 1, the Tq new ones being the last Tq; query i is at position
 * L_b - Tq + i and sees keys j <= L_b - Tq + i (causal, aligned with the end
 * of the cache).
 *   q: device bf16 [B, Tq, n_head, head_dim], rotated here at its position.
 *   k_cache, v_cache: device bf16 caches with room for cache_capacity tokens
 *     per entry; token t of K/V head kv of entry b starts at element
 *     b * cache_batch_stride + t * cache_token_stride + kv * cache_head_stride
 *     (head_dim contiguous elements; the same layout for both caches). A
 *     contiguous [B, cache_capacity, n_kv_head, head_dim] cache has strides
 *     (cache_capacity * n_kv_head * head_dim, n_kv_head * head_dim, head_dim);
 *     a head-major [B, n_kv_head, cache_capacity, head_dim] one
 *     (n_kv_head * cache_capacity * head_dim, head_dim, cache_capacity *
 *     head_dim). Strides are multiples of 8 elements. Rows 0 .. L_b - 1 of
 *     entry b are used; the keys are stored already rotated at their
 *     positions (cgr_rope_rotate), the values as they are.
 *   cache_seqlens: device int32 [B], each in [Tq, max_seqlen]; max_seqlen <=
 *     cache_capacity and <= rope_max_pos.
 *   window: W > 0 keeps only keys with 0 <= (L_b - Tq + i) - j < W; 0: none.
 *   o: device bf16 [B, Tq, n_head, head_dim]; lse: device float32
 *     [B, n_head, Tq] (natural log-sum-exp), or NULL.
 *   dtype: CGR_BF16 only. Scores are products of the bf16 keys with the
 *     rotated, scaled query carried as two bf16 parts (16 significant bits);
 *     P.V multiplies bf16 P by bf16 V; f32 accumulation.
 *   workspace: at least cgr_attn_decode_workspace_size(B, Tq, max_seqlen,
 *     n_head, n_kv_head, head_dim) bytes, 256-byte aligned, for this call only.
 * cache_seqlens lives on the device and is checked there: entries outside
 * [Tq, max_seqlen] are left unwritten and the call's error word (read with
 * cgr_varlen_device_status on the workspace) becomes 1; otherwise 0.
 */
CGR_API cgr_status cgr_gqa_rope_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* cache_seqlens, void* o, float* lse, int B, int Tq,
                                    int cache_capacity, int64_t cache_batch_stride,
                                    int64_t cache_token_stride, int64_t cache_head_stride,
                                    int max_seqlen, int n_head, int n_kv_head, int head_dim,
                                    cgr_dtype dtype, const float* rope_cos, const float* rope_sin,
                                    int rope_max_pos, cgr_rope_style style, int window,
                                    float softmax_scale, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * Bytes of device workspace cgr_rmsnorm_qkv_rope needs (0 for invalid sizes):
 * a 256-byte header, one float per token, and the projection weight with the
 * norm's weight folded in (bf16).
 */
CGR_API size_t cgr_rmsnorm_qkv_rope_workspace_size(int n_tokens, int n_embd, int n_head, int n_kv_head,
                                           int head_dim);

/*
 * The block's steps before attention, fused: pre-norm RMSNorm ("The
 * Transformer Block & the Model", "RMSNorm: normalizing before every
 * sub-layer"), the bias-free q, k, v projections and RoPE ("Attention from
 * Scratch", "Attention, the math": project, then rotate). For token t:
 *   xn = x[t] / sqrt(mean(x[t]^2) + eps) * norm_weight
 *   q[t] = xn W_q^T,  k[t] = xn W_k^T,  v[t] = xn W_v^T
 * then q[t] (rotate bit 0) and k[t] (rotate bit 1) are rotated at position
 * positions[t]. rotate = 0 leaves RoPE to the attention call (which rotates
 * q and k itself); 2 gives the rotated keys a KV cache stores; 3 rotates both.
 *   x: device bf16 [n_tokens, n_embd], n_embd a multiple of 32.
 *   norm_weight: device bf16 [n_embd].
 *   w_qkv: device bf16 [(n_head + 2 n_kv_head) * head_dim, n_embd]: the rows of
 *     W_q, then W_k, then W_v (the [out, in] layout of a linear layer).
 *   positions: device int32 [n_tokens]; a token whose position lies outside
 *     [0, rope_max_pos) is left unwritten and sets the call's error word to 1
 *     (read it with cgr_varlen_device_status on the workspace).
 *   q: device bf16 [n_tokens, n_head, head_dim]; k, v: device bf16
 *     [n_tokens, n_kv_head, head_dim]; written in full otherwise.
 *   head_dim in {32, 64, 128}; tables and style as for the forward.
 *   workspace: at least cgr_rmsnorm_qkv_rope_workspace_size(...) bytes,
 *     256-byte aligned, for this call only.
 * Numerics: W diag(norm_weight) is rounded once to bf16, products on bf16
 * matrix cores with f32 sums, the 1/rms factor and RoPE in f32, one rounding
 * of each output to bf16.
 */
CGR_API cgr_status cgr_rmsnorm_qkv_rope(const void* x, const void* norm_weight, float eps, const void* w_qkv,
                                const int32_t* positions, void* q, void* k, void* v, int n_tokens,
                                int n_embd, int n_head, int n_kv_head, int head_dim, cgr_dtype dtype,
                                const float* rope_cos, const float* rope_sin, int rope_max_pos,
                                cgr_rope_style style, int rotate, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * cgr_gqa_rope_attn_fwd_varlen with no workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. The call allocates nothing. The
 * batch's work schedule lives in a 1 MiB device array inside the library,
 * one per GPU, held until the process ends; the caller passes only inputs
 * and outputs. Arguments as for cgr_gqa_rope_attn_fwd_varlen, except:
 *   device_status: NULL, or device int32, 4-byte aligned, that receives the
 *     schedule's error word (0, or the codes cgr_varlen_device_status
 *     reports for a malformed cu_seqlens).
 * Limit: cgr_attn_fwd_varlen_workspace_size(num_seqs, total_tokens) must not
 * exceed 1 MiB (about 4 million tokens), else CGR_ERR_WORKSPACE and nothing
 * is enqueued. The keys are rotated once when the batch's tile images fit in
 * the array as well (small batches), else per tile; the results are the same
 * bits either way, and those of cgr_gqa_rope_attn_fwd_varlen.
 * Every call on a GPU uses that GPU's one array: calls that overlap on one GPU
 * (other streams, or other threads without ordering) race and give undefined
 * results.
 */
CGR_API cgr_status cgr_gqa_rope_attn_fwd_varlen_noalloc(
    const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens, int num_seqs,
    int total_tokens, int max_seqlen, int n_head, int n_kv_head, int head_dim, cgr_dtype dtype,
    const float* rope_cos, const float* rope_sin, int rope_max_pos, cgr_rope_style style, cgr_mask mask,
    int window, float softmax_scale, cgr_qk_operand qk_operand, int32_t* device_status, void* stream);

/*
 * Reads the device error word the last varlen, decode or rmsnorm_qkv_rope call on `workspace` left:
 * waits for `stream`, then stores 0 (the device-side sizes were well formed)
 * or a positive code in *host_status. Varlen: 1: cu_seqlens[0] != 0,
 * 2: decreasing, 3: a sequence longer than max_seqlen, 4:
 * cu_seqlens[num_seqs] != total_tokens. Decode: 1: a cache length outside
 * [Tq, max_seqlen]. rmsnorm_qkv_rope: 1: a position outside [0, rope_max_pos).
 */
CGR_API cgr_status cgr_varlen_device_status(const void* workspace, void* stream, int32_t* host_status);

/* Thread-local description of the last non-OK status returned on this thread. */
CGR_API const char* cgr_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
CGR_API int cgr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CGR_H */
