// C-ABI entry points of libcgr: argument checks, launch configuration and
// error reporting. Every check that can be made on the host is made before
// anything is enqueued.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "attn_bwd_kernel.h"
#include "attn_decode_kernel.h"
#include "attn_fp8_kernel.h"
#include "attn_fwd_kernel.h"
#include "qkv_kernel.h"
#include "cgr.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

cgr_status fail(cgr_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

cgr_status hip_fail(const char* what, hipError_t e) {
  return fail(CGR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Compute units of the current device, cached per device ordinal.
int cu_count(int* out) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return 0;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return (int)e;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return 0;
}

// Checks shared by the dense and the packed forward. `need_pos` is the
// largest RoPE position + 1 the call can reach.
cgr_status check_common(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, int n_head, int n_kv_head, int head_dim,
                        cgr_dtype dtype, const float* cs, const float* sn, int rope_max_pos,
                        int need_pos, cgr_rope_style style, cgr_mask mask, float softmax_scale,
                        cgr_qk_operand qk) {
  if (!q || !k || !v || !o) return fail(CGR_ERR_INVALID_ARG, "q, k, v and o must be non-null");
  if (!cs || !sn) return fail(CGR_ERR_INVALID_ARG, "rope_cos and rope_sin must be non-null");
  if (n_head < 1 || n_kv_head < 1)
    return fail(CGR_ERR_INVALID_ARG, "n_head (%d) and n_kv_head (%d) must be >= 1", n_head,
                n_kv_head);
  if (n_head % n_kv_head != 0)
    return fail(CGR_ERR_INVALID_ARG, "n_head (%d) must be divisible by n_kv_head (%d)", n_head,
                n_kv_head);
  if (head_dim < 2 || head_dim % 2 != 0)
    return fail(CGR_ERR_INVALID_ARG, "head_dim (%d) must be even: RoPE rotates pairs", head_dim);
  if (head_dim != 32 && head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(CGR_ERR_UNSUPPORTED, "head_dim %d is not one of 32, 64, 128, 256", head_dim);
  if (dtype != CGR_F32 && dtype != CGR_BF16)
    return fail(CGR_ERR_UNSUPPORTED, "dtype %d is not CGR_F32 or CGR_BF16", (int)dtype);
  if (head_dim == 256 && dtype != CGR_BF16)
    return fail(CGR_ERR_UNSUPPORTED, "head_dim 256 is supported for CGR_BF16 only");
  if (style != CGR_ROPE_INTERLEAVED && style != CGR_ROPE_HALF)
    return fail(CGR_ERR_UNSUPPORTED, "unknown rope style %d", (int)style);
  if (mask != CGR_MASK_NONE && mask != CGR_MASK_CAUSAL)
    return fail(CGR_ERR_UNSUPPORTED, "unknown mask %d", (int)mask);
  if (qk != CGR_QK_F16 && qk != CGR_QK_BF16)
    return fail(CGR_ERR_UNSUPPORTED, "unknown qk operand %d", (int)qk);
  if (!std::isfinite(softmax_scale))
    return fail(CGR_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(cs, 16) || !aligned(sn, 16))
    return fail(CGR_ERR_ALIGNMENT, "q, k, v, o, rope_cos and rope_sin must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(CGR_ERR_ALIGNMENT, "lse must be 4-byte aligned");
  if (rope_max_pos < need_pos)
    return fail(CGR_ERR_INVALID_ARG, "rope tables cover %d positions, the call needs %d",
                rope_max_pos, need_pos);
  // The kernels address one sequence of one tensor with 32-bit byte offsets.
  if ((long)(need_pos + 256) * n_head * head_dim * 4 > (long)INT_MAX)
    return fail(CGR_ERR_UNSUPPORTED, "a sequence of %d tokens x %d heads x %d exceeds 2 GiB",
                need_pos, n_head, head_dim);
  return CGR_OK;
}

cgr_status check_window(int window, cgr_mask mask) {
  if (window < 0) return fail(CGR_ERR_INVALID_ARG, "window (%d) must be >= 0 (0: none)", window);
  if (window > 0 && mask != CGR_MASK_CAUSAL)
    return fail(CGR_ERR_INVALID_ARG, "a sliding window needs CGR_MASK_CAUSAL");
  return CGR_OK;
}

cgr::AttnArgs make_args(const void* q, const void* k, const void* v, void* o, float* lse,
                        const float* cs, const float* sn, int n_head, int n_kv_head, int head_dim,
                        float softmax_scale) {
  cgr::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.rope_cos = cs;
  a.rope_sin = sn;
  a.H = n_head;
  a.KV = n_kv_head;
  const double scale = softmax_scale > 0.f ? (double)softmax_scale : 1.0 / std::sqrt((double)head_dim);
  a.qscale = (float)(scale * 1.4426950408889634074);  // log2(e): exp2 does the exponentials
  return a;
}

hipError_t launch_by_dim(const cgr::AttnArgs& a, int head_dim, cgr_dtype dtype, cgr_qk_operand qk,
                         cgr_rope_style style, cgr_mask mask, bool varlen, int grid,
                         hipStream_t s, int phases = cgr::PHASE_ALL, bool small = false) {
  const int f32 = dtype == CGR_F32, qkb = qk == CGR_QK_BF16, sty = (int)style,
            cau = mask == CGR_MASK_CAUSAL;
  switch (head_dim) {
    case 32: return cgr::launch_attn_d32(a, f32, qkb, sty, cau, varlen, grid, s, phases, small);
    case 64: return cgr::launch_attn_d64(a, f32, qkb, sty, cau, varlen, grid, s, phases, small);
    case 128: return cgr::launch_attn_d128(a, f32, qkb, sty, cau, varlen, grid, s, phases, small);
    default: return cgr::launch_attn_d256(a, f32, qkb, sty, cau, varlen, grid, s, phases, small);
  }
}

// Upper bound on the (sequence, query block) items of a packed batch:
// sum_s ceil(L_s / BM) <= total / BM + num_seqs. The workspace is sized for
// blocks of 32 rows, which covers every block height the kernels use.
long varlen_max_items(int num_seqs, int total_tokens) {
  static_assert(cgr::kMinBM >= 32, "workspace bound assumes query blocks of >= 32 rows");
  return ((long)total_tokens + 31) / 32 + (long)num_seqs;
}

// Backward workspace: the rotated q (operand type) and k, then the per-tile
// accumulator starting values, then (more than kBwdHeadsPerUnit query heads
// per K/V head) the dk/dv units' f32 partial sums; each part starts on a
// 256-byte boundary.
struct BwdLayout {
  size_t qr, kr, ld, part, ctr, total;
  int hsplit;
};
int bwd_hsplit(int n_head, int n_kv_head) {
  const int G = n_head / n_kv_head;
  return (G + cgr::kBwdHeadsPerUnit - 1) / cgr::kBwdHeadsPerUnit;
}
BwdLayout bwd_layout_rows(size_t rows, size_t ld_tiles, int n_head, int n_kv_head, int head_dim) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  BwdLayout l;
  l.qr = 0;
  l.kr = up(rows * n_head * head_dim * 2);
  l.ld = l.kr + up(rows * n_kv_head * head_dim * 2);
  l.part = l.ld + up(ld_tiles * 64 * 4);
  l.hsplit = bwd_hsplit(n_head, n_kv_head);
  const size_t end = l.hsplit > 1 ? l.part + 2 * (size_t)l.hsplit * rows * n_kv_head * head_dim * 4
                                  : l.ld + ld_tiles * 64 * 4;
  // Then 256 bytes for the gradient kernels' claim counters.
  l.ctr = up(end);
  l.total = l.ctr + 256;
  return l;
}
BwdLayout bwd_layout(int B, int T, int n_head, int n_kv_head, int head_dim) {
  const size_t nt = ((size_t)T + cgr::kBwdTileRows - 1) / cgr::kBwdTileRows;
  return bwd_layout_rows((size_t)B * T, (size_t)B * n_head * nt, n_head, n_kv_head, head_dim);
}

// Packed batches: the same parts over total_tokens rows, the per-tile values
// in 32-row slots (ceil(total / 32) + num_seqs per head: each sequence starts
// a slot of its own).
long bwd_varlen_slots(int num_seqs, int total_tokens) {
  return ((long)total_tokens + cgr::kBwdTileRows - 1) / cgr::kBwdTileRows + num_seqs;
}
BwdLayout bwd_varlen_layout(int num_seqs, int total_tokens, int n_head, int n_kv_head, int head_dim) {
  return bwd_layout_rows((size_t)total_tokens, (size_t)n_head * bwd_varlen_slots(num_seqs, total_tokens), n_head,
                         n_kv_head, head_dim);
}

// The checks that the dense and the packed backward share beyond the
// forward's own.
cgr_status bwd_check(const float* lse, const void* dout, void* dq, void* dk, void* dv, int head_dim,
                     cgr_dtype dtype, int window, cgr_mask mask, const void* workspace, size_t workspace_bytes,
                     const BwdLayout& lay) {
  if (head_dim == 256) return fail(CGR_ERR_UNSUPPORTED, "the backward is built for head_dim 32, 64, 128");
  cgr_status st = check_window(window, mask);
  if (st != CGR_OK) return st;
  if (!lse || !dout || !dq || !dk || !dv)
    return fail(CGR_ERR_INVALID_ARG, "lse, dout, dq, dk and dv must be non-null");
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return fail(CGR_ERR_ALIGNMENT, "dout, dq, dk and dv must be 16-byte aligned");
  if (dtype != CGR_BF16)
    return fail(CGR_ERR_UNSUPPORTED, "the backward takes bf16 tensors only (dtype %d)", (int)dtype);
  if (!workspace) return fail(CGR_ERR_WORKSPACE, "workspace must be non-null");
  if (!aligned(workspace, 256)) return fail(CGR_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  if (workspace_bytes < lay.total)
    return fail(CGR_ERR_WORKSPACE, "workspace has %zu bytes, the call needs %zu", workspace_bytes, lay.total);
  // The kernels address the per-tile values with one 32-bit buffer range.
  if (lay.part - lay.ld > (size_t)UINT32_MAX)
    return fail(CGR_ERR_UNSUPPORTED, "n_head x the query rows is too large for one call");
  return CGR_OK;
}

// Fill in the tensors, workspace parts and scales, then launch the three
// kernels of the instance (sizes and the packed fields set by the caller).
cgr_status bwd_launch(cgr::BwdArgs& a, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv, int head_dim,
                      const float* rope_cos, const float* rope_sin, cgr_rope_style style, cgr_mask mask,
                      int window, float softmax_scale, cgr_qk_operand qk_operand, void* workspace,
                      const BwdLayout& lay, long rows, void* stream) {
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.qr = (char*)workspace + lay.qr;
  a.kr = (char*)workspace + lay.kr;
  a.ld = (float*)((char*)workspace + lay.ld);
  a.hsplit = lay.hsplit;
  {
    // dq units of 2^lhp heads: the largest power of two <= 8 dividing G.
    const int G = a.H / a.KV;
    a.lhp = 0;
    while (a.lhp < 3 && (G >> a.lhp) % 2 == 0) ++a.lhp;
  }
  a.part_rows = rows;
  a.part = (float*)((char*)workspace + lay.part);
  a.ctr = (int32_t*)((char*)workspace + lay.ctr);
  a.window = window;
  const double scale = softmax_scale > 0.f ? (double)softmax_scale : 1.0 / std::sqrt((double)head_dim);
  a.scale = (float)scale;
  a.qscale = (float)(scale * 1.4426950408889634074);
  const int qkb = qk_operand == CGR_QK_BF16, sty = (int)style, cau = mask == CGR_MASK_CAUSAL;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  switch (head_dim) {
    case 32: e = cgr::launch_attn_bwd_d32(a, qkb, sty, cau, s); break;
    case 64: e = cgr::launch_attn_bwd_d64(a, qkb, sty, cau, s); break;
    default: e = cgr::launch_attn_bwd_d128(a, qkb, sty, cau, s); break;
  }
  if (e != hipSuccess) return hip_fail("backward launch", e);
  return CGR_OK;
}

// Decode split policy, a function of the sizes alone (so the workspace size
// needs no device): about 2048 single-wave workgroups (eight per CU are
// resident at once, so every chunk starts in the first wave of them), chunks
// a multiple of the 32-key tile, no more chunks than tiles.
struct DecodePlan {
  int rg, ns, ch;
  size_t lse_off, o_off, total;
};
DecodePlan decode_plan(int B, int Tq, int max_seqlen, int n_head, int n_kv_head, int head_dim) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  DecodePlan p;
  const int G = n_head / n_kv_head;
  p.rg = (G * Tq + 31) / 32;
  const long pairs = (long)B * n_kv_head * p.rg;
  const int tiles = (max_seqlen + cgr::kDecodeBN - 1) / cgr::kDecodeBN;
  long ns = (2048 + pairs - 1) / pairs;
  if (ns > tiles) ns = tiles;
  if (ns < 1) ns = 1;
  const int per = (int)((max_seqlen + ns - 1) / ns);
  p.ch = ((per + cgr::kDecodeBN - 1) / cgr::kDecodeBN) * cgr::kDecodeBN;
  p.ns = (max_seqlen + p.ch - 1) / p.ch;
  const size_t rows = (size_t)B * n_head * Tq * p.ns;
  p.lse_off = 256;  // int32 header: [2] is the error word
  p.o_off = p.lse_off + up(rows * 4);
  p.total = p.o_off + rows * head_dim * 4;
  return p;
}

// The dense-batch forward behind cgr_gqa_rope_attn_fwd and its two halves
// (cgr_attn_fwd_rotate_keys, cgr_gqa_rope_attn_fwd_rotated): checks, launch
// configuration, then the phases asked for.
cgr_status dense_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int T,
                     int n_head, int n_kv_head, int head_dim, cgr_dtype dtype, const float* rope_cos,
                     const float* rope_sin, int rope_max_pos, cgr_rope_style style, cgr_mask mask,
                     int window, float softmax_scale, cgr_qk_operand qk_operand, const int32_t* seqlens,
                     void* workspace, size_t workspace_bytes, void* stream, int phases) {
  if (seqlens != nullptr && !aligned(seqlens, 4))
    return fail(CGR_ERR_ALIGNMENT, "seqlens must be 4-byte aligned");
  if (B < 1 || T < 1) return fail(CGR_ERR_INVALID_ARG, "B (%d) and T (%d) must be >= 1", B, T);
  cgr_status st = check_common(q, k, v, o, lse, n_head, n_kv_head, head_dim, dtype, rope_cos,
                               rope_sin, rope_max_pos, T, style, mask, softmax_scale, qk_operand);
  if (st != CGR_OK) return st;
  if ((st = check_window(window, mask)) != CGR_OK) return st;
  const bool use_ws = workspace != nullptr && dtype == CGR_BF16;
  if (use_ws) {
    if (!aligned(workspace, 16)) return fail(CGR_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
    const size_t need = cgr_attn_fwd_workspace_size(B, T, n_kv_head, head_dim);
    if (workspace_bytes < need)
      return fail(CGR_ERR_WORKSPACE, "workspace has %zu bytes, the call needs %zu", workspace_bytes, need);
  }
  if ((long)B * T > INT_MAX) return fail(CGR_ERR_INVALID_ARG, "B*T must fit in int32");
  const int G = n_head / n_kv_head;
  int hp = dtype == CGR_F32 ? 1 : cgr::fwd_heads_per_unit(head_dim, G);
  long grid = (long)((T + cgr::fwd_block_rows(head_dim, hp) - 1) / cgr::fwd_block_rows(head_dim, hp)) * B *
              (n_head / hp);
  // A whole (not split) bf16 call whose grid would leave compute units idle
  // runs on the small-unit instances (twice the units, each half as long) and
  // rotates its keys on every tile: at that size a separate rotation pass
  // costs more than it saves. Any workspace given is then left untouched. The
  // results are the same bits either way (every row's arithmetic is the same).
  bool small = false;
  if (dtype == CGR_BF16 && window == 0 && phases == cgr::PHASE_ALL && head_dim != 256) {
    int cus = 0;
    const int ce = cu_count(&cus);
    if (ce != 0) return hip_fail("device query", (hipError_t)ce);
    if (grid < cus) {
      small = true;
      hp = cgr::fwd_heads_per_unit(head_dim, G, cgr::kSmallNW);
      const int bm = cgr::fwd_block_rows(head_dim, hp, cgr::kSmallNW);
      grid = (long)((T + bm - 1) / bm) * B * (n_head / hp);
    }
  }
  if (grid > INT_MAX) return fail(CGR_ERR_INVALID_ARG, "too many work units");
  cgr::AttnArgs a = make_args(q, k, v, o, lse, rope_cos, rope_sin, n_head, n_kv_head, head_dim,
                              softmax_scale);
  a.B = B;
  a.T = T;
  a.total_tokens = B * T;
  a.window = window;
  a.hp = hp;
  a.seqlens = seqlens;
  a.krot = use_ws && !small ? workspace : nullptr;
  const hipError_t e = launch_by_dim(a, head_dim, dtype, qk_operand, style, mask, false, (int)grid,
                                     (hipStream_t)stream, phases, small);
  if (e != hipSuccess) return hip_fail("attention launch", e);
  return CGR_OK;
}

// Workspace of a packed call that rotates the keys once: the schedule, then
// (on a 256-byte boundary) the K tile images ([K/V head][slot], slots =
// ceil(total / BN) + num_seqs, which bounds the slots the sequences' tiles
// take; see varlen_prep_kernel).
struct VarlenLayout {
  size_t images, total;
  long slots;
};
VarlenLayout varlen_layout(int num_seqs, int total_tokens, int n_kv_head, int head_dim) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  VarlenLayout l{};
  const int bn = cgr::fwd_tile_keys(head_dim);
  l.slots = ((long)total_tokens + bn - 1) / bn + num_seqs;
  l.images = up(cgr_attn_fwd_varlen_workspace_size(num_seqs, total_tokens));
  l.total = l.images + (size_t)n_kv_head * l.slots * cgr::fwd_kimg_bytes(head_dim);
  return l;
}

}  // namespace

namespace cgr {
cgr_status report_error(cgr_status st, const char* msg) { return fail(st, "%s", msg); }

// Every host check of a packed-batch forward call except those of the workspace.
cgr_status varlen_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const int32_t* cu_seqlens, int num_seqs, int total_tokens, int max_seqlen, int n_head,
                        int n_kv_head, int head_dim, cgr_dtype dtype, const float* rope_cos,
                        const float* rope_sin, int rope_max_pos, cgr_rope_style style, cgr_mask mask,
                        int window, float softmax_scale, cgr_qk_operand qk_operand) {
  if (!cu_seqlens) return fail(CGR_ERR_INVALID_ARG, "cu_seqlens must be non-null");
  if (!aligned(cu_seqlens, 4)) return fail(CGR_ERR_ALIGNMENT, "cu_seqlens must be 4-byte aligned");
  if (num_seqs < 1) return fail(CGR_ERR_INVALID_ARG, "num_seqs (%d) must be >= 1", num_seqs);
  if (total_tokens < 0 || max_seqlen < 0)
    return fail(CGR_ERR_INVALID_ARG, "total_tokens and max_seqlen must be >= 0");
  if (max_seqlen > total_tokens)
    return fail(CGR_ERR_INVALID_ARG, "max_seqlen (%d) exceeds total_tokens (%d)", max_seqlen,
                total_tokens);
  cgr_status st = check_common(q, k, v, o, lse, n_head, n_kv_head, head_dim, dtype, rope_cos,
                               rope_sin, rope_max_pos, max_seqlen, style, mask, softmax_scale,
                               qk_operand);
  if (st != CGR_OK) return st;
  return check_window(window, mask);
}

// The packed-batch forward behind cgr_gqa_rope_attn_fwd_varlen and
// cgr_gqa_rope_attn_fwd_varlen_noalloc: checks, the schedule prepass, the
// attention kernel. status_out (optional) receives the prepass's error word.
cgr_status varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      const int32_t* cu_seqlens, int num_seqs, int total_tokens, int max_seqlen, int n_head,
                      int n_kv_head, int head_dim, cgr_dtype dtype, const float* rope_cos,
                      const float* rope_sin, int rope_max_pos, cgr_rope_style style, cgr_mask mask, int window,
                      float softmax_scale, cgr_qk_operand qk_operand, void* workspace, size_t workspace_bytes,
                      int32_t* status_out, void* stream) {
  cgr_status st = varlen_check(q, k, v, o, lse, cu_seqlens, num_seqs, total_tokens, max_seqlen, n_head,
                               n_kv_head, head_dim, dtype, rope_cos, rope_sin, rope_max_pos, style, mask, window,
                               softmax_scale, qk_operand);
  if (st != CGR_OK) return st;
  const size_t need = cgr_attn_fwd_varlen_workspace_size(num_seqs, total_tokens);
  if (!workspace) return fail(CGR_ERR_WORKSPACE, "workspace must be non-null");
  if (!aligned(workspace, 16)) return fail(CGR_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(CGR_ERR_WORKSPACE, "workspace has %zu bytes, the call needs %zu", workspace_bytes,
                need);
  const long max_items = varlen_max_items(num_seqs, total_tokens);
  if ((max_items + 7) * n_head > INT_MAX) return fail(CGR_ERR_INVALID_ARG, "too many work units");

  // Keys rotated once (16-bit I/O) when the workspace also holds their images.
  const VarlenLayout lay = varlen_layout(num_seqs, total_tokens, n_kv_head, head_dim);
  const bool use_kimg = dtype == CGR_BF16 && workspace_bytes >= lay.total;
  if (use_kimg && (long)n_kv_head * lay.slots > INT_MAX)
    return fail(CGR_ERR_INVALID_ARG, "too many key tiles");

  hipStream_t s = (hipStream_t)stream;
  int32_t* sched = (int32_t*)workspace;
  const int hp = dtype == CGR_F32 ? 1 : cgr::fwd_heads_per_unit(head_dim, n_head / n_kv_head);
  cgr::AttnArgs a = make_args(q, k, v, o, lse, rope_cos, rope_sin, n_head, n_kv_head, head_dim,
                              softmax_scale);
  a.cu_seqlens = cu_seqlens;
  a.sched = sched;
  a.B = num_seqs;
  a.T = max_seqlen;
  a.total_tokens = total_tokens;
  a.window = window;
  a.hp = hp;
  a.max_items = (int)max_items;
  a.status_out = status_out;
  if (use_kimg) {
    // The schedule runs inside the key rotation's launch.
    a.krot = (char*)workspace + lay.images;
    a.kimg_slots = (int)lay.slots;
  } else {
    hipError_t e = cgr::launch_varlen_schedule(cu_seqlens, num_seqs, total_tokens, max_seqlen,
                                               cgr::fwd_block_rows(head_dim, hp), cgr::fwd_tile_keys(head_dim),
                                               mask == CGR_MASK_CAUSAL, sched, (int)max_items, status_out, s);
    if (e != hipSuccess) return hip_fail("schedule launch", e);
  }
  // One workgroup per unit of the bound on the items (rounded up to 8) times
  // the head groups; those past the schedule's count exit at once.
  long grid = (max_items + 7) / 8 * 8 * (n_head / hp);
  const hipError_t e = launch_by_dim(a, head_dim, dtype, qk_operand, style, mask, true, (int)grid, s);
  if (e != hipSuccess) return hip_fail("attention launch", e);
  return CGR_OK;
}
}  // namespace cgr

extern "C" {

cgr_status cgr_rope_tables(int max_pos, int head_dim, double base, float* cos_out, float* sin_out,
                           void* stream) {
  if (!cos_out || !sin_out) return fail(CGR_ERR_INVALID_ARG, "cos_out and sin_out must be non-null");
  if (max_pos < 1) return fail(CGR_ERR_INVALID_ARG, "max_pos (%d) must be >= 1", max_pos);
  if (head_dim < 2 || head_dim % 2 != 0)
    return fail(CGR_ERR_INVALID_ARG, "head_dim (%d) must be even and >= 2", head_dim);
  if (!(base > 0.0) || !std::isfinite(base))
    return fail(CGR_ERR_INVALID_ARG, "base must be positive and finite");
  if (!aligned(cos_out, 4) || !aligned(sin_out, 4))
    return fail(CGR_ERR_ALIGNMENT, "tables must be 4-byte aligned");
  if ((long)max_pos * (head_dim / 2) > (long)INT_MAX * 256)
    return fail(CGR_ERR_INVALID_ARG, "table too large");
  const hipError_t e = cgr::launch_rope_tables(max_pos, head_dim, base, cos_out, sin_out,
                                               (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("rope_tables launch", e);
  return CGR_OK;
}

cgr_status cgr_gqa_rope_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                 int B, int T, int n_head, int n_kv_head, int head_dim,
                                 cgr_dtype dtype, const float* rope_cos, const float* rope_sin,
                                 int rope_max_pos, cgr_rope_style style, cgr_mask mask, int window,
                                 float softmax_scale, cgr_qk_operand qk_operand,
                                 const int32_t* seqlens, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return dense_fwd(q, k, v, o, lse, B, T, n_head, n_kv_head, head_dim, dtype, rope_cos, rope_sin, rope_max_pos,
                   style, mask, window, softmax_scale, qk_operand, seqlens, workspace, workspace_bytes, stream,
                   cgr::PHASE_ALL);
}

cgr_status cgr_attn_fwd_rotate_keys(const void* k, int B, int T, int n_kv_head, int head_dim, cgr_dtype dtype,
                                    const float* rope_cos, const float* rope_sin, int rope_max_pos,
                                    cgr_rope_style style, cgr_qk_operand qk_operand, const int32_t* seqlens,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != CGR_BF16) return fail(CGR_ERR_UNSUPPORTED, "keys are rotated once for CGR_BF16 I/O only");
  if (workspace == nullptr) return fail(CGR_ERR_WORKSPACE, "the rotated keys need a workspace");
  // Only k, the tables and the workspace are read or written; the query-side
  // checks see k in place of q, v and o, and one query head per K/V head.
  return dense_fwd(k, k, k, const_cast<void*>(k), nullptr, B, T, n_kv_head, n_kv_head, head_dim, dtype, rope_cos,
                   rope_sin, rope_max_pos, style, CGR_MASK_CAUSAL, 0, 0.f, qk_operand, seqlens, workspace,
                   workspace_bytes, stream, cgr::PHASE_ROTATE);
}

cgr_status cgr_gqa_rope_attn_fwd_rotated(const void* q, const void* k, const void* v, void* o, float* lse,
                                         int B, int T, int n_head, int n_kv_head, int head_dim,
                                         cgr_dtype dtype, const float* rope_cos, const float* rope_sin,
                                         int rope_max_pos, cgr_rope_style style, cgr_mask mask, int window,
                                         float softmax_scale, cgr_qk_operand qk_operand,
                                         const int32_t* seqlens, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  if (dtype != CGR_BF16) return fail(CGR_ERR_UNSUPPORTED, "keys are rotated once for CGR_BF16 I/O only");
  if (workspace == nullptr) return fail(CGR_ERR_WORKSPACE, "the rotated keys need a workspace");
  return dense_fwd(q, k, v, o, lse, B, T, n_head, n_kv_head, head_dim, dtype, rope_cos, rope_sin, rope_max_pos,
                   style, mask, window, softmax_scale, qk_operand, seqlens, workspace,
                   workspace_bytes, stream, cgr::PHASE_ATTEND);
}

size_t cgr_attn_fwd_workspace_size(int B, int T, int n_kv_head, int head_dim) {
  if (B < 1 || T < 1 || n_kv_head < 1) return 0;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128 && head_dim != 256) return 0;
  const int bn = cgr::fwd_tile_keys(head_dim);
  // The tile images, then 256 bytes that hold the attention kernel's work counter.
  return (size_t)B * n_kv_head * ((T + bn - 1) / bn) * cgr::fwd_kimg_bytes(head_dim) + 256;
}

size_t cgr_attn_fwd_fp8_workspace_size(int B, int T, int n_kv_head, int head_dim) {
  if (B < 1 || T < 1 || n_kv_head < 1 || head_dim != cgr::kFp8D) return 0;
  const size_t nt = ((size_t)T + cgr::kFp8BN - 1) / cgr::kFp8BN;
  return 2 * (size_t)B * n_kv_head * nt * cgr::kFp8Tile;
}

cgr_status cgr_gqa_rope_attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                                     int B, int T, int n_head, int n_kv_head, int head_dim,
                                     float q_descale, float k_descale, float v_descale,
                                     const float* rope_cos, const float* rope_sin, int rope_max_pos,
                                     cgr_rope_style style, cgr_mask mask, float softmax_scale,
                                     const int32_t* seqlens, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  if (!q || !k || !v || !o) return fail(CGR_ERR_INVALID_ARG, "q, k, v and o must be non-null");
  if (!rope_cos || !rope_sin) return fail(CGR_ERR_INVALID_ARG, "rope_cos and rope_sin must be non-null");
  if (B < 1 || T < 1) return fail(CGR_ERR_INVALID_ARG, "B (%d) and T (%d) must be >= 1", B, T);
  if (n_head < 1 || n_kv_head < 1)
    return fail(CGR_ERR_INVALID_ARG, "n_head (%d) and n_kv_head (%d) must be >= 1", n_head, n_kv_head);
  if (n_head % n_kv_head != 0)
    return fail(CGR_ERR_INVALID_ARG, "n_head (%d) must be divisible by n_kv_head (%d)", n_head, n_kv_head);
  if (head_dim != cgr::kFp8D)
    return fail(CGR_ERR_UNSUPPORTED, "the fp8 forward is built for head_dim 128 (got %d)", head_dim);
  if (style != CGR_ROPE_INTERLEAVED && style != CGR_ROPE_HALF)
    return fail(CGR_ERR_UNSUPPORTED, "unknown rope style %d", (int)style);
  if (mask != CGR_MASK_NONE && mask != CGR_MASK_CAUSAL) return fail(CGR_ERR_UNSUPPORTED, "unknown mask %d", (int)mask);
  if (!std::isfinite(softmax_scale)) return fail(CGR_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (!(q_descale > 0.f) || !(k_descale > 0.f) || !(v_descale > 0.f) || !std::isfinite(q_descale) ||
      !std::isfinite(k_descale) || !std::isfinite(v_descale))
    return fail(CGR_ERR_INVALID_ARG, "the descales must be finite and > 0");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(rope_cos, 16) ||
      !aligned(rope_sin, 16))
    return fail(CGR_ERR_ALIGNMENT, "q, k, v, o, rope_cos and rope_sin must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(CGR_ERR_ALIGNMENT, "lse must be 4-byte aligned");
  if (seqlens && !aligned(seqlens, 4)) return fail(CGR_ERR_ALIGNMENT, "seqlens must be 4-byte aligned");
  if (rope_max_pos < T)
    return fail(CGR_ERR_INVALID_ARG, "rope tables cover %d positions, the call needs %d", rope_max_pos, T);
  if ((long)(T + 256) * n_head * head_dim * 2 > (long)INT_MAX)
    return fail(CGR_ERR_UNSUPPORTED, "a sequence of %d tokens x %d heads x %d exceeds 2 GiB", T, n_head, head_dim);
  if ((long)B * T > INT_MAX) return fail(CGR_ERR_INVALID_ARG, "B*T must fit in int32");
  const size_t need = cgr_attn_fwd_fp8_workspace_size(B, T, n_kv_head, head_dim);
  if (!workspace) return fail(CGR_ERR_WORKSPACE, "workspace must be non-null");
  if (!aligned(workspace, 16)) return fail(CGR_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(CGR_ERR_WORKSPACE, "workspace has %zu bytes, the call needs %zu", workspace_bytes, need);
  // score in log2 units = (sum of Q~ K~) * c / gamma with Q~ = rot(q8) gamma,
  // K~ = rot(k8) / 2: c = q_descale * 2 k_descale * scale * log2(e) = f 2^e,
  // f in [1/2, 1); gamma = f / 2 and the block scale 2^(e + 1).
  const double scale = softmax_scale > 0.f ? (double)softmax_scale : 1.0 / std::sqrt((double)head_dim);
  const double c = (double)q_descale * 2.0 * (double)k_descale * scale * 1.4426950408889634074;
  int e = 0;
  const double f = std::frexp(c, &e);
  const int E = e + 1;
  if (E < -127 || E > 127) return fail(CGR_ERR_INVALID_ARG, "q_descale * k_descale * softmax_scale is out of range");
  const long nt = ((long)T + cgr::kFp8BN - 1) / cgr::kFp8BN;
  const long grid = ((long)T + cgr::kFp8BM - 1) / cgr::kFp8BM * B * n_head;
  if (grid > INT_MAX || (long)B * n_kv_head * nt > INT_MAX) return fail(CGR_ERR_INVALID_ARG, "too many work units");
  cgr::Fp8Args a{};
  a.q = (const uint8_t*)q;
  a.k = (const uint8_t*)k;
  a.v = (const uint8_t*)v;
  a.kimg = (uint8_t*)workspace;
  a.vimg = (uint8_t*)workspace + need / 2;
  a.o = o;
  a.lse = lse;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.seqlens = seqlens;
  a.B = B;
  a.T = T;
  a.H = n_head;
  a.KV = n_kv_head;
  a.NT = (int)nt;
  a.qgamma = (float)(f * 0.5);
  const uint32_t byte = (uint32_t)(127 + E);
  a.kscale = (int)(byte * 0x01010101u);
  a.vdescale = v_descale;
  const hipError_t err = cgr::launch_attn_fp8(a, (int)style, mask == CGR_MASK_CAUSAL, (hipStream_t)stream);
  if (err != hipSuccess) return hip_fail("fp8 attention launch", err);
  return CGR_OK;
}

size_t cgr_attn_fwd_varlen_workspace_size(int num_seqs, int total_tokens) {
  if (num_seqs < 1 || total_tokens < 0) return 0;
  return (size_t)cgr::kSchedHeaderInts * 4 + (size_t)varlen_max_items(num_seqs, total_tokens) * 8;
}

size_t cgr_attn_fwd_varlen_rotated_workspace_size(int num_seqs, int total_tokens, int n_kv_head,
                                                  int head_dim) {
  if (num_seqs < 1 || total_tokens < 0 || n_kv_head < 1) return 0;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128 && head_dim != 256) return 0;
  return varlen_layout(num_seqs, total_tokens, n_kv_head, head_dim).total;
}

cgr_status cgr_gqa_rope_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                                        float* lse, const int32_t* cu_seqlens, int num_seqs,
                                        int total_tokens, int max_seqlen, int n_head,
                                        int n_kv_head, int head_dim, cgr_dtype dtype,
                                        const float* rope_cos, const float* rope_sin,
                                        int rope_max_pos, cgr_rope_style style, cgr_mask mask,
                                        int window, float softmax_scale, cgr_qk_operand qk_operand,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return cgr::varlen_fwd(q, k, v, o, lse, cu_seqlens, num_seqs, total_tokens, max_seqlen, n_head, n_kv_head,
                         head_dim, dtype, rope_cos, rope_sin, rope_max_pos, style, mask, window, softmax_scale,
                         qk_operand, workspace, workspace_bytes, nullptr, stream);
}

size_t cgr_attn_bwd_workspace_size(int B, int T, int n_head, int n_kv_head, int head_dim) {
  if (B < 1 || T < 1 || n_head < 1 || n_kv_head < 1 || head_dim < 2) return 0;
  return bwd_layout(B, T, n_head, n_kv_head, head_dim).total;
}

cgr_status cgr_gqa_rope_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                 const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                 int B, int T, int n_head, int n_kv_head, int head_dim,
                                 cgr_dtype dtype, const float* rope_cos, const float* rope_sin,
                                 int rope_max_pos, cgr_rope_style style, cgr_mask mask, int window,
                                 float softmax_scale, cgr_qk_operand qk_operand, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (B < 1 || T < 1) return fail(CGR_ERR_INVALID_ARG, "B (%d) and T (%d) must be >= 1", B, T);
  cgr_status st = check_common(q, k, v, o, lse, n_head, n_kv_head, head_dim, dtype, rope_cos,
                               rope_sin, rope_max_pos, T, style, mask, softmax_scale, qk_operand);
  if (st != CGR_OK) return st;
  if ((long)B * T > INT_MAX) return fail(CGR_ERR_INVALID_ARG, "B*T must fit in int32");
  const BwdLayout lay = bwd_layout(B, T, n_head, n_kv_head, head_dim);
  if ((st = bwd_check(lse, dout, dq, dk, dv, head_dim, dtype, window, mask, workspace, workspace_bytes, lay)) !=
      CGR_OK)
    return st;
  const long grid_q = (long)((T + 255) / 256) * B * n_head;
  if (grid_q > INT_MAX) return fail(CGR_ERR_INVALID_ARG, "too many work units");
  cgr::BwdArgs a{};
  a.B = B;
  a.T = T;
  a.H = n_head;
  a.KV = n_kv_head;
  a.NT = (T + cgr::kBwdTileRows - 1) / cgr::kBwdTileRows;
  return bwd_launch(a, q, k, v, o, lse, dout, dq, dk, dv, head_dim, rope_cos, rope_sin, style, mask, window,
                    softmax_scale, qk_operand, workspace, lay, (long)B * T, stream);
}

size_t cgr_attn_bwd_varlen_workspace_size(int num_seqs, int total_tokens, int n_head, int n_kv_head,
                                          int head_dim) {
  if (num_seqs < 1 || total_tokens < 0 || n_head < 1 || n_kv_head < 1 || head_dim < 2) return 0;
  return bwd_varlen_layout(num_seqs, total_tokens, n_head, n_kv_head, head_dim).total;
}

cgr_status cgr_gqa_rope_attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                        const int32_t* cu_seqlens, int num_seqs, int total_tokens,
                                        int max_seqlen, int n_head, int n_kv_head, int head_dim,
                                        cgr_dtype dtype, const float* rope_cos, const float* rope_sin,
                                        int rope_max_pos, cgr_rope_style style, cgr_mask mask, int window,
                                        float softmax_scale, cgr_qk_operand qk_operand, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  cgr_status st = cgr::varlen_check(q, k, v, o, lse, cu_seqlens, num_seqs, total_tokens, max_seqlen, n_head,
                               n_kv_head, head_dim, dtype, rope_cos, rope_sin, rope_max_pos, style, mask, window,
                               softmax_scale, qk_operand);
  if (st != CGR_OK) return st;
  const BwdLayout lay = bwd_varlen_layout(num_seqs, total_tokens, n_head, n_kv_head, head_dim);
  if ((st = bwd_check(lse, dout, dq, dk, dv, head_dim, dtype, window, mask, workspace, workspace_bytes, lay)) !=
      CGR_OK)
    return st;
  const long slots = bwd_varlen_slots(num_seqs, total_tokens);
  if (slots * n_head > INT_MAX) return fail(CGR_ERR_INVALID_ARG, "too many work units");
  if (total_tokens == 0) return CGR_OK;  // nothing to write
  cgr::BwdArgs a{};
  a.B = 1;
  a.T = max_seqlen;
  a.H = n_head;
  a.KV = n_kv_head;
  a.NT = 0;
  a.cu_seqlens = cu_seqlens;
  a.nseq = num_seqs;
  a.total = total_tokens;
  a.NSL = (int)slots;
  return bwd_launch(a, q, k, v, o, lse, dout, dq, dk, dv, head_dim, rope_cos, rope_sin, style, mask, window,
                    softmax_scale, qk_operand, workspace, lay, total_tokens, stream);
}

size_t cgr_attn_decode_workspace_size(int B, int Tq, int max_seqlen, int n_head, int n_kv_head,
                                      int head_dim) {
  if (B < 1 || Tq < 1 || max_seqlen < Tq || n_head < 1 || n_kv_head < 1 || n_head % n_kv_head ||
      head_dim < 2)
    return 0;
  return decode_plan(B, Tq, max_seqlen, n_head, n_kv_head, head_dim).total;
}

cgr_status cgr_gqa_rope_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* cache_seqlens, void* o, float* lse, int B, int Tq,
                                    int cache_capacity, int64_t cache_batch_stride,
                                    int64_t cache_token_stride, int64_t cache_head_stride,
                                    int max_seqlen, int n_head, int n_kv_head, int head_dim,
                                    cgr_dtype dtype, const float* rope_cos, const float* rope_sin,
                                    int rope_max_pos, cgr_rope_style style, int window,
                                    float softmax_scale, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  if (B < 1 || Tq < 1) return fail(CGR_ERR_INVALID_ARG, "B (%d) and Tq (%d) must be >= 1", B, Tq);
  if (!cache_seqlens) return fail(CGR_ERR_INVALID_ARG, "cache_seqlens must be non-null");
  if (!aligned(cache_seqlens, 4)) return fail(CGR_ERR_ALIGNMENT, "cache_seqlens must be 4-byte aligned");
  if (max_seqlen < Tq || max_seqlen > cache_capacity)
    return fail(CGR_ERR_INVALID_ARG, "need Tq (%d) <= max_seqlen (%d) <= cache_capacity (%d)", Tq,
                max_seqlen, cache_capacity);
  cgr_status st = check_common(q, k_cache, v_cache, o, lse, n_head, n_kv_head, head_dim, dtype,
                               rope_cos, rope_sin, rope_max_pos, max_seqlen, style, CGR_MASK_CAUSAL,
                               softmax_scale, CGR_QK_BF16);
  if (st != CGR_OK) return st;
  if (dtype != CGR_BF16)
    return fail(CGR_ERR_UNSUPPORTED, "decode takes bf16 tensors only (dtype %d)", (int)dtype);
  if (head_dim == 256) return fail(CGR_ERR_UNSUPPORTED, "decode is built for head_dim 32, 64, 128");
  if ((st = check_window(window, CGR_MASK_CAUSAL)) != CGR_OK) return st;
  if (cache_batch_stride < 0 || cache_token_stride < head_dim || cache_head_stride < head_dim ||
      cache_batch_stride % 8 || cache_token_stride % 8 || cache_head_stride % 8)
    return fail(CGR_ERR_INVALID_ARG,
                "cache strides must be non-negative multiples of 8 elements, token and head strides "
                ">= head_dim");
  // One (entry, K/V head) is addressed with 32-bit byte offsets.
  if (((long)cache_capacity - 1) * cache_token_stride * 2 + head_dim * 2 > (long)INT_MAX)
    return fail(CGR_ERR_UNSUPPORTED, "one cache entry of %d tokens spans more than 2 GiB", cache_capacity);
  const DecodePlan plan = decode_plan(B, Tq, max_seqlen, n_head, n_kv_head, head_dim);
  if (!workspace) return fail(CGR_ERR_WORKSPACE, "workspace must be non-null");
  if (!aligned(workspace, 256)) return fail(CGR_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  if (workspace_bytes < plan.total)
    return fail(CGR_ERR_WORKSPACE, "workspace has %zu bytes, the call needs %zu", workspace_bytes,
                plan.total);
  if ((long)B * n_kv_head * plan.rg * plan.ns > INT_MAX || (long)B * n_head * Tq * head_dim > INT_MAX)
    return fail(CGR_ERR_INVALID_ARG, "too many work units");
  cgr::DecodeArgs a{};
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.sb = cache_batch_stride;
  a.st = cache_token_stride;
  a.sh = cache_head_stride;
  a.seqlens = cache_seqlens;
  a.o = o;
  a.lse = lse;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.status = (int32_t*)workspace + 2;
  a.part_lse = (float*)((char*)workspace + plan.lse_off);
  a.part_o = (float*)((char*)workspace + plan.o_off);
  a.B = B;
  a.Tq = Tq;
  a.S = cache_capacity;
  a.H = n_head;
  a.KV = n_kv_head;
  a.NS = plan.ns;
  a.CH = plan.ch;
  a.RG = plan.rg;
  a.M = max_seqlen;
  a.window = window;
  const double scale = softmax_scale > 0.f ? (double)softmax_scale : 1.0 / std::sqrt((double)head_dim);
  a.qscale = (float)(scale * 1.4426950408889634074);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  switch (head_dim) {
    case 32: e = cgr::launch_decode_d32(a, (int)style, s); break;
    case 64: e = cgr::launch_decode_d64(a, (int)style, s); break;
    default: e = cgr::launch_decode_d128(a, (int)style, s); break;
  }
  if (e != hipSuccess) return hip_fail("decode launch", e);
  return CGR_OK;
}

cgr_status cgr_rope_rotate(const void* x, void* out, const int32_t* positions, int n_tokens,
                           int n_heads, int head_dim, cgr_dtype dtype, const float* rope_cos,
                           const float* rope_sin, int rope_max_pos, cgr_rope_style style,
                           int32_t* device_status, void* stream) {
  if (!x || !out || !positions || !rope_cos || !rope_sin)
    return fail(CGR_ERR_INVALID_ARG, "x, out, positions, rope_cos and rope_sin must be non-null");
  if (n_tokens < 0 || n_heads < 1)
    return fail(CGR_ERR_INVALID_ARG, "n_tokens (%d) must be >= 0 and n_heads (%d) >= 1", n_tokens,
                n_heads);
  if (head_dim != 32 && head_dim != 64 && head_dim != 128)
    return fail(CGR_ERR_UNSUPPORTED, "head_dim %d is not one of 32, 64, 128", head_dim);
  if (dtype != CGR_F32 && dtype != CGR_BF16)
    return fail(CGR_ERR_UNSUPPORTED, "dtype %d is not CGR_F32 or CGR_BF16", (int)dtype);
  if (style != CGR_ROPE_INTERLEAVED && style != CGR_ROPE_HALF)
    return fail(CGR_ERR_UNSUPPORTED, "unknown rope style %d", (int)style);
  if (rope_max_pos < 1) return fail(CGR_ERR_INVALID_ARG, "rope_max_pos must be >= 1");
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(rope_cos, 16) || !aligned(rope_sin, 16) ||
      !aligned(positions, 4) || (device_status && !aligned(device_status, 4)))
    return fail(CGR_ERR_ALIGNMENT, "x, out and the tables must be 16-byte aligned, positions 4-byte");
  if (n_tokens == 0) return CGR_OK;
  const long rows = (long)n_tokens * n_heads;
  if (rows * (head_dim / 16) > (long)UINT32_MAX * 256)
    return fail(CGR_ERR_INVALID_ARG, "too many rows");
  hipStream_t s = (hipStream_t)stream;
  const int f32 = dtype == CGR_F32;
  hipError_t e;
  switch (head_dim) {
    case 32: e = cgr::launch_rope_rotate_d32(x, out, positions, rows, n_heads, f32, rope_cos, rope_sin, rope_max_pos, (int)style, device_status, s); break;
    case 64: e = cgr::launch_rope_rotate_d64(x, out, positions, rows, n_heads, f32, rope_cos, rope_sin, rope_max_pos, (int)style, device_status, s); break;
    default: e = cgr::launch_rope_rotate_d128(x, out, positions, rows, n_heads, f32, rope_cos, rope_sin, rope_max_pos, (int)style, device_status, s); break;
  }
  if (e != hipSuccess) return hip_fail("rope_rotate launch", e);
  return CGR_OK;
}

size_t cgr_rmsnorm_qkv_rope_workspace_size(int n_tokens, int n_embd, int n_head, int n_kv_head,
                                            int head_dim) {
  if (n_tokens < 1 || n_embd < 1 || n_head < 1 || n_kv_head < 1 || head_dim < 2) return 0;
  const size_t O = (size_t)(n_head + 2 * n_kv_head) * head_dim;
  return 256 + (((size_t)n_tokens * 4 + 255) & ~(size_t)255) + O * n_embd * 2;
}

cgr_status cgr_rmsnorm_qkv_rope(const void* x, const void* norm_weight, float eps, const void* w_qkv,
                                const int32_t* positions, void* q, void* k, void* v, int n_tokens,
                                int n_embd, int n_head, int n_kv_head, int head_dim, cgr_dtype dtype,
                                const float* rope_cos, const float* rope_sin, int rope_max_pos,
                                cgr_rope_style style, int rotate, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!x || !norm_weight || !w_qkv || !positions || !q || !k || !v || !rope_cos || !rope_sin)
    return fail(CGR_ERR_INVALID_ARG, "every tensor pointer must be non-null");
  if (n_tokens < 1 || n_embd < 1 || n_head < 1 || n_kv_head < 1)
    return fail(CGR_ERR_INVALID_ARG, "n_tokens, n_embd, n_head and n_kv_head must be >= 1");
  if (n_head % n_kv_head != 0)
    return fail(CGR_ERR_INVALID_ARG, "n_head (%d) must be divisible by n_kv_head (%d)", n_head, n_kv_head);
  if (head_dim != 32 && head_dim != 64 && head_dim != 128)
    return fail(CGR_ERR_UNSUPPORTED, "head_dim %d is not one of 32, 64, 128", head_dim);
  if (n_embd % 32 != 0) return fail(CGR_ERR_UNSUPPORTED, "n_embd (%d) must be a multiple of 32", n_embd);
  if (dtype != CGR_BF16) return fail(CGR_ERR_UNSUPPORTED, "bf16 tensors only (dtype %d)", (int)dtype);
  if (style != CGR_ROPE_INTERLEAVED && style != CGR_ROPE_HALF)
    return fail(CGR_ERR_UNSUPPORTED, "unknown rope style %d", (int)style);
  if (rotate < 0 || rotate > 3) return fail(CGR_ERR_INVALID_ARG, "rotate must be 0..3 (bit 0: q, bit 1: k)");
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(CGR_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (rope_max_pos < 1) return fail(CGR_ERR_INVALID_ARG, "rope_max_pos must be >= 1");
  if (!aligned(x, 16) || !aligned(norm_weight, 16) || !aligned(w_qkv, 16) || !aligned(q, 16) ||
      !aligned(k, 16) || !aligned(v, 16) || !aligned(rope_cos, 16) || !aligned(rope_sin, 16) ||
      !aligned(positions, 4))
    return fail(CGR_ERR_ALIGNMENT, "tensors must be 16-byte aligned (positions 4-byte)");
  const long O = (long)(n_head + 2 * n_kv_head) * head_dim;
  if ((long)n_tokens * n_embd * 2 > (long)INT_MAX || O * n_embd * 2 > (long)INT_MAX)
    return fail(CGR_ERR_UNSUPPORTED, "x or the projection weight spans more than 2 GiB");
  const size_t need = cgr_rmsnorm_qkv_rope_workspace_size(n_tokens, n_embd, n_head, n_kv_head, head_dim);
  if (!workspace) return fail(CGR_ERR_WORKSPACE, "workspace must be non-null");
  if (!aligned(workspace, 256)) return fail(CGR_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(CGR_ERR_WORKSPACE, "workspace has %zu bytes, the call needs %zu", workspace_bytes, need);
  cgr::QkvArgs a{};
  a.x = x;
  a.norm_w = norm_weight;
  a.w = w_qkv;
  a.positions = positions;
  a.q = q;
  a.k = k;
  a.v = v;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.status = (int32_t*)workspace + 2;
  a.rstd = (float*)((char*)workspace + 256);
  a.wn = (char*)workspace + 256 + (((size_t)n_tokens * 4 + 255) & ~(size_t)255);
  a.N = n_tokens;
  a.C = n_embd;
  a.H = n_head;
  a.KV = n_kv_head;
  a.O = (int)O;
  a.P = rope_max_pos;
  a.rot_q = rotate & 1;
  a.rot_k = (rotate >> 1) & 1;
  a.eps = eps;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  switch (head_dim) {
    case 32: e = cgr::launch_qkv_d32(a, (int)style, s); break;
    case 64: e = cgr::launch_qkv_d64(a, (int)style, s); break;
    default: e = cgr::launch_qkv_d128(a, (int)style, s); break;
  }
  if (e != hipSuccess) return hip_fail("rmsnorm_qkv_rope launch", e);
  return CGR_OK;
}

cgr_status cgr_varlen_device_status(const void* workspace, void* stream, int32_t* host_status) {
  if (!workspace || !host_status)
    return fail(CGR_ERR_INVALID_ARG, "workspace and host_status must be non-null");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(host_status, (const int32_t*)workspace + 2, sizeof(int32_t),
                                hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail("status copy", e);
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail("stream synchronize", e);
  return CGR_OK;
}

const char* cgr_last_error(void) { return g_last_error.c_str(); }

int cgr_version(void) { return 10000; }

}  // extern "C"
