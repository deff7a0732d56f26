// Backward of the fused causal GQA + RoPE attention for gfx950 (internal to
// libcgr).
//
// What is computed: the chain rule through the forward's definition ("Attention
// from Scratch", section "Attention, the math"; "Train It & Run for Real",
// section "Coming from CUDA: where's .backward()?": every op of the model,
// attention and RoPE included, carries its backward). Per sequence and query
// head h with K/V head h / G, in the rotated frame (q~ = R q, k~ = R k):
//   P_ij  = exp(scale q~_i.k~_j - lse_i)      (the forward's log-sum-exp)
//   dP_ij = dO_i . v_j,  D_i = dO_i . O_i = sum_j P_ij dP_ij
//   dS_ij = P_ij (dP_ij - D_i)
//   dv_j += sum_i P_ij dO_i
//   dk~_j += scale sum_i dS_ij q~_i,   dq~_i = scale sum_j dS_ij k~_j
//   dq = R^T dq~,  dk = R^T dk~   (the transposed rotation, at the row's position)
// dk and dv sum over the G query heads that share the K/V head.
//
// Three kernels (and a fourth with many query heads per K/V head):
//   * bwd_prep_kernel: q~ * scale*log2(e) and k~ in the Q.K^T operand type (so
//     the rotation is done once, not once per tile that reads them), and per
//     32-row tile of every (sequence, head) the two accumulator starting
//     values -lse*log2(e) and -D.
//   * attn_bwd_dkdv_kernel: one workgroup per (sequence, K/V head, 128 keys,
//     group of up to 4 query heads). Each wave keeps 32 keys' k~ in registers
//     as a matrix-core operand and accumulates dk~^T and dv^T for them over
//     every query row of its query heads; S = q~ k~^T puts one key per lane
//     column, so P and dS feed dv^T += dO^T P and dk~^T += q~^T dS straight
//     from registers. With more than 4 query heads per K/V head the head
//     groups write f32 partial sums and bwd_dkv_reduce_kernel adds them.
//   * attn_bwd_dq_kernel: one workgroup per (sequence, 2^lhp query heads of
//     one K/V head, 256 / 2^lhp rows), the forward's layout: S^T = k~ q~^T
//     puts one query per lane column and dq~^T += k~^T dS^T takes dS^T from
//     registers.
// Recomputing S and dP in both kernels costs two extra matrix products per
// tile against sharing dS through memory, and buys a backward without atomics
// or a dS round trip: every output element is written once, by one lane, in a
// fixed order (bit-for-bit repeatable).
#pragma once

#include "tile_common.h"

namespace cgr {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;  // [B, H, T], natural log (the forward's)
  void* dq;
  void* dk;
  void* dv;
  const float* rope_cos;  // [P, D/2]
  const float* rope_sin;
  // Workspace (written by bwd_prep_kernel).
  void* qr;   // [B, T, H, D] operand type: R q * scale * log2(e)
  void* kr;   // [B, T, KV, D] operand type: R k
  float* ld;  // [B, H, NT][64] (dense) or [H, NSL][64] (packed): per 32-row tile,
              // -lse*log2(e) (rows 0..31) then -D
  int B, T, H, KV, NT;
  // Packed batches (cu_seqlens non-null): nseq sequences, total tokens, T =
  // max_seqlen; tensors [total, heads, D], lse [H, total]. Sequence s's blocks
  // of 2^k rows take slots (c_s >> k) + s on (slot_owner); NSL is the number
  // of 32-row slots per head in ld.
  const int32_t* cu_seqlens;
  int nseq, total, NSL;
  // dk/dv units take at most kBwdHeadsPerUnit query heads of their K/V head;
  // with more (hsplit > 1) each writes f32 partial sums, dv then dk~ (before
  // the transposed rotation), to part[split][row][K/V head][D], rows = B*T or
  // total, dv's splits first, and bwd_dkv_reduce_kernel adds them in split
  // order.
  int hsplit;
  long part_rows;
  float* part;
  // dq units: 2^lhp query heads of one K/V head (lhp <= 3, 2^lhp divides G)
  // x 256 / 2^lhp rows; wave w takes head w >> (3 - lhp) of the unit's heads
  // and rows 32 (w mod 2^(3 - lhp)) on.
  int lhp;
  int window;    // > 0 (causal only): keys 0 <= i - j < window; 0: none
  float qscale;  // scale * log2(e)
  float scale;
  // Dense causal calls: claim counters of the dk/dv ([0]) and dq ([1])
  // kernels' lightest ranks (zeroed by bwd_prep_kernel; see claim_unit).
  int32_t* ctr;
};

// The lightest ranks of a dense causal backward kernel (a quarter of them,
// kfwd_dyn_ranks) are not placed by workgroup index: the workgroups past the
// statically placed ones (two for each such unit) claim them in order from a
// counter, so an XCD that runs ahead of the others (their clocks differ by
// 5-6 % under load) takes more of them. Returns the claim's number: the index
// of the claimed unit among those units, or a number past them when none is
// left. Each of those workgroups calls it once, with all its threads.
__device__ __forceinline__ int claim_unit(int32_t* ctr) {
  __shared__ int claim;
  if (threadIdx.x == 0) claim = atomicAdd(ctr, 1);
  __syncthreads();
  return claim;
}

constexpr int kBwdTileRows = 32;  // rows per ld tile
// Query heads per dk/dv unit: with G > 4 (MQA, few K/V heads) a K/V head's
// keys are split over ceil(G / 4) units so that the grid fills the chip and
// no single unit carries all G heads' rows.
constexpr int kBwdHeadsPerUnit = 4;

// Packed batches: sequence s's blocks of 2^lb tokens take slots (c_s >> lb) + s
// on (c_s = cu_seqlens[s]). The next sequence's first slot lies past s's last
// ((c_s >> lb) + ceil(L_s / 2^lb) <= (c_{s+1} >> lb) + 1), so no slot has two
// sequences, and all stay below ceil(total / 2^lb) + nseq. The owner of a
// slot is the last sequence whose first slot is at or before it; callers
// check that the block lies inside it (slots between sequences belong to
// none). The search's reads stay inside cu_seqlens whatever it holds.
__device__ __forceinline__ int slot_owner(const int32_t* cu, int nseq, int lb, int slot) {
  int lo = 0, hi = nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((cu[mid] >> lb) + mid <= slot) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Packed batches: whether sequence s (tokens c0 .. c0 + L - 1) lies inside the
// batch as the forward validated it; a unit of a sequence that does not
// touches no memory.
__device__ __forceinline__ bool seq_ok(const BwdArgs& a, int c0, int L) {
  return c0 >= 0 && L >= 0 && L <= a.T && c0 <= a.total - L;
}

// ---------------------------------------------------------------------------
// Prepass. Item = (row, group g < D/16), covering the chunk pair (g, g + D/16)
// so that both pairings find their partners (as the forward's K loader). The
// query part runs over rows padded to whole 32-row tiles; padding rows get
// -lse = -inf (no probability) and -D = 0.
template <int D, typename QK, int STYLE>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  constexpr int IPR = D / 16;  // items per row
  const long tid = (long)blockIdx.x * 256 + threadIdx.x;
  const int Tp = a.NT * kBwdTileRows;
  const long nq = (long)a.B * Tp * a.H * IPR;
  const long nk = (long)a.B * a.T * a.KV * IPR;
  const int g = (int)(tid % IPR);
  if (tid == 0) a.ctr[0] = a.ctr[1] = 0;  // the claim counters of the two gradient kernels
  if (tid < nq) {
    const long row = tid / IPR;  // ((b * Tp + t) * H + h)
    const int h = (int)(row % a.H);
    const long bt = row / a.H;
    const int t = (int)(bt % Tp), b = (int)(bt / Tp);
    const bool ok = t < a.T;
    float dot = 0.f;
    if (ok) {
      const long e0 = (((long)b * a.T + t) * a.H + h) * D;
      const uint16_t* qp = (const uint16_t*)a.q + e0;
      u32x4 w0[1] = {*(const u32x4*)(qp + 8 * g)}, w1[1] = {*(const u32x4*)(qp + 8 * g + D / 2)};
      float x0[8], x1[8];
      raw_to_f32<uint16_t>(w0, x0);
      raw_to_f32<uint16_t>(w1, x1);
      f32x4 c[2], s[2];
      load_tab<D, STYLE>(a.rope_cos + (long)t * (D / 2), a.rope_sin + (long)t * (D / 2), g, true, c, s);
      rope_pair<STYLE>(x0, x1, c, s);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x0[j] *= a.qscale;
        x1[j] *= a.qscale;
      }
      uint16_t* qo = (uint16_t*)a.qr + e0;
      *(u32x4*)(qo + 8 * g) = to_frag<QK>(x0).v;
      *(u32x4*)(qo + 8 * g + D / 2) = to_frag<QK>(x1).v;
      // D_i over this item's 16 elements.
      const uint16_t* op = (const uint16_t*)a.o + e0;
      const uint16_t* dp = (const uint16_t*)a.dout + e0;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int off = 8 * g + half * (D / 2);
        u32x4 wo[1] = {*(const u32x4*)(op + off)}, wd[1] = {*(const u32x4*)(dp + off)};
        float xo[8], xd[8];
        raw_to_f32<uint16_t>(wo, xo);
        raw_to_f32<uint16_t>(wd, xd);
#pragma unroll
        for (int j = 0; j < 8; ++j) dot += xo[j] * xd[j];
      }
    }
#pragma unroll
    for (int m = 1; m < IPR; m <<= 1) dot += __shfl_xor(dot, m, 64);
    if (g == 0) {
      float* l = a.ld + (((long)b * a.H + h) * a.NT + t / kBwdTileRows) * 64 + t % kBwdTileRows;
      l[0] = ok ? -a.lse[((long)b * a.H + h) * a.T + t] * 1.4426950408889634f : -INFINITY;
      l[32] = ok ? -dot : 0.f;
    }
  } else if (tid < nq + nk) {
    const long row = (tid - nq) / IPR;  // ((b * T + t) * KV + kv)
    const long bt = row / a.KV;
    const int t = (int)(bt % a.T);
    const long e0 = row * D;
    const uint16_t* kp = (const uint16_t*)a.k + e0;
    u32x4 w0[1] = {*(const u32x4*)(kp + 8 * g)}, w1[1] = {*(const u32x4*)(kp + 8 * g + D / 2)};
    float x0[8], x1[8];
    raw_to_f32<uint16_t>(w0, x0);
    raw_to_f32<uint16_t>(w1, x1);
    f32x4 c[2], s[2];
    load_tab<D, STYLE>(a.rope_cos + (long)t * (D / 2), a.rope_sin + (long)t * (D / 2), g, true, c, s);
    rope_pair<STYLE>(x0, x1, c, s);
    uint16_t* ko = (uint16_t*)a.kr + e0;
    *(u32x4*)(ko + 8 * g) = to_frag<QK>(x0).v;
    *(u32x4*)(ko + 8 * g + D / 2) = to_frag<QK>(x1).v;
  }
}

// The prepass of a packed batch. Query items (32-row slot, head, row of the
// slot, group) write the rotated q of their token and the slot's starting
// values (rows past their sequence, and slots between sequences, get -inf and
// 0); key items (token, K/V head, group) find their token's sequence by
// binary search over cu_seqlens (positions restart at 0 in every sequence).
template <int D, typename QK, int STYLE>
__global__ __launch_bounds__(256) void bwd_prep_varlen_kernel(BwdArgs a) {
  constexpr int IPR = D / 16;
  const long tid = (long)blockIdx.x * 256 + threadIdx.x;
  const long nq = (long)a.NSL * a.H * kBwdTileRows * IPR;
  const long nk = (long)a.total * a.KV * IPR;
  const int g = (int)(tid % IPR);
  if (tid < nq) {
    const long row = tid / IPR;  // (slot * H + h) * 32 + r
    const int r = (int)(row % kBwdTileRows);
    const long sh = row / kBwdTileRows;
    const int h = (int)(sh % a.H), slot = (int)(sh / a.H);
    const int s = slot_owner(a.cu_seqlens, a.nseq, 5, slot);
    const int c0 = a.cu_seqlens[s], L = a.cu_seqlens[s + 1] - c0;
    const int t = (slot - ((c0 >> 5) + s)) * kBwdTileRows + r;
    const bool ok = seq_ok(a, c0, L) && t >= 0 && t < L;
    float dot = 0.f;
    if (ok) {
      const long e0 = ((long)(c0 + t) * a.H + h) * D;
      const uint16_t* qp = (const uint16_t*)a.q + e0;
      u32x4 w0[1] = {*(const u32x4*)(qp + 8 * g)}, w1[1] = {*(const u32x4*)(qp + 8 * g + D / 2)};
      float x0[8], x1[8];
      raw_to_f32<uint16_t>(w0, x0);
      raw_to_f32<uint16_t>(w1, x1);
      f32x4 c[2], sn[2];
      load_tab<D, STYLE>(a.rope_cos + (long)t * (D / 2), a.rope_sin + (long)t * (D / 2), g, true, c, sn);
      rope_pair<STYLE>(x0, x1, c, sn);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x0[j] *= a.qscale;
        x1[j] *= a.qscale;
      }
      uint16_t* qo = (uint16_t*)a.qr + e0;
      *(u32x4*)(qo + 8 * g) = to_frag<QK>(x0).v;
      *(u32x4*)(qo + 8 * g + D / 2) = to_frag<QK>(x1).v;
      const uint16_t* op = (const uint16_t*)a.o + e0;
      const uint16_t* dp = (const uint16_t*)a.dout + e0;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int off = 8 * g + half * (D / 2);
        u32x4 wo[1] = {*(const u32x4*)(op + off)}, wd[1] = {*(const u32x4*)(dp + off)};
        float xo[8], xd[8];
        raw_to_f32<uint16_t>(wo, xo);
        raw_to_f32<uint16_t>(wd, xd);
#pragma unroll
        for (int j = 0; j < 8; ++j) dot += xo[j] * xd[j];
      }
    }
#pragma unroll
    for (int m = 1; m < IPR; m <<= 1) dot += __shfl_xor(dot, m, 64);
    if (g == 0) {
      float* l = a.ld + ((long)h * a.NSL + slot) * 64 + r;
      l[0] = ok ? -a.lse[(long)h * a.total + c0 + t] * 1.4426950408889634f : -INFINITY;
      l[32] = ok ? -dot : 0.f;
    }
  } else if (tid < nq + nk) {
    const long row = (tid - nq) / IPR;  // p * KV + kv
    const int p = (int)(row / a.KV);
    // The sequence holding token p: the last s with cu_seqlens[s] <= p.
    int lo = 0, hi = a.nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cu_seqlens[mid] <= p) lo = mid;
      else hi = mid - 1;
    }
    const int t = p - a.cu_seqlens[lo];
    const long e0 = row * D;
    u32x4 o0 = {0u, 0u, 0u, 0u}, o1 = {0u, 0u, 0u, 0u};
    if (t >= 0 && t < a.T) {
      const uint16_t* kp = (const uint16_t*)a.k + e0;
      u32x4 w0[1] = {*(const u32x4*)(kp + 8 * g)}, w1[1] = {*(const u32x4*)(kp + 8 * g + D / 2)};
      float x0[8], x1[8];
      raw_to_f32<uint16_t>(w0, x0);
      raw_to_f32<uint16_t>(w1, x1);
      f32x4 c[2], sn[2];
      load_tab<D, STYLE>(a.rope_cos + (long)t * (D / 2), a.rope_sin + (long)t * (D / 2), g, true, c, sn);
      rope_pair<STYLE>(x0, x1, c, sn);
      o0 = to_frag<QK>(x0).v;
      o1 = to_frag<QK>(x1).v;
    }
    uint16_t* ko = (uint16_t*)a.kr + e0;
    *(u32x4*)(ko + 8 * g) = o0;
    *(u32x4*)(ko + 8 * g + D / 2) = o1;
  }
}

// ---------------------------------------------------------------------------
// dk, dv. Workgroup = 8 waves = two groups of 4; wave w holds keys
// k0 + 32(w%4) .. +31 of the workgroup's 128. The work items are (32-row
// query step, query head of the K/V group); group 0 takes the even items and
// group 1 the odd ones, so the two waves of a SIMD (w and w+4, same keys)
// split the work, and their partial sums meet in LDS at the end.
// Per item and wave (32 query rows x 32 keys):
//   S  = q~ k~^T - lse        (rows = queries, lane column = key; log2 units)
//   dP = dO v^T - D
//   P = 2^S;  dS = P dP
//   dv^T += dO^T P            (dO^T by transposing LDS reads)
//   dk~^T += q~^T dS
template <int D_, typename QK_, bool CAUSAL_, int STYLE_, bool WIN_ = false>
struct BwdCfg {
  static constexpr int D = D_;
  using QK = QK_;
  static constexpr bool CAUSAL = CAUSAL_;
  static constexpr int STYLE = STYLE_;
  static constexpr bool WIN = WIN_ && CAUSAL_;  // sliding-window instances are separate
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int TILE = 32 * 2 * D;                // one 32-row operand tile
  static constexpr int GSTAGE = 2 * TILE + 256;          // q~, dO, ld of one group
  static constexpr int KV_STAGE = 2 * GSTAGE;            // both groups
  static constexpr int BK = 128;                         // keys per dk/dv workgroup
  static constexpr int BQ = 256;                         // rows x heads per dq workgroup
  static constexpr int BN = 64;                          // keys per dq tile
  static constexpr int KT = BN * 2 * D;                  // one dq key tile
};

template <class C>
__global__ __launch_bounds__(512, 2) void attn_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int D = C::D, KSTEPS = C::KSTEPS, DB = C::DB;
  using QK = typename C::QK;
  __shared__ __attribute__((aligned(16))) char st0[C::KV_STAGE], st1[C::KV_STAGE];
  __shared__ __attribute__((aligned(16))) char vk[C::BK * 2 * C::D];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wig = wave & 3;
  const int l32 = lane & 31, hh = lane >> 5;
  const int G = a.H / a.KV;
  // Split sp of a unit takes query heads g0 .. g0 + nh - 1 of the K/V head.
  const int sp = (int)(blockIdx.x % (unsigned)a.hsplit), u = (int)(blockIdx.x / (unsigned)a.hsplit);
  const int g0 = sp * kBwdHeadsPerUnit, nh = min(kBwdHeadsPerUnit, G - g0);
  int kb, kvh, L, tok0;
  long ldt0, ldh;  // ld tile of the sequence's row 0 at head 0; tiles per head
  if (a.cu_seqlens) {
    // Packed: unit = (128-key slot, K/V head), the heads innermost (with 8 or
    // more K/V heads each XCD keeps the same heads). Each sequence's first
    // (heaviest, causal) block comes before its later ones.
    static_assert(C::BK == 1 << 7, "slots of 128 keys");
    const int slot = u / a.KV;
    kvh = u - slot * a.KV;
    const int s = slot_owner(a.cu_seqlens, a.nseq, 7, slot);
    tok0 = a.cu_seqlens[s];
    L = a.cu_seqlens[s + 1] - tok0;
    kb = slot - ((tok0 >> 7) + s);
    if (!seq_ok(a, tok0, L) || kb < 0 || kb * C::BK >= L) return;
    ldt0 = (tok0 >> 5) + s;
    ldh = a.NSL;
  } else {
    // Heavy blocks first (causal: the first keys see the most queries); when
    // the (batch, K/V head) groups divide evenly over the 8 XCDs, each XCD
    // keeps whole groups, whose queries it then streams through one L2.
    const int groups = a.B * a.KV;
    int rank, gsel;
    const int nK = (a.T + C::BK - 1) / C::BK, R0 = nK - kfwd_dyn_ranks(nK);
    if (C::CAUSAL && !C::WIN && a.hsplit == 1 && u >= R0 * groups) {
      const int d = claim_unit(a.ctr);
      if (d >= (nK - R0) * groups) return;
      rank = R0 + d / groups;
      gsel = d - (rank - R0) * groups;
    } else if ((groups & 7) == 0) {
      const int x = u & 7, i = u >> 3, per = groups >> 3;
      rank = i / per;
      gsel = (i - rank * per) * 8 + x;
    } else {
      rank = u / groups;
      gsel = u - rank * groups;
    }
    kb = rank;
    const int b = gsel / a.KV;
    kvh = gsel - b * a.KV;
    L = a.T;
    tok0 = b * a.T;
    ldt0 = (long)b * a.H * a.NT;
    ldh = a.NT;
  }
  const int k0 = kb * C::BK, kw0 = k0 + 32 * wig;
  const int qs = a.H * D, ks = a.KV * D;  // token strides (elements)

  // This wave's keys: k~ as the B operand of S in registers (k-step s of lane
  // (key l32, hh) = elements 16s + 8hh .. +7); v, the B operand of dP, is read
  // from the workgroup's LDS copy (registers are short: the two accumulators
  // take half of them).
  const rsrc_t rkr = make_rsrc((const uint16_t*)a.kr + ((long)tok0 * ks + kvh * D),
                               (uint32_t)(((L - 1) * ks + D) * 2));
  const rsrc_t rv = make_rsrc((const uint16_t*)a.v + ((long)tok0 * ks + kvh * D),
                              (uint32_t)(((L - 1) * ks + D) * 2));
  u32x4 kf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) kf[s] = buf_load16(rkr, (kw0 + l32) * ks * 2 + (2 * s + hh) * 16, 0);
  tile_to_lds<D, C::BK>(rv, vk, ks * 2, k0 * ks * 2, wave, 8, lane);
  const int vrow = 32 * wig + l32;

  // Rows that can see these keys: from the first key on (causal), up to the
  // last key + W - 1 (sliding window).
  const int W = C::WIN ? a.window : 0;
  const int q_first = C::CAUSAL ? k0 : 0;
  const int q_end = W > 0 ? min(L, k0 + C::BK - 1 + W) : L;
  const int n_steps = (q_end - q_first + 31) / 32;
  const int n_items = nh * n_steps;
  const int n_iter = (n_items + 1) / 2;
  const long ld_tiles = a.cu_seqlens ? (long)a.H * a.NSL : (long)a.B * a.H * a.NT;
  const rsrc_t rld = make_rsrc(a.ld, (uint32_t)(ld_tiles * 256));

  // Item n = (query step, head g) with the heads innermost and the steps from
  // the last rows back: the workgroups of one K/V head (which share an XCD)
  // then stream the same query rows at about the same time, and both groups
  // of a workgroup work on the same rows, so most reloads hit L2.
  auto item = [&](int n, int& g, int& qrow0) {
    const int sidx = n / nh;
    g = g0 + n - sidx * nh;
    qrow0 = q_first + 32 * (n_steps - 1 - sidx);
  };
  // Loads of iteration i (this group's item 2i + grp) into a stage.
  const TileCopy<D, 32, 4> qcopy(wig, qs * 2, lane);
  auto issue = [&](int i, char* st) {
    const int n = 2 * i + grp;
    if (n >= n_items) return;
    int g, qrow0;
    item(n, g, qrow0);
    const int h = kvh * G + g;
    char* gs = st + grp * C::GSTAGE;
    const long hoff = (long)tok0 * qs + (long)h * D;
    const rsrc_t rq = make_rsrc((const uint16_t*)a.qr + hoff, (uint32_t)(((L - 1) * qs + D) * 2));
    const rsrc_t rd = make_rsrc((const uint16_t*)a.dout + hoff, (uint32_t)(((L - 1) * qs + D) * 2));
    qcopy(rq, gs, qrow0 * qs * 2);
    qcopy(rd, gs + C::TILE, qrow0 * qs * 2);
    if (wig == 0) {
      const long t = ldt0 + (long)h * ldh + qrow0 / 32;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rld, (lds_void*)(gs + 2 * C::TILE), 4, lane * 4,
                                               (int)(t * 256), 0, 0);
    }
  };

  const TrOffsets<D> tro(lane);
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dk[db] = dv[db] = (f32x16){};

  auto compute = [&](int i, const char* st) {
    const int n = 2 * i + grp;
    if (n >= n_items) return;
    int g, qrow0;
    item(n, g, qrow0);
    if (C::CAUSAL && qrow0 < kw0) return;  // every key of the wave is later than every row
    if (W > 0 && qrow0 - (kw0 + 31) >= W) return;  // every row is past every key's window
    const char* gs = st + grp * C::GSTAGE;
    const char* Qt = gs;
    const char* Ot = gs + C::TILE;
    const float* ldt = (const float*)(gs + 2 * C::TILE);
    f32x16 sacc, dpacc;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 x = *(const f32x4*)(ldt + 8 * r + 4 * hh);
      const f32x4 y = *(const f32x4*)(ldt + 32 + 8 * r + 4 * hh);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        sacc[4 * r + m] = x[m];
        dpacc[4 * r + m] = y[m];
      }
    }
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      sacc = mma32(frag<QK>(row_frag<D>(Qt, l32, s, hh)), frag<QK>(kf[s]), sacc);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      dpacc = mma32(frag<OpBF16>(row_frag<D>(Ot, l32, s, hh)), frag<OpBF16>(row_frag<D>(vk, vrow, s, hh)),
                    dpacc);
    if (C::CAUSAL && qrow0 == kw0) {
      // Diagonal block: key l32 is visible to row 8(i/4) + 4hh + i%4 iff key <= row.
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (l32 > 8 * (r >> 2) + 4 * hh + (r & 3)) sacc[r] = -INFINITY;
    }
    if (W > 0 && qrow0 + 31 - kw0 >= W) {
      // Window's far edge: row - key >= W is hidden.
      const int lim = W - 1 + kw0 + l32 - qrow0 - 4 * hh;  // row offset must be <= lim
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) > lim) sacc[r] = -INFINITY;
    }
    u32x4 pb[2], sb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = 8 * t + 2 * m;
        const float p0 = fast_exp2(sacc[r]), p1 = fast_exp2(sacc[r + 1]);
        pb[t][m] = pack2(OpBF16{}, p0, p1);
        sb[t][m] = pack2(QK{}, p0 * dpacc[r], p1 * dpacc[r + 1]);
      }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dv[db] = mma32(frag<OpBF16>(tr_frag<D>(Ot, 16 * t, db, tro)), frag<OpBF16>(pb[t]), dv[db]);
        dk[db] = mma32(frag<QK>(tr_frag<D>(Qt, 16 * t, db, tro)), frag<QK>(sb[t]), dk[db]);
      }
  };

  issue(0, st0);
  wait_vmem();
  __syncthreads();
  int i = 0;
  for (; i + 1 < n_iter; i += 2) {
    issue(i + 1, st1);
    compute(i, st0);
    wait_vmem();
    __syncthreads();
    issue(i + 2, st0);
    compute(i + 1, st1);
    wait_vmem();
    __syncthreads();
  }
  if (i < n_iter) {
    compute(i, st0);
    __syncthreads();
  }

  // Group 1 hands its partial sums to group 0 through LDS, RR registers of
  // one 32-wide block at a time, alternating between the two stage arrays (a
  // piece is written only after the barrier that follows the previous piece,
  // by which time group 0 has read the piece before that). Word (wig, r) of
  // lane l sits at (wig * RR + r) * 64 + l.
  constexpr int RR = C::KV_STAGE >= 16 * 1024 ? 16 : 8;
  static_assert(C::KV_STAGE >= RR * 1024, "a reduction piece fits a stage");
  auto reduce = [&](f32x16 (&acc)[DB], int p0) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int hf = 0; hf < 16 / RR; ++hf) {
        const int p = p0 + db * (16 / RR) + hf;
        float* red = (float*)((p & 1) ? st1 : st0);
        if (grp == 1) {
#pragma unroll
          for (int r = 0; r < RR; ++r) red[(wig * RR + r) * 64 + lane] = acc[db][hf * RR + r];
        }
        __syncthreads();
        if (grp == 0) {
#pragma unroll
          for (int r = 0; r < RR; ++r) acc[db][hf * RR + r] += red[(wig * RR + r) * 64 + lane];
        }
      }
  };
  reduce(dv, 0);
  reduce(dk, DB * (16 / RR));
  if (grp != 0) return;

  const int key = kw0 + l32;
  if (a.hsplit > 1) {
    // This split's f32 partial sums; the reduction pass finishes them.
    const long split_elems = a.part_rows * ks;
    const uint32_t range = (uint32_t)(((L - 1) * ks + D) * 4);
    const long off = (long)tok0 * ks + kvh * D;
    store_acc_f32<D>(dv, make_rsrc(a.part + sp * split_elems + off, range), key * ks * 4, hh);
    store_acc_f32<D>(dk, make_rsrc(a.part + (a.hsplit + sp) * split_elems + off, range), key * ks * 4, hh);
    return;
  }
  const rsrc_t rdv = make_rsrc((uint16_t*)a.dv + ((long)tok0 * ks + kvh * D), (uint32_t)(((L - 1) * ks + D) * 2));
  const rsrc_t rdk = make_rsrc((uint16_t*)a.dk + ((long)tok0 * ks + kvh * D), (uint32_t)(((L - 1) * ks + D) * 2));
  store_acc_bf16<D>(dv, 1.f, rdv, key * ks * 2, hh);
  // dk~ = scale * sum dS q~ and the q~ operand carried scale*log2(e): one ln 2.
  if (key < L) rope_transpose_acc<D, C::STYLE>(dk, a.rope_cos, a.rope_sin, key, hh);
  store_acc_bf16<D>(dk, 0.69314718055994531f, rdk, key * ks * 2, hh);
}

// The end of a split dk/dv (hsplit > 1): per (row, K/V head) the splits'
// partial sums of dv and dk~ added in split order, dk = R^T dk~ * ln 2 at the
// row's position (the q~ operand carried scale*log2(e)), both rounded to
// bf16. Thread = (row, K/V head, group g): elements 8g..8g+7 and the same
// eight D/2 further on, which hold whole rotation pairs in both pairings.
template <int D, int STYLE>
__global__ __launch_bounds__(256) void bwd_dkv_reduce_kernel(BwdArgs a) {
  constexpr int IPR = D / 16;
  const long tid = (long)blockIdx.x * 256 + threadIdx.x;
  if (tid >= a.part_rows * a.KV * IPR) return;
  const int g = (int)(tid % IPR);
  const long row = tid / IPR;  // token * KV + kvh
  const int p = (int)(row / a.KV);
  int t;
  if (a.cu_seqlens) {
    // Rows of a sequence whose units exited (not inside the batch) stay unwritten.
    int lo = 0, hi = a.nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.cu_seqlens[mid] <= p) lo = mid;
      else hi = mid - 1;
    }
    const int c0 = a.cu_seqlens[lo], L = a.cu_seqlens[lo + 1] - c0;
    t = p - c0;
    if (!seq_ok(a, c0, L) || t < 0 || t >= L) return;
  } else {
    t = p % a.T;
  }
  const long split_elems = a.part_rows * a.KV * D;
  const float* pv = a.part + row * D + 8 * g;
  const float* pk = pv + a.hsplit * split_elems;
  float v0[8], v1[8], k0[8], k1[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v0[j] = v1[j] = k0[j] = k1[j] = 0.f;
  for (int sp = 0; sp < a.hsplit; ++sp) {
    const long o = sp * split_elems;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 a0 = *(const f32x4*)(pv + o + 4 * h), a1 = *(const f32x4*)(pv + o + D / 2 + 4 * h);
      const f32x4 b0 = *(const f32x4*)(pk + o + 4 * h), b1 = *(const f32x4*)(pk + o + D / 2 + 4 * h);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        v0[4 * h + m] += a0[m];
        v1[4 * h + m] += a1[m];
        k0[4 * h + m] += b0[m];
        k1[4 * h + m] += b1[m];
      }
    }
  }
  // R^T is the rotation by the negated angle.
  f32x4 c[2], sn[2];
  load_tab<D, STYLE>(a.rope_cos + (long)t * (D / 2), a.rope_sin + (long)t * (D / 2), g, true, c, sn);
  sn[0] = -sn[0];
  sn[1] = -sn[1];
  rope_pair<STYLE>(k0, k1, c, sn);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    k0[j] *= 0.69314718055994531f;
    k1[j] *= 0.69314718055994531f;
  }
  uint16_t* dvo = (uint16_t*)a.dv + row * D + 8 * g;
  uint16_t* dko = (uint16_t*)a.dk + row * D + 8 * g;
  *(u32x4*)dvo = to_frag<OpBF16>(v0).v;
  *(u32x4*)(dvo + D / 2) = to_frag<OpBF16>(v1).v;
  *(u32x4*)dko = to_frag<OpBF16>(k0).v;
  *(u32x4*)(dko + D / 2) = to_frag<OpBF16>(k1).v;
}

// ---------------------------------------------------------------------------
// dq. Workgroup = 8 waves x 32 query rows: 2^lhp query heads of one K/V head
// (the largest power of two up to 8 that divides G) x 256 / 2^lhp rows, so
// that with several heads the waves' rows end close together at the causal
// diagonal; key tiles of 64 stream through LDS (k~ and v, double-buffered,
// direct loads) for all of them. Per tile and wave:
//   S^T  = k~ q~^T - lse      (rows = keys, lane column = query)
//   dP^T = v dO^T - D
//   P^T = 2^S^T;  dS^T = P^T dP^T
//   dq~^T += k~^T dS^T        (k~^T by transposing LDS reads)
template <class C>
__global__ __launch_bounds__(512, 2) void attn_bwd_dq_kernel(BwdArgs a) {
  constexpr int D = C::D, KSTEPS = C::KSTEPS, DB = C::DB, BN = C::BN;
  using QK = typename C::QK;
  __shared__ __attribute__((aligned(16))) char kt0s[C::KT], kt1s[C::KT];
  __shared__ __attribute__((aligned(16))) char vt0s[C::KT], vt1s[C::KT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int G = a.H / a.KV;
  // A unit: 2^lhp heads (head group hg of the K/V head) x BQ = 256 / 2^lhp rows.
  const int lhp = a.lhp, NHG = G >> lhp;
  const int lbq = 8 - lhp, BQ = 1 << lbq;
  const int u = blockIdx.x;
  int qb, kvh, hg, L, tok0;
  long ldt0, ldh;  // ld tile of the sequence's row 0 at head 0; tiles per head
  if (a.cu_seqlens) {
    // Packed: unit = (BQ-row slot, head group), the head groups innermost and
    // the slots from the last back (causal: each sequence's last, heaviest
    // block first). With a multiple of 8 K/V heads, group i of a slot takes
    // K/V head ((i / 8) / NHG) * 8 + i % 8, so each XCD keeps the same K/V
    // heads.
    const int per = a.H >> lhp;
    const int slot = (int)gridDim.x / per - 1 - u / per;  // the grid has every slot
    const int i = u - (u / per) * per;
    if ((a.KV & 7) == 0) {
      kvh = ((i >> 3) / NHG) * 8 + (i & 7);
      hg = (i >> 3) % NHG;
    } else {
      kvh = i / NHG;
      hg = i % NHG;
    }
    const int s = slot_owner(a.cu_seqlens, a.nseq, lbq, slot);
    tok0 = a.cu_seqlens[s];
    L = a.cu_seqlens[s + 1] - tok0;
    qb = slot - ((tok0 >> lbq) + s);
    if (!seq_ok(a, tok0, L) || qb < 0 || qb * BQ >= L) return;
    ldt0 = (tok0 >> 5) + s;
    ldh = a.NSL;
  } else {
    const int nQ = (a.T + BQ - 1) >> lbq;
    const int groups = a.B * a.KV;
    int rank, gsel;
    const int R0 = nQ - kfwd_dyn_ranks(nQ);
    if (C::CAUSAL && !C::WIN && u >= R0 * groups * NHG) {
      const int d = claim_unit(a.ctr + 1);
      if (d >= (nQ - R0) * groups * NHG) return;
      rank = R0 + d / (groups * NHG);
      const int rem = d - (rank - R0) * groups * NHG;
      gsel = rem / NHG;
      hg = rem - gsel * NHG;
    } else if ((groups & 7) == 0) {
      const int x = u & 7, i = u >> 3, per = (groups >> 3) * NHG;
      rank = i / per;
      const int rem = i - rank * per;
      gsel = (rem / NHG) * 8 + x;
      hg = rem % NHG;
    } else {
      const int per = groups * NHG;
      rank = u / per;
      const int rem = u - rank * per;
      gsel = rem / NHG;
      hg = rem % NHG;
    }
    qb = C::CAUSAL ? nQ - 1 - rank : rank;
    const int b = gsel / a.KV;
    kvh = gsel - b * a.KV;
    L = a.T;
    tok0 = b * a.T;
    ldt0 = (long)b * a.H * a.NT;
    ldh = a.NT;
  }
  const int head = kvh * G + (hg << lhp) + (wave >> (3 - lhp));
  const int qs = a.H * D, ks = a.KV * D;
  const int q0 = qb * BQ, qw0 = q0 + 32 * (wave & ((8 >> lhp) - 1)), my_q = qw0 + l32;
  const bool wave_has_rows = qw0 < L;
  const int wave_last = min(qw0 + 31, L - 1);
  const int q_hi = min(q0 + BQ, L);
  const int n_tiles = C::CAUSAL ? (q_hi + BN - 1) / BN : (L + BN - 1) / BN;
  // Sliding window: from the tile holding the first row's earliest visible key.
  const int W = C::WIN ? a.window : 0;
  const int j0 = W > 0 ? max(0, q0 - W + 1) / BN : 0;

  // This lane's query row as B operands: q~ (for S^T) and dO (for dP^T).
  const long hoff = (long)tok0 * qs + (long)head * D;
  const rsrc_t rq = make_rsrc((const uint16_t*)a.qr + hoff, (uint32_t)(((L - 1) * qs + D) * 2));
  const rsrc_t rd = make_rsrc((const uint16_t*)a.dout + hoff, (uint32_t)(((L - 1) * qs + D) * 2));
  u32x4 qf[KSTEPS], df[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const int off = my_q * qs * 2 + (2 * s + hh) * 16;
    qf[s] = buf_load16(rq, off, 0);
    df[s] = buf_load16(rd, off, 0);
  }
  float neg_lse = -INFINITY, neg_d = 0.f;
  if (my_q < L) {
    const float* l = a.ld + (ldt0 + (long)head * ldh + my_q / 32) * 64 + my_q % 32;
    neg_lse = l[0];
    neg_d = l[32];
  }

  const rsrc_t rkr = make_rsrc((const uint16_t*)a.kr + ((long)tok0 * ks + kvh * D), (uint32_t)(((L - 1) * ks + D) * 2));
  const rsrc_t rv = make_rsrc((const uint16_t*)a.v + ((long)tok0 * ks + kvh * D), (uint32_t)(((L - 1) * ks + D) * 2));
  const TileCopy<D, BN, 8> kvcopy(wave, ks * 2, lane);
  auto issue = [&](int j, char* kt, char* vt) {
    if (j >= n_tiles) return;
    kvcopy(rkr, kt, j * BN * ks * 2);
    kvcopy(rv, vt, j * BN * ks * 2);
  };

  const TrOffsets<D> tro(lane);
  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = (f32x16){};

  // MASK: the body with the causal mask (tiles that reach past the unit's
  // first row); the other body is for tiles every row sees whole, so the
  // mask's selects are not executed (predicated) on every tile.
  auto compute = [&](int j, const char* Kt, const char* Vt, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if (!wave_has_rows || (C::CAUSAL && j * BN > wave_last)) return;
    if (W > 0 && j * BN + BN - 1 < qw0 - W + 1) return;  // left of every row's window
    const bool domask = MASK && C::CAUSAL && j * BN + BN - 1 > qw0;
    const bool wmask = W > 0 && j * BN < wave_last - W + 1;
    const int lim = my_q - j * BN - 4 * hh;  // key offset in the tile must be <= lim
    const int lo = my_q - W + 1 - j * BN - 4 * hh;  // ... and >= lo under a window
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      f32x16 sacc = (f32x16){} + neg_lse, dpacc = (f32x16){} + neg_d;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
        sacc = mma32(frag<QK>(row_frag<D>(Kt, 32 * kb + l32, s, hh)), frag<QK>(qf[s]), sacc);
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
        dpacc = mma32(frag<OpBF16>(row_frag<D>(Vt, 32 * kb + l32, s, hh)), frag<OpBF16>(df[s]), dpacc);
      if (domask) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) sacc[r] = -INFINITY;
      }
      if (wmask) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + 8 * (r >> 2) + (r & 3) < lo) sacc[r] = -INFINITY;
      }
      u32x4 sb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int r = 8 * t + 2 * m;
          const float p0 = fast_exp2(sacc[r]), p1 = fast_exp2(sacc[r + 1]);
          sb[t][m] = pack2(QK{}, p0 * dpacc[r], p1 * dpacc[r + 1]);
        }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          dq[db] = mma32(frag<QK>(tr_frag<D>(Kt, 32 * kb + 16 * t, db, tro)), frag<QK>(sb[t]), dq[db]);
    }
  };

  // Tile j0 + 2m uses stage 0, j0 + 2m + 1 stage 1. Tiles below n_plain end
  // before the unit's first row (no causal mask for any wave; windowed units
  // keep the masked body throughout).
  const int n_plain = C::CAUSAL && !C::WIN ? min(n_tiles, (q0 + 1) / BN) : j0;
  issue(j0, kt0s, vt0s);
  wait_vmem();
  __syncthreads();
  int j = j0;
  for (; j + 1 < n_plain; j += 2) {
    issue(j + 1, kt1s, vt1s);
    compute(j, kt0s, vt0s, std::false_type{});
    wait_vmem();
    __syncthreads();
    issue(j + 2, kt0s, vt0s);
    compute(j + 1, kt1s, vt1s, std::false_type{});
    wait_vmem();
    __syncthreads();
  }
  for (; j + 1 < n_tiles; j += 2) {
    issue(j + 1, kt1s, vt1s);
    compute(j, kt0s, vt0s, std::true_type{});
    wait_vmem();
    __syncthreads();
    issue(j + 2, kt0s, vt0s);
    compute(j + 1, kt1s, vt1s, std::true_type{});
    wait_vmem();
    __syncthreads();
  }
  if (j < n_tiles) compute(j, kt0s, vt0s, std::true_type{});

  if (!wave_has_rows) return;
  if (my_q < L) rope_transpose_acc<D, C::STYLE>(dq, a.rope_cos, a.rope_sin, my_q, hh);
  const rsrc_t rdq = make_rsrc((uint16_t*)a.dq + hoff, (uint32_t)(((L - 1) * qs + D) * 2));
  store_acc_bf16<D>(dq, a.scale, rdq, my_q * qs * 2, hh);
}

// Launch the three kernels of one instance (arguments validated by the caller).
// Packed batches: a grid of every 128-key slot (dk, dv) and every 256-row
// slot (dq) of the batch; units of slots that hold no block exit at once.
template <class C>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  constexpr int D = C::D;
  long items, k_units, q_units;
  if (a.cu_seqlens) {
    items = ((long)a.NSL * kBwdTileRows * a.H + (long)a.total * a.KV) * (D / 16);
    k_units = ((long)a.total + C::BK - 1) / C::BK + a.nseq;
    q_units = ((long)a.total + (C::BQ >> a.lhp) - 1) / (C::BQ >> a.lhp) + a.nseq;
  } else {
    items = ((long)a.B * a.NT * kBwdTileRows * a.H + (long)a.B * a.T * a.KV) * (D / 16);
    k_units = (long)(a.T + C::BK - 1) / C::BK * a.B;
    q_units = (long)(a.T + (C::BQ >> a.lhp) - 1) / (C::BQ >> a.lhp) * a.B;
  }
  if (a.cu_seqlens)
    hipLaunchKernelGGL((bwd_prep_varlen_kernel<D, typename C::QK, C::STYLE>),
                       dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_prep_kernel<D, typename C::QK, C::STYLE>), dim3((unsigned)((items + 255) / 256)),
                       dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  long dkdv_grid = k_units * a.KV * a.hsplit, dq_grid = q_units * (a.H >> a.lhp);
  if (!a.cu_seqlens && C::CAUSAL && !C::WIN) {
    // Two workgroups for every claimed unit (claim_unit; the placed grid's
    // own workgroups of those ranks already cover each once).
    const int nK = (a.T + C::BK - 1) / C::BK, nQ = (a.T + (C::BQ >> a.lhp) - 1) / (C::BQ >> a.lhp);
    const long more_k = (long)kfwd_dyn_ranks(nK) * a.B * a.KV, more_q = (long)kfwd_dyn_ranks(nQ) * a.B * (a.H >> a.lhp);
    if (a.hsplit == 1 && dkdv_grid + more_k <= 0x7fffffffL) dkdv_grid += more_k;
    if (dq_grid + more_q <= 0x7fffffffL) dq_grid += more_q;
  }
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel<C>, dim3((unsigned)dkdv_grid), dim3(512), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.hsplit > 1) {
    const long threads = a.part_rows * a.KV * (D / 16);
    hipLaunchKernelGGL((bwd_dkv_reduce_kernel<D, C::STYLE>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attn_bwd_dq_kernel<C>, dim3((unsigned)dq_grid), dim3(512), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_attn_bwd_d(const BwdArgs& a, int qk_bf16, int style, int causal, hipStream_t stream) {
#define CGR_BL(QK, CAU, STY, WIN) return launch_bwd<BwdCfg<D, QK, CAU, STY, WIN>>(a, stream)
#define CGR_BS(QK, CAU, WIN) \
  if (style == STYLE_HALF) { CGR_BL(QK, CAU, STYLE_HALF, WIN); } else { CGR_BL(QK, CAU, STYLE_INTERLEAVED, WIN); }
#define CGR_BM(QK)                                                                               \
  if (causal && a.window > 0) { CGR_BS(QK, true, true) }                                        \
  else if (causal) { CGR_BS(QK, true, false) } else { CGR_BS(QK, false, false) }
  if (qk_bf16) {
    CGR_BM(OpBF16)
  } else {
    CGR_BM(OpF16)
  }
#undef CGR_BM
#undef CGR_BS
#undef CGR_BL
}

}  // namespace cgr
