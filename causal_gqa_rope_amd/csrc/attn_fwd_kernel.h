// Fused causal GQA + RoPE attention forward for gfx950 (internal to libcgr).
//
// What is computed ("Attention from Scratch", section "Attention, the math"):
// for query head h of a sequence, with its K/V head h / (H/KV),
//   O_i = sum_j softmax_j(scale * rope(q_i, i) . rope(k_j, j)) v_j
// over the keys j the mask allows (j <= i when causal), plus the row's
// log-sum-exp. RoPE ("Embeddings & the Residual Stream", "Positional
// information: RoPE") rotates feature pairs of q and k by p * base^(-2i/d).
// The score matrix is produced and consumed tile by tile with an online
// softmax, so it never leaves the chip ("Attention from Scratch", "Coming
// from CUDA: FlashAttention").
//
// Work unit: one (sequence, query head, block of BM = 32 * NW query rows),
// run by a workgroup of NW waves; wave w owns query rows 32w..32w+31. Two
// bodies share the unit decomposition:
//   * UnitFast (bf16 I/O): buffer loads, V straight into LDS, a fixed per-row
//     softmax reference with a rescaling fallback, a one-tile software
//     pipeline (see its own comments).
//   * Unit (f32 I/O): the plain tile loop on f32 matrix cores, described next.
//
// Per unit (Unit):
//   * Q rows are loaded once, rotated in f32 at their positions, multiplied by
//     scale*log2(e) and rounded once to the Q.K^T operand type; they stay in
//     registers as the B operand of S^T = K Q^T.
//   * Key/value tiles of BN rows stream through LDS, double-buffered: while
//     tile j is multiplied, tile j+1 is already loading into registers; K is
//     rotated at the key positions on its way into LDS.
//   * S^T (keys x queries) comes out of 32x32 MFMAs with each lane holding
//     one query column, so the row max / row sum need only one exchange with
//     the partner lane (lane ^ 32) and the probabilities P feed the next
//     product straight from registers: O^T += V^T P^T.
//   * Causal: tiles entirely above the diagonal are never visited; only tiles
//     that straddle the diagonal (or the ragged end of a sequence) evaluate
//     the mask.
//   * Epilogue: O = O^T / l, rounded to the I/O type; lse = ln2 * (m + log2 l).
#pragma once

#include <type_traits>

#include "device_common.h"
#include "varlen_schedule.h"

namespace cgr {

enum { STYLE_INTERLEAVED = 0, STYLE_HALF = 1 };

// Waves each SIMD keeps resident (register budget 512 / this per lane).
#ifndef CGR_WAVES_PER_SIMD
#define CGR_WAVES_PER_SIMD 2
#endif

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* rope_cos;  // [P, D/2]
  const float* rope_sin;
  const int32_t* cu_seqlens;  // packed batches
  const int32_t* seqlens;     // dense batches: valid tokens per entry (right padding), or null
  int32_t* sched;             // packed batches: [0] items, [1] unused, [2] error, then items
  void* krot;                 // with a workspace (16-bit I/O): k rotated once, in the Q.K^T operand type,
                              // as tile images
  int kimg_slots;             // packed batches with k images: image slots per K/V head
  int max_items;              // packed batches: room for work items in `sched`
  int32_t* status_out;        // packed batches: optional second copy of the schedule's error word
  int B, T, H, KV;
  int total_tokens;
  int window;    // > 0 (causal only): keys 0 <= i - j < window; 0: none
  int hp;        // query heads per unit (divides NW and the group): wave w takes
                 // head head0 + w % hp and rows 32 (w / hp) .. of the unit's block
  float qscale;  // softmax_scale * log2(e), folded into Q
};


// The workgroup's LDS: two stages of K and two of V, each its own array, so
// the compiler can tell a direct-to-LDS load into one of them from reads of
// the others and does not wait for the load before those reads. The four
// base pointers are plain values that no lambda captures (a captured copy
// lives in memory, and a run-time choice read back from memory sends the
// accesses through flat pointers): helpers take the stage they touch as an
// argument.
#define CGR_LDS_PARAMS char *ks0, char *ks1, char *vs0, char *vs1, char *qst
__device__ __forceinline__ char* stage_of(int j, char* s0, char* s1) { return (j & 1) ? s1 : s0; }

// Row stride (dwords) of the V tile in LDS: the transposing reads of one
// half-wave touch 4 rows x 64 bytes, which land on disjoint banks when the
// stride is 16 or 48 (mod 64) dwords.
constexpr int v_stride_dwords(int row_dwords) {
  int s = row_dwords;
  while ((s % 64) != 16 && (s % 64) != 48) ++s;
  return s;
}

// NW_: waves per workgroup (0: the default for the head_dim).
template <int D_, typename IO_, typename QK_, bool CAUSAL_, int STYLE_, bool WIN_ = false,
          bool KPRE_ = false, int NW_ = 0>
struct Cfg {
  static constexpr int D = D_;
  using IO = IO_;  // float, or uint16_t holding bf16 bits
  using QK = QK_;  // OpF16 / OpBF16 / OpF32
  static constexpr bool F32 = std::is_same<IO, float>::value;
  using PV = typename std::conditional<F32, OpF32, OpBF16>::type;
  static constexpr bool CAUSAL = CAUSAL_;
  static constexpr int STYLE = STYLE_;
  // Sliding-window instances (causal only) are separate: the others compile
  // without any of the window's code.
  static constexpr bool WIN = WIN_ && CAUSAL_;
  // K already rotated and rounded to the operand type by krot_kernel (a
  // workspace was given): the tiles only copy it into LDS.
  static constexpr bool KPRE = KPRE_ && !std::is_same<IO_, float>::value;

#ifndef CGR_NW
#define CGR_NW 8
#endif
#ifndef CGR_BN
#define CGR_BN 64
#endif
  // head_dim 256 (bf16 I/O): one wave per SIMD, each with the whole register
  // file (its O accumulator alone is 128 registers per lane), four waves per
  // workgroup and 32-key tiles, so K, V and the Q staging fit in LDS.
  static constexpr bool WIDE = D_ == 256;
  static constexpr int NW = WIDE ? 4 : NW_ > 0 ? NW_ : CGR_NW;
  static constexpr int WPS = WIDE ? 1 : CGR_WAVES_PER_SIMD;  // waves per SIMD
  static constexpr int THREADS = 64 * NW;
  static constexpr int BM = 32 * NW;  // query rows per unit
  static constexpr int BN = WIDE ? 32 : CGR_BN;   // keys per tile
  static constexpr int ESZ = F32 ? 4 : 2;
  static constexpr int KSTEPS = D / 16;  // 32x32x16 k-steps over the head dim
  static constexpr int DB = D / 32;      // 32-wide blocks of the head dim
  static constexpr int NKB = BN / 32;    // 32-key blocks per tile

  static constexpr int K_STRIDE = D * ESZ + 16;  // bytes per K row in LDS
  // f32 I/O: padded row-major V. bf16 I/O: unpadded row-major V, 16-byte
  // chunks XOR-swizzled per row (see UnitFast), written by direct
  // global->LDS loads.
  static constexpr int V_STRIDE = F32 ? D * 4 + 16 : 2 * D;
  static constexpr int K_BYTES = BN * K_STRIDE;
  // A tile image of once-rotated keys: BN unpadded rows of 2*D bytes with
  // XOR-swizzled 16-byte chunks (tswz), copied into the K stage as is.
  static constexpr int K_IMG = BN * 2 * D;
  static constexpr int V_BYTES = BN * V_STRIDE;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int SMEM = 2 * STAGE;
  // Direct V loads: 1 KiB (64 lanes x 16 B) per wave instruction.
  static constexpr int V_WAVE_LOADS = (V_BYTES / 1024 + NW - 1) / NW;
  // Per-wave staging of its 32 query rows (bf16 I/O): Q on the way into the
  // matrix-core operand layout, O on the way out; rows padded like K. It is
  // dynamic LDS, which sits after the static K/V stages: those stay within
  // reach of the 16-bit offsets of the LDS instructions.
  static constexpr int Q_STRIDE = 2 * D + 16;
  static constexpr int Q_STAGE_BYTES = F32 ? 0 : NW * 32 * Q_STRIDE;

  // Loader work items. K: (row, 8-element group g < D/16), which carries the
  // group pair (g, g + D/16) so that both RoPE pairings find their partners.
  static constexpr int K_ITEMS = BN * (D / 16);
  static constexpr int KU = (K_ITEMS + THREADS - 1) / THREADS;
  static constexpr int KW = F32 ? 2 : 1;  // 16-byte words per 8-element group
  // V: 16-byte chunks.
  static constexpr int V_CHUNKS = D * ESZ / 16;
  static constexpr int V_ITEMS = BN * V_CHUNKS;
  static constexpr int VU = (V_ITEMS + THREADS - 1) / THREADS;

  static_assert(D == 32 || D == 64 || D == 128 || D == 256, "head_dim");
  static_assert(!(WIDE && F32), "head_dim 256 is built for bf16 I/O only");
};

// Eight consecutive elements from global memory as floats (zeros when !ok).
template <typename IO>
__device__ __forceinline__ void load8_raw(const IO* p, bool ok, u32x4 (&w)[std::is_same<IO, float>::value ? 2 : 1]) {
  constexpr int W = std::is_same<IO, float>::value ? 2 : 1;
#pragma unroll
  for (int i = 0; i < W; ++i) w[i] = ok ? *((const u32x4*)p + i) : (u32x4){0, 0, 0, 0};
}

template <typename IO>
__device__ __forceinline__ void raw_to_f32(const u32x4 (&w)[std::is_same<IO, float>::value ? 2 : 1], float (&x)[8]) {
  if constexpr (std::is_same<IO, float>::value) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = __uint_as_float(w[0][i]);
      x[4 + i] = __uint_as_float(w[1][i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(w[0][i]);
      x[2 * i + 1] = bf16_hi(w[0][i]);
    }
  }
}

// cos/sin for the group pair (g, g + D/16) of a row at table row `cs`/`sn`.
//   interleaved: group g holds pairs 4g..4g+3, group g + D/16 pairs 4g+D/4..+3.
//   half:        element 8g+j pairs with 8g+j+D/2, pair index 8g+j.
template <int D, int STYLE>
__device__ __forceinline__ void load_tab(const float* cs, const float* sn, int g, bool ok,
                                         f32x4 (&c)[2], f32x4 (&s)[2]) {
  const int o0 = STYLE == STYLE_INTERLEAVED ? 4 * g : 8 * g;
  const int o1 = STYLE == STYLE_INTERLEAVED ? 4 * g + D / 4 : 8 * g + 4;
  if (ok) {
    c[0] = *(const f32x4*)(cs + o0);
    c[1] = *(const f32x4*)(cs + o1);
    s[0] = *(const f32x4*)(sn + o0);
    s[1] = *(const f32x4*)(sn + o1);
  } else {
    c[0] = c[1] = s[0] = s[1] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
}

// Rotate the group pair in place: (a, b) -> (a cos - b sin, a sin + b cos).
// Each output is one rounded product and one fused multiply-add, written out
// so that every kernel that rotates keys (per tile, or once up front) rounds
// them identically, whatever contractions the compiler would choose.
__device__ __forceinline__ float rot_a(float a, float b, float c, float s) { return __builtin_fmaf(a, c, -(b * s)); }
__device__ __forceinline__ float rot_b(float a, float b, float c, float s) { return __builtin_fmaf(a, s, b * c); }
template <int STYLE>
__device__ __forceinline__ void rope_pair(float (&x0)[8], float (&x1)[8], const f32x4 (&c)[2],
                                          const f32x4 (&s)[2]) {
  if constexpr (STYLE == STYLE_INTERLEAVED) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float a = x0[2 * m], b = x0[2 * m + 1];
      x0[2 * m] = rot_a(a, b, c[0][m], s[0][m]);
      x0[2 * m + 1] = rot_b(a, b, c[0][m], s[0][m]);
      a = x1[2 * m];
      b = x1[2 * m + 1];
      x1[2 * m] = rot_a(a, b, c[1][m], s[1][m]);
      x1[2 * m + 1] = rot_b(a, b, c[1][m], s[1][m]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float cj = c[j >> 2][j & 3], sj = s[j >> 2][j & 3];
      const float a = x0[j], b = x1[j];
      x0[j] = rot_a(a, b, cj, sj);
      x1[j] = rot_b(a, b, cj, sj);
    }
  }
}

template <class C>
struct TileRegs {
  u32x4 k[C::KU][2][C::KW];
  f32x4 c[C::KU][2], s[C::KU][2];
  u32x4 v[C::VU];
};

template <class C>
struct Unit {
  using IO = typename C::IO;
  static constexpr int D = C::D, BN = C::BN;

  // Issue the global loads of key/value tile `kt0` into registers.
  static __device__ __forceinline__ void load_tile(TileRegs<C>& r, const IO* kp, const IO* vp,
                                                   long ks, int kt0, int L, const float* cosb,
                                                   const float* sinb) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < C::KU; ++u) {
      const int e = tid + u * C::THREADS;
      const int row = e / (D / 16), g = e % (D / 16);
      const bool ok = (e < C::K_ITEMS) && (kt0 + row < L);
      const IO* src = kp + (long)(kt0 + row) * ks;
      load8_raw<IO>(src + 8 * g, ok, r.k[u][0]);
      load8_raw<IO>(src + 8 * g + D / 2, ok, r.k[u][1]);
      const long t = (long)(kt0 + row) * (D / 2);
      load_tab<D, C::STYLE>(cosb + t, sinb + t, g, ok, r.c[u], r.s[u]);
    }
#pragma unroll
    for (int u = 0; u < C::VU; ++u) {
      const int e = tid + u * C::THREADS;
      const int row = e / C::V_CHUNKS, ch = e % C::V_CHUNKS;
      const bool ok = (e < C::V_ITEMS) && (kt0 + row < L);
      r.v[u] = ok ? *(const u32x4*)((const char*)(vp + (long)(kt0 + row) * ks) + 16 * ch)
                  : (u32x4){0, 0, 0, 0};
    }
  }

  // Rotate K, round it to the operand type and write K and V into an LDS stage.
  static __device__ __forceinline__ void store_tile(const TileRegs<C>& r, char* Ks, char* Vs) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < C::KU; ++u) {
      const int e = tid + u * C::THREADS;
      if (e < C::K_ITEMS) {
        const int row = e / (D / 16), g = e % (D / 16);
        float x0[8], x1[8];
        raw_to_f32<IO>(r.k[u][0], x0);
        raw_to_f32<IO>(r.k[u][1], x1);
        rope_pair<C::STYLE>(x0, x1, r.c[u], r.s[u]);
        char* dst = Ks + row * C::K_STRIDE + g * 8 * C::ESZ;
        if constexpr (C::F32) {
          // Rows are 16-byte aligned only: two 16-byte stores per group.
          *(f32x4*)dst = (f32x4){x0[0], x0[1], x0[2], x0[3]};
          *(f32x4*)(dst + 16) = (f32x4){x0[4], x0[5], x0[6], x0[7]};
          *(f32x4*)(dst + (D / 2) * 4) = (f32x4){x1[0], x1[1], x1[2], x1[3]};
          *(f32x4*)(dst + (D / 2) * 4 + 16) = (f32x4){x1[4], x1[5], x1[6], x1[7]};
        } else {
          *(u32x4*)dst = to_frag<typename C::QK>(x0).v;
          *(u32x4*)(dst + D) = to_frag<typename C::QK>(x1).v;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < C::VU; ++u) {
      const int e = tid + u * C::THREADS;
      if (e < C::V_ITEMS) {
        const int row = e / C::V_CHUNKS, ch = e % C::V_CHUNKS;
        *(u32x4*)(Vs + row * C::V_STRIDE + 16 * ch) = r.v[u];
      }
    }
  }

  // A-operand fragment of rotated K: key row `row`, k-step s.
  static __device__ __forceinline__ Frag<typename C::QK> k_frag(const char* Ks, int row, int s,
                                                                int hh) {
    const char* p = Ks + row * C::K_STRIDE + (2 * s + hh) * 8 * C::ESZ;
    Frag<typename C::QK> f;
    if constexpr (C::F32) {
      const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 16);
      f.v = (f32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
      f.v = *(const u32x4*)p;
    }
    return f;
  }

  // A-operand fragment of V^T for output block db, key block kb, k-step t:
  // lane (d = db*32 + lane%32, hh = lane/32) gets V[key][d] for
  // key = kb*32 + 16t + 8*(j/4) + 4*hh + j%4, j = 0..7.
  static __device__ __forceinline__ Frag<typename C::PV> v_frag(const char* Vs, int vbase, int kb,
                                                                int t, int db) {
    Frag<typename C::PV> f;
    if constexpr (C::F32) {
      const int lane = threadIdx.x & 63;
      const int d = db * 32 + (lane & 31), hh = lane >> 5;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = kb * 32 + 16 * t + 8 * (j >> 2) + 4 * hh + (j & 3);
        f.v[j] = *(const float*)(Vs + key * C::V_STRIDE + d * 4);
      }
    } else {
      const char* p = Vs + vbase + (kb * 32 + 16 * t) * C::V_STRIDE + db * 64;
      const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
      const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * C::V_STRIDE));
      const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
      f.v = (u32x4){ua[0], ua[1], ub[0], ub[1]};
    }
    return f;
  }

  // One work unit: query rows qb*bm .. (bm = 32 NW / hp) of a sequence of L
  // tokens starting at token tok0, query heads head0 .. head0 + hp - 1 of one
  // K/V group. lse[] of local row 0 of head h is at lse_b + h * lse_h.
  static __device__ __forceinline__ void run(const AttnArgs& a, int tok0, int L, int qb, int head0,
                                             long lse_b, long lse_h, CGR_LDS_PARAMS) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int hp = a.hp, bm = 32 * C::NW / hp;
    const int head = head0 + wave % hp;
    const long lse_base = lse_b + (long)head * lse_h;
    const int G = a.H / a.KV, kvh = head / G;
    const long qs = (long)a.H * D, ks = (long)a.KV * D;
    const IO* qp = (const IO*)a.q + (long)tok0 * qs + (long)head * D;
    const IO* kp = (const IO*)a.k + (long)tok0 * ks + (long)kvh * D;
    const IO* vp = (const IO*)a.v + (long)tok0 * ks + (long)kvh * D;

    const int q0 = qb * bm;
    const int qw0 = q0 + (wave / hp) * 32;
    const int my_q = qw0 + l32;
    const bool wave_has_rows = qw0 < L;
    const int wave_last = min(qw0 + 31, L - 1);
    const int q_hi = min(q0 + bm, L);
    const int n_tiles = C::CAUSAL ? (q_hi + BN - 1) / BN : (L + BN - 1) / BN;
    // Sliding window: the unit starts at the tile holding its first row's
    // earliest visible key.
    const int W = C::WIN ? a.window : 0;
    const int j0 = W > 0 ? max(0, q0 - W + 1) / BN : 0;

    // ---- Q: rotate at position my_q, fold in scale*log2(e), round once.
    Frag<typename C::QK> qf[C::KSTEPS];
    {
      const bool ok = my_q < L;
      const IO* src = qp + (long)(ok ? my_q : 0) * qs;
      const long t = (long)(ok ? my_q : 0) * (D / 2);
#pragma unroll
      for (int s2 = 0; s2 < D / 32; ++s2) {
        const int g = 2 * s2 + hh;  // k-step s2 holds group g; k-step s2 + D/32 holds g + D/16
        u32x4 w0[C::KW], w1[C::KW];
        load8_raw<IO>(src + 8 * g, ok, w0);
        load8_raw<IO>(src + 8 * g + D / 2, ok, w1);
        f32x4 c[2], s[2];
        load_tab<D, C::STYLE>(a.rope_cos + t, a.rope_sin + t, g, ok, c, s);
        float x0[8], x1[8];
        raw_to_f32<IO>(w0, x0);
        raw_to_f32<IO>(w1, x1);
        rope_pair<C::STYLE>(x0, x1, c, s);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          x0[j] *= a.qscale;
          x1[j] *= a.qscale;
        }
        qf[s2] = to_frag<typename C::QK>(x0);
        qf[s2 + D / 32] = to_frag<typename C::QK>(x1);
      }
    }

    // Lane's base byte offset for the transposing V reads (see v_frag).
    const int gi = lane >> 4, li = lane & 15;
    const int vbase = (4 * hh + (li >> 2)) * C::V_STRIDE + (16 * (gi & 1) + 4 * (li & 3)) * 2;

    float m_run = -INFINITY;  // running row max (log2 units)
    float l_run = 0.f;        // this lane's share of the running row sum
    f32x16 oacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] = (f32x16){};

    TileRegs<C> regs;
    __syncthreads();  // the previous unit of this workgroup is done with LDS
    load_tile(regs, kp, vp, ks, j0 * BN, L, a.rope_cos, a.rope_sin);
    store_tile(regs, stage_of(j0, ks0, ks1), stage_of(j0, vs0, vs1));
    __syncthreads();

    for (int j = j0; j < n_tiles; ++j) {
      const int kt0 = j * BN;
      if (j + 1 < n_tiles) load_tile(regs, kp, vp, ks, kt0 + BN, L, a.rope_cos, a.rope_sin);
      const char* Ks = stage_of(j, ks0, ks1);
      const char* Vs = stage_of(j, vs0, vs1);
      const bool active = wave_has_rows && (!C::CAUSAL || kt0 <= wave_last) &&
                          (W <= 0 || kt0 + BN - 1 >= qw0 - W + 1);
      if (active) {
        // S^T = K Q^T for the BN keys of this tile (log2 units, scale folded in).
        f32x16 sacc[C::NKB];
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) sacc[kb] = (f32x16){};
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb)
            sacc[kb] = mma32(k_frag(Ks, kb * 32 + l32, s, hh), qf[s], sacc[kb]);
        }
        // Mask: only tiles that straddle the diagonal, the sequence end or the
        // window's left edge.
        const bool need_mask = (C::CAUSAL ? (kt0 + BN - 1 > qw0) : (kt0 + BN > L)) ||
                               (W > 0 && kt0 < wave_last - W + 1);
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kt0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
              if ((C::CAUSAL && key > my_q) || key >= L || (W > 0 && key < my_q - W + 1))
                sacc[kb][i] = -INFINITY;
            }
        }
        // Online softmax. Without a window tile 0 holds key 0, which every
        // row may see; with one, a row may see nothing in its first tiles, and
        // then m stays -inf and p = 0 (m_use keeps exp2 away from -inf - -inf).
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        mx = pair_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(sacc[kb][i] - m_use);
            sacc[kb][i] = p;
            rs += p;
          }
        l_run = l_run * alpha + rs;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
        // O^T += V^T P^T
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            float p8[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) p8[jj] = sacc[kb][8 * t + jj];
            const Frag<typename C::PV> pf = to_frag<typename C::PV>(p8);
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
              oacc[db] = mma32(v_frag(Vs, vbase, kb, t, db), pf, oacc[db]);
          }
      }
      if (j + 1 < n_tiles) store_tile(regs, stage_of(j + 1, ks0, ks1), stage_of(j + 1, vs0, vs1));
      __syncthreads();
    }

    // ---- Epilogue.
    const float l_tot = pair_sum(l_run);
    if (my_q < L) {
      const float inv = 1.f / l_tot;
      IO* dst = (IO*)a.o + (long)(tok0 + my_q) * qs + (long)head * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int d = db * 32 + 8 * a4 + 4 * hh;
          const float o0 = oacc[db][4 * a4] * inv, o1 = oacc[db][4 * a4 + 1] * inv;
          const float o2 = oacc[db][4 * a4 + 2] * inv, o3 = oacc[db][4 * a4 + 3] * inv;
          if constexpr (C::F32) {
            *(f32x4*)(dst + d) = (f32x4){o0, o1, o2, o3};
          } else {
            *(u32x2*)(dst + d) = (u32x2){pack2(OpBF16{}, o0, o1), pack2(OpBF16{}, o2, o3)};
          }
        }
      if (a.lse != nullptr && hh == 0) a.lse[lse_base + my_q] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
    }
  }
};

// ---------------------------------------------------------------------------
// bf16 I/O body. Same unit and same arithmetic as Unit, with the work per key
// tile cut down to what the matrix cores cannot do:
//   * All global reads are buffer loads: the per-lane offsets are fixed for
//     the unit and the tile advance is one scalar offset; rows past the end of
//     the sequence fall outside the buffer's range and read as zeros, so
//     ragged tails need no predicates.
//   * V goes from global memory straight into LDS (no registers): each wave
//     load writes 1 KiB, 16 bytes per lane, in lane order. The row-major V
//     tile is stored with its 16-byte chunks XOR-swizzled per row so the
//     transposing reads of one half-wave (4 rows x 64 bytes) hit distinct
//     banks.
//   * The loop body is straight-line code: tiles that need the causal or
//     sequence-end mask run in a second loop, so the accumulators never pass
//     a data-dependent join (which would make the compiler copy them).
//   * Row sums add the bf16-rounded p (the values the P.V product uses) with
//     packed dot products against (1, 1).
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // Raw buffer (stride 0): reads at byte offsets >= bytes return zeros.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ f32x4 buf_load16f(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// 16 bytes per lane into LDS at lds_base + 16 * lane (lds_base wave-uniform).
__device__ __forceinline__ void buf_load16_lds(rsrc_t r, char* lds_base, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, soff, 0, 0);
}
// Wait until this wave's outstanding global/buffer loads (including those
// that write LDS directly) have landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Waits until at most N of this wave's vector-memory operations are
// outstanding (N < 64); later code stays below the wait.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
  __builtin_amdgcn_sched_barrier(0);
}

template <class C>
struct UnitFast {
  static constexpr int D = C::D, BN = C::BN, NW = C::NW, THREADS = C::THREADS;
  static constexpr int KI = C::KU;
  using QK = typename C::QK;

  // XOR swizzle of the 16-byte chunks of V row r (an involution).
  static __device__ __forceinline__ int vswz_mask(int r) {
    if constexpr (D >= 128) return (r & 3) << 2;
    else if constexpr (D == 64) return ((r >> 1) & 1) << 2;
    else return 0;
  }

  static __device__ __forceinline__ void run(const AttnArgs& a, int tok0, int L, int qb, int head0,
                                             long lse_b, long lse_h, long img0, long img_kvs,
                                             CGR_LDS_PARAMS) {
    // `wave` is the same in every lane: keeping it scalar makes every wave-level
    // decision below (active tiles, masking, V blocks) a scalar branch.
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // The unit's waves split over hp query heads of one K/V group x 32-row
    // blocks: each K/V tile in LDS serves all of them.
    const int hp = a.hp, bm = 32 * NW / hp;
    const int head = head0 + wave % hp, wrow = wave / hp;
    const long lse_base = lse_b + (long)head * lse_h;
    const int l32 = lane & 31, hh = lane >> 5;
    const int G = a.H / a.KV, kvh = head / G;
    const int qs = a.H * D, ks = a.KV * D;  // token strides (elements)
    const uint16_t* qbase = (const uint16_t*)a.q + (long)tok0 * qs + (long)head * D;
    const uint16_t* kbase = (const uint16_t*)a.k + (long)tok0 * ks + (long)kvh * D;
    const uint16_t* vbase = (const uint16_t*)a.v + (long)tok0 * ks + (long)kvh * D;
    const rsrc_t rq = make_rsrc(qbase, (uint32_t)(((L - 1) * qs + D) * 2));
    // Once-rotated keys: the sequence's tile images of K_IMG bytes for this
    // K/V head are consecutive, from image img0 + kvh * img_kvs on; one
    // unit's images are one range.
    const rsrc_t rk = C::KPRE
        ? make_rsrc((const char*)a.krot + (img0 + kvh * img_kvs) * C::K_IMG,
                    (uint32_t)(((L + BN - 1) / BN) * C::K_IMG))
        : make_rsrc(kbase, (uint32_t)(((L - 1) * ks + D) * 2));
    const rsrc_t rv = make_rsrc(vbase, (uint32_t)(((L - 1) * ks + D) * 2));
    const rsrc_t rc = make_rsrc(a.rope_cos, (uint32_t)(L * (D / 2) * 4));
    const rsrc_t rs = make_rsrc(a.rope_sin, (uint32_t)(L * (D / 2) * 4));

    const int q0 = qb * bm;
    const int qw0 = q0 + wrow * 32;
    const int my_q = qw0 + l32;
    const bool wave_has_rows = qw0 < L;
    const int wave_last = min(qw0 + 31, L - 1);
    const int q_hi = min(q0 + bm, L);
    const int n_tiles = C::CAUSAL ? (q_hi + BN - 1) / BN : (L + BN - 1) / BN;
    // Sliding window: such units run the rescaling loop below (the fast
    // path's reference comes from tile 0, which a window may hide), from the
    // tile holding their first row's earliest visible key.
    const int W = C::WIN ? a.window : 0;
    const int j0 = W > 0 ? max(0, q0 - W + 1) / BN : 0;

    // ---- Q. A lane of the matrix-core operand holds one query row, so loading
    // Q (and its cos/sin rows) straight into that layout would touch 32 rows
    // per wave instruction. Instead each wave loads its 32 rows with whole
    // rows per instruction, rotates them at their positions in that layout
    // (scale*log2(e) folded in, one rounding to the operand type), writes them
    // to its own LDS staging area and reads them back as operand fragments.
    // The loads are issued here; the rest (stage_q) runs once the first K
    // tiles' loads are in flight too.
    constexpr int QCH = D / 8;  // 16-byte chunks (8 elements) per row
    constexpr bool Q_HALF = C::STYLE == STYLE_HALF;
    // An item is one chunk (interleaved pairs sit inside it) or, for the half
    // pairing, a chunk and its partner chunk D/2 further on.
    constexpr int QI_PER_ROW = Q_HALF ? QCH / 2 : QCH;
    constexpr int QI = 32 * QI_PER_ROW / 64;  // items per lane
    static_assert(32 * QI_PER_ROW % 64 == 0, "whole items per lane");
    char* const q_stage = qst + wave * 32 * C::Q_STRIDE;
    u32x4 q_raw[QI][Q_HALF ? 2 : 1];
    f32x4 q_cos[QI][Q_HALF ? 2 : 1], q_sin[QI][Q_HALF ? 2 : 1];
    // The prologue's loads go out in this order: the first K and V tiles,
    // then the Q rows and their cos/sin rows (issue_q), so the tiles, read
    // from L2, are in flight while the Q rows come from HBM.
    auto issue_q = [&]() {
#pragma unroll
      for (int i = 0; i < QI; ++i) {
        const int flat = i * 64 + lane, r = flat / QI_PER_ROW, c = flat % QI_PER_ROW;
        const int row = qw0 + r;  // rows past the sequence read as zeros (buffer range)
        const int qo = row * qs * 2 + c * 16, to = row * (D / 2) * 4;
        q_raw[i][0] = buf_load16(rq, qo, 0);
        if constexpr (Q_HALF) {
          q_raw[i][1] = buf_load16(rq, qo + D, 0);
          q_cos[i][0] = buf_load16f(rc, to + c * 32, 0);
          q_cos[i][1] = buf_load16f(rc, to + c * 32 + 16, 0);
          q_sin[i][0] = buf_load16f(rs, to + c * 32, 0);
          q_sin[i][1] = buf_load16f(rs, to + c * 32 + 16, 0);
        } else {
          q_cos[i][0] = buf_load16f(rc, to + c * 16, 0);
          q_sin[i][0] = buf_load16f(rs, to + c * 16, 0);
        }
      }
    };
    Frag<QK> qf[C::KSTEPS];
    // f16 operands: a rotated query (times scale*log2(e)) or key outside the
    // f16 range enters the product as NaN (to_frag_or_nan, here and in the key
    // rotation), so every row that meets it ends with a NaN row sum and the
    // unit is redone by wide_pass.
    constexpr bool F16OP = std::is_same<QK, OpF16>::value;
    // Q fragments straight from global memory (the windowed path): each lane
    // loads its own row's groups, k-step s2 holding group g = 2 s2 + hh and
    // k-step s2 + D/32 group g + D/16.
    auto load_q_direct = [&]() {
      const bool ok = my_q < L;
      const long tq = (long)(ok ? my_q : 0);
#pragma unroll
      for (int s2 = 0; s2 < D / 32; ++s2) {
        const int g = 2 * s2 + hh;
        u32x4 w0[1], w1[1];
        load8_raw<uint16_t>(qbase + tq * qs + 8 * g, ok, w0);
        load8_raw<uint16_t>(qbase + tq * qs + 8 * g + D / 2, ok, w1);
        f32x4 c[2], s[2];
        load_tab<D, C::STYLE>(a.rope_cos + tq * (D / 2), a.rope_sin + tq * (D / 2), g, ok, c, s);
        float x0[8], x1[8];
        raw_to_f32<uint16_t>(w0, x0);
        raw_to_f32<uint16_t>(w1, x1);
        rope_pair<C::STYLE>(x0, x1, c, s);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          x0[j] *= a.qscale;
          x1[j] *= a.qscale;
        }
        qf[s2] = to_frag_or_nan<QK>(x0);
        qf[s2 + D / 32] = to_frag_or_nan<QK>(x1);
      }
    };
    auto stage_q = [&]() {
#pragma unroll
      for (int i = 0; i < QI; ++i) {
        const int flat = i * 64 + lane, r = flat / QI_PER_ROW, c = flat % QI_PER_ROW;
        char* dst = q_stage + r * C::Q_STRIDE + c * 16;
        float x0[8], x1[8];
        const u32x4 w0[1] = {q_raw[i][0]};
        raw_to_f32<uint16_t>(w0, x0);
        if constexpr (Q_HALF) {
          const u32x4 w1[1] = {q_raw[i][1]};
          raw_to_f32<uint16_t>(w1, x1);
          rope_pair<STYLE_HALF>(x0, x1, q_cos[i], q_sin[i]);
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            // Explicit FMAs (as for K): the bits must not depend on how the
            // compiler contracts the products in a given instance.
            const float x = x0[2 * m], y = x0[2 * m + 1];
            x0[2 * m] = rot_a(x, y, q_cos[i][0][m], q_sin[i][0][m]);
            x0[2 * m + 1] = rot_b(x, y, q_cos[i][0][m], q_sin[i][0][m]);
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) x0[j] *= a.qscale;
        *(u32x4*)dst = to_frag_or_nan<QK>(x0).v;
        if constexpr (Q_HALF) {
#pragma unroll
          for (int j = 0; j < 8; ++j) x1[j] *= a.qscale;
          *(u32x4*)(dst + D) = to_frag_or_nan<QK>(x1).v;
        }
      }
      // Operand fragments: k-step s of lane (l32, hh) holds elements 16s+8hh..+7
      // of row l32, the same split as the K fragments.
#pragma unroll
      for (int s2 = 0; s2 < C::KSTEPS; ++s2)
        qf[s2].v = *(const u32x4*)(q_stage + l32 * C::Q_STRIDE + 32 * s2 + 16 * hh);
    };

    // ---- Per-lane load offsets. K item u of this thread is (row0 + u*RPU,
    // group g0): the lane part is fixed, the item and tile parts are uniform
    // (scalar offsets) or compile-time (instruction immediates).
    constexpr int RPU = THREADS / (D / 16);  // K rows between a thread's items
    const int row0 = tid / (D / 16), g0 = tid % (D / 16);
    // Does this thread own K item u? Compile-time yes when the items divide evenly.
    auto has_k = [&](int u) {
      if constexpr (C::K_ITEMS % THREADS == 0) return true;
      else return row0 + u * RPU < BN;
    };
    const int k_vo = (row0 * ks + 8 * g0) * 2;
    constexpr int TAB_O1 = C::STYLE == STYLE_INTERLEAVED ? D : 16;  // bytes from o0 to o1
    const int t_vo = (row0 * (D / 2) + (C::STYLE == STYLE_INTERLEAVED ? 4 * g0 : 8 * g0)) * 4;
    const int k_lds = row0 * C::K_STRIDE + g0 * 16;
    // V: 1 KiB per wave load = VROWS rows. The swizzle follows the row within
    // the tile, blk * VROWS + v_r, and repeats every 4 rows: with 4 or more
    // rows per load the lane's chunk does not depend on the block; with 2
    // (head_dim 256) it depends on the block's parity.
    constexpr int VWL = C::V_WAVE_LOADS;
    constexpr int VROWS = 1024 / (2 * D);
    const int v_r = lane / (2 * D / 16), v_pch = lane % (2 * D / 16);
    const int v_vo = v_r * ks * 2 + 16 * (v_pch ^ vswz_mask(v_r));
    const int v_vo_odd = VROWS >= 4 ? v_vo : v_r * ks * 2 + 16 * (v_pch ^ vswz_mask(VROWS + v_r));

    // K (to registers) and V (straight to LDS) of the tile at kt0; the K
    // registers are consumed by store_k once this tile's products are issued.
    constexpr int VU_REG = 1;  // (V never passes through registers)
    auto load_v = [&](int kt0, char* vs, u32x4 (&vw)[VU_REG]) {
#pragma unroll
      for (int u = 0; u < VWL; ++u) {
        const int blk = wave * VWL + u;
        if (C::V_BYTES == NW * VWL * 1024 || blk * 1024 < C::V_BYTES)
          buf_load16_lds(rv, vs + blk * 1024, (blk & 1) ? v_vo_odd : v_vo, (kt0 + blk * VROWS) * ks * 2);
      }
    };
    // K of the tile at kt0: rotated in registers (store_k writes it to LDS
    // later), or, once-rotated, its tile image straight into LDS at kdst.
    auto load_k = [&](int kt0, char* kdst, u32x4 (&kw)[KI][2], f32x4 (&kc)[KI][2], f32x4 (&ksn)[KI][2]) {
      if constexpr (C::KPRE) {
        constexpr int NBLK = C::K_IMG / 1024;
        static_assert(C::K_IMG % 1024 == 0, "whole 1-KiB loads");
        const int soff = (kt0 / BN) * C::K_IMG;
#pragma unroll
        for (int u = 0; u < (NBLK + NW - 1) / NW; ++u) {
          const int blk = wave + u * NW;
          if (NBLK % NW == 0 || blk < NBLK) buf_load16_lds(rk, kdst + blk * 1024, lane * 16, soff + blk * 1024);
        }
        return;
      }
#pragma unroll
      for (int u = 0; u < KI; ++u) {
        if (has_k(u)) {
          const int so = (kt0 + u * RPU) * ks * 2;
          kw[u][0] = buf_load16(rk, k_vo, so);
          kw[u][1] = buf_load16(rk, k_vo + D, so);
          if constexpr (!C::KPRE) {
            const int st = (kt0 + u * RPU) * (D / 2) * 4;
            kc[u][0] = buf_load16f(rc, t_vo, st);
            kc[u][1] = buf_load16f(rc, t_vo + TAB_O1, st);
            ksn[u][0] = buf_load16f(rs, t_vo, st);
            ksn[u][1] = buf_load16f(rs, t_vo + TAB_O1, st);
          }
        }
      }
    };
    auto issue_loads = [&](int kt0, char* ks_, char* vs, u32x4 (&kw)[KI][2], f32x4 (&kc)[KI][2],
                           f32x4 (&ksn)[KI][2], u32x4 (&vw)[VU_REG]) {
      load_v(kt0, vs, vw);
      load_k(kt0, ks_, kw, kc, ksn);
    };
    // Rotate K at the key positions and write it to LDS.
    auto store_k = [&](int kt0, char* kst, const u32x4 (&kw)[KI][2], f32x4 (&kc)[KI][2],
                       f32x4 (&ksn)[KI][2], const u32x4 (&vw)[VU_REG]) {
#pragma unroll
      for (int u = 0; u < KI; ++u) {
        if (has_k(u)) {
          char* dst = kst + k_lds + u * RPU * C::K_STRIDE;
          if constexpr (C::KPRE) {
            // loaded straight into LDS by load_k
          } else {
            float x0[8], x1[8];
            const u32x4 w0[1] = {kw[u][0]}, w1[1] = {kw[u][1]};
            raw_to_f32<uint16_t>(w0, x0);
            raw_to_f32<uint16_t>(w1, x1);
            rope_pair<C::STYLE>(x0, x1, kc[u], ksn[u]);
            *(u32x4*)dst = to_frag_or_nan<QK>(x0).v;
            *(u32x4*)(dst + D) = to_frag_or_nan<QK>(x1).v;
          }
        }
      }
    };

    // Lane offsets of the K fragment reads and of the transposing V reads.
    const int k_rd = l32 * C::K_STRIDE + hh * 16;
    // Swizzled images: chunk 2s + hh of row kb*32 + l32 (the swizzle repeats
    // every 16 rows, so it depends on l32 only).
    int k_rds[C::KPRE ? C::KSTEPS : 1];
    if constexpr (C::KPRE) {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) k_rds[s] = l32 * 2 * D + 16 * ((2 * s + hh) ^ tswz<D>(l32));
    }
    const int gi = lane >> 4, li = lane & 15;
    const int vx = D >= 128 ? (li >> 2) : (D == 64 ? (((4 * hh + (li >> 2)) >> 1) & 1) : 0);
    const int v_lane = (4 * hh + (li >> 2)) * (2 * D) + 16 * (2 * (gi & 1) + ((li & 3) >> 1)) +
                       8 * (li & 1);
    int v_rd[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) v_rd[db] = v_lane + 64 * (db ^ vx);

    const uint32_t ones_bf16 = 0x3f803f80u;
    f32x16 oacc[C::DB];
    float l_run = 0.f;  // this lane's share of the row sum
    u32x4 kw[KI][2];
    f32x4 kc[KI][2], ksn[KI][2];
    u32x4 vw[VU_REG];

    // Stage tile j (K rotated, V) in LDS.
    auto start = [&](int j, char* kst, char* vst) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] = (f32x16){};
      l_run = 0.f;
      __syncthreads();  // earlier users of this workgroup's LDS are done
      issue_loads(j * BN, kst, vst, kw, kc, ksn, vw);
      store_k(j * BN, kst, kw, kc, ksn, vw);
      wait_vmem();
      __syncthreads();
    };
    // Start loading tile j+1 (every wave, every tile).
    auto prefetch = [&](int j, char* knext, char* vnext) {
      if (j + 1 < n_tiles) issue_loads((j + 1) * BN, knext, vnext, kw, kc, ksn, vw);
    };
    // S^T = K Q^T + cinit (log2 units, scale folded in).
    auto scores = [&](const char* Ks, f32x16 (&sacc)[C::NKB], const f32x16& cinit) {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s)
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
          Frag<QK> kf;
          if constexpr (C::KPRE)
            kf.v = *(const u32x4*)(Ks + k_rds[s] + kb * 32 * 2 * D);
          else
            kf.v = *(const u32x4*)(Ks + k_rd + kb * 32 * C::K_STRIDE + 32 * s);
          sacc[kb] = mma32(kf, qf[s], s == 0 ? cinit : sacc[kb]);
        }
    };
    // Keys past this lane's row (causal) or past the sequence end get -inf.
    // Key of accumulator (kb, i): kt0 + kb*32 + 8*(i/4) + 4*hh + i%4.
    auto mask = [&](int j, f32x16 (&sacc)[C::NKB]) {
      const int lim = (C::CAUSAL ? min(my_q, L - 1) : L - 1) - j * BN - 4 * hh;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 8 * (i >> 2) + (i & 3) > lim) sacc[kb][i] = -INFINITY;
    };
    // The window's left edge as well: keys before my_q - W + 1 get -inf too.
    auto mask_window = [&](int j, f32x16 (&sacc)[C::NKB]) {
      const int lim = min(my_q, L - 1) - j * BN - 4 * hh;
      const int lo = my_q - W + 1 - j * BN - 4 * hh;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = kb * 32 + 8 * (i >> 2) + (i & 3);
          if (off > lim || off < lo) sacc[kb][i] = -INFINITY;
        }
    };
    auto rowmax = [&](const f32x16 (&sacc)[C::NKB]) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      return pair_max(mx);
    };
    // P = 2^(s - shift), rounded to bf16 for the P.V product (the row sum adds
    // the rounded values, by packed dot products with (1, 1)); then
    // O^T = alpha O^T + V^T P^T. SHIFT/SCALE select the optional terms.
    auto probs = [&](const f32x16 (&sacc)[C::NKB], auto shift_tag, float shift,
                     u32x4 (&pf)[C::NKB][2]) {
      constexpr bool SHIFT = decltype(shift_tag)::value;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float s0 = sacc[kb][8 * t + 2 * q], s1 = sacc[kb][8 * t + 2 * q + 1];
            if constexpr (SHIFT) {
              s0 -= shift;
              s1 -= shift;
            }
            const uint32_t pk = pack2(OpBF16{}, fast_exp2(s0), fast_exp2(s1));
            pf[kb][t][q] = pk;
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                                    __builtin_bit_cast(bf16x2, ones_bf16), l_run,
                                                    false);
          }
    };
    auto pv = [&](const char* Vs, const u32x4 (&pf)[C::NKB][2], auto scale_tag, float alpha) {
      constexpr bool SCALE = decltype(scale_tag)::value;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          Frag<OpBF16> pfr;
          pfr.v = pf[kb][t];
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const char* p = Vs + v_rd[db] + (kb * 32 + 16 * t) * (2 * D);
            const s16x4 ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
            const s16x4 rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * 2 * D));
            const u32x2 ua = __builtin_bit_cast(u32x2, ra), ub = __builtin_bit_cast(u32x2, rb);
            Frag<OpBF16> vf;
            vf.v = (u32x4){ua[0], ua[1], ub[0], ub[1]};
            if constexpr (SCALE)
              oacc[db] = mma32(vf, pfr, (kb == 0 && t == 0) ? oacc[db] * alpha : oacc[db]);
            else
              oacc[db] = mma32(vf, pfr, oacc[db]);
          }
        }
    };
    auto softmax_pv = [&](const char* Vs, const f32x16 (&sacc)[C::NKB], auto shift_tag,
                          float shift, auto scale_tag, float alpha) {
      u32x4 pf[C::NKB][2];
      probs(sacc, shift_tag, shift, pf);
      pv(Vs, pf, scale_tag, alpha);
    };
    // Rotate and store K of tile j+1, wait for its V, then barrier.
    auto finish = [&](int j, char* knext) {
      if (j + 1 < n_tiles) store_k((j + 1) * BN, knext, kw, kc, ksn, vw);
      wait_vmem();
      __syncthreads();
    };
    // Tiles below n_plain need no mask for any wave of the unit: every key of
    // the tile precedes the unit's first row (causal) and lies inside the
    // sequence. Tile 0 holds key 0, which every row may see.
    const int n_plain = C::CAUSAL ? min(n_tiles, (q0 + 1) / BN) : L / BN;

    // ---- Fast path. Each row's reference m is its exact max over tile 0;
    // the S^T accumulator of later tiles starts from -m, so the matrix cores
    // return s - m and p = 2^(s - m) needs no further arithmetic. p may exceed
    // 1 when later keys score higher; the result is as exact as with the
    // running max as long as nothing overflows: bf16 p has f32's exponent
    // range, and p is only ever larger than with the running max (no extra
    // underflow). The checks after the pass (a row sum not below 2^126, which
    // bounds every p, or an O accumulator that is not finite) send the unit to
    // the rescaling path.
    //
    // Software-pipelined by one tile: iteration j computes S of tile j+1 on
    // the matrix cores while the vector units turn S of tile j into P, then
    // O += V_j P_j while tile j+2's K is rotated. LDS holds K one tile ahead
    // of V: at the top of iteration j, stage (j+1)&1 has K_{j+1} and stage
    // j&1 has V_j; the loads of iteration j fill V_{j+1} and, through
    // registers, K_{j+2}.
    // ---- Rescaling path (classic online softmax: m' = max(m, tile max), O
    // and l scaled by 2^(m - m') every tile): every windowed unit, and units
    // whose scores grow too far beyond the first tile (the whole workgroup
    // then redoes the unit). Returns the final row max. WIN selects the
    // window's tile range and mask at compile time, so the fallback of the
    // unwindowed path carries none of that code.
    auto rescale_pass = [&](auto win_tag) -> float {
      constexpr bool WIN = decltype(win_tag)::value;
      const int jb = WIN ? j0 : 0;
      float m_run = -INFINITY;
      start(jb, stage_of(jb, ks0, ks1), stage_of(jb, vs0, vs1));
      for (int j = jb; j < n_tiles; ++j) {
        prefetch(j, stage_of(j + 1, ks0, ks1), stage_of(j + 1, vs0, vs1));
        if (wave_has_rows && (!C::CAUSAL || j * BN <= wave_last) &&
            (!WIN || j * BN + BN - 1 >= qw0 - W + 1)) {
          f32x16 sacc[C::NKB];
          scores(stage_of(j, ks0, ks1), sacc, (f32x16){});
          if constexpr (WIN)
            mask_window(j, sacc);
          else
            mask(j, sacc);
          // A row may see no key of its first tiles under a window: m stays
          // -inf and p = 0 (m_use keeps exp2 away from -inf - -inf).
          const float m_new = fmaxf(m_run, rowmax(sacc));
          const float m_use = m_new == -INFINITY ? 0.f : m_new;
          const float alpha = fast_exp2(m_run - m_use);
          m_run = m_new;
          l_run *= alpha;
          softmax_pv(stage_of(j, vs0, vs1), sacc, std::true_type{}, m_use, std::true_type{}, alpha);
        }
        finish(j, stage_of(j + 1, ks0, ks1));
      }
      return m_run;
    };
    // ---- Wide-range pass: units whose rotated queries or keys leave the range
    // of the f16 operand (a NaN row sum: see to_frag_or_nan). The classic online softmax over the unit's
    // tiles, one LDS stage, with every operand carried as a bf16 hi + lo pair:
    // S = K_hi Q_hi + K_hi Q_lo + K_lo Q_hi (16 significant bits, f32's range;
    // K_lo Q_lo is below the f32 accumulation's rounding). Queries and keys are
    // rotated again from the raw inputs, so nothing out of range is reused.
    auto wide_pass = [&](auto win_tag) -> float {
      constexpr bool WIN = decltype(win_tag)::value;
      const int jb = WIN ? j0 : 0;
      Frag<OpBF16> qh[C::KSTEPS], ql[C::KSTEPS];
      {
        const bool ok = my_q < L;
        const long tq = (long)(ok ? my_q : 0);
#pragma unroll
        for (int s2 = 0; s2 < D / 32; ++s2) {
          const int g = 2 * s2 + hh;
          u32x4 w0[1], w1[1];
          load8_raw<uint16_t>(qbase + tq * qs + 8 * g, ok, w0);
          load8_raw<uint16_t>(qbase + tq * qs + 8 * g + D / 2, ok, w1);
          f32x4 c[2], s[2];
          load_tab<D, C::STYLE>(a.rope_cos + tq * (D / 2), a.rope_sin + tq * (D / 2), g, ok, c, s);
          float x0[8], x1[8];
          raw_to_f32<uint16_t>(w0, x0);
          raw_to_f32<uint16_t>(w1, x1);
          rope_pair<C::STYLE>(x0, x1, c, s);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            x0[j] *= a.qscale;
            x1[j] *= a.qscale;
          }
          split_bf16(x0, qh[s2], ql[s2]);
          split_bf16(x1, qh[s2 + D / 32], ql[s2 + D / 32]);
        }
      }
      const rsrc_t rkr = make_rsrc(kbase, (uint32_t)(((L - 1) * ks + D) * 2));
      float m_run = -INFINITY;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] = (f32x16){};
      l_run = 0.f;
      for (int j = jb; j < n_tiles; ++j) {
        __syncthreads();  // the stages' earlier readers are done
        load_v(j * BN, vs0, vw);
        // Raw K of tile j at its positions, split into hi (stage ks0) and lo
        // (stage ks1), padded rows as in the per-tile rotation.
#pragma unroll
        for (int u = 0; u < KI; ++u) {
          if (has_k(u)) {
            const int so = (j * BN + u * RPU) * ks * 2, st = (j * BN + u * RPU) * (D / 2) * 4;
            const u32x4 w0[1] = {buf_load16(rkr, k_vo, so)}, w1[1] = {buf_load16(rkr, k_vo + D, so)};
            const f32x4 c[2] = {buf_load16f(rc, t_vo, st), buf_load16f(rc, t_vo + TAB_O1, st)};
            const f32x4 sn[2] = {buf_load16f(rs, t_vo, st), buf_load16f(rs, t_vo + TAB_O1, st)};
            float x0[8], x1[8];
            raw_to_f32<uint16_t>(w0, x0);
            raw_to_f32<uint16_t>(w1, x1);
            rope_pair<C::STYLE>(x0, x1, c, sn);
            Frag<OpBF16> h0, l0, h1, l1;
            split_bf16(x0, h0, l0);
            split_bf16(x1, h1, l1);
            const int o = k_lds + u * RPU * C::K_STRIDE;
            *(u32x4*)(ks0 + o) = h0.v;
            *(u32x4*)(ks0 + o + D) = h1.v;
            *(u32x4*)(ks1 + o) = l0.v;
            *(u32x4*)(ks1 + o + D) = l1.v;
          }
        }
        wait_vmem();
        __syncthreads();
        if (wave_has_rows && (!C::CAUSAL || j * BN <= wave_last) &&
            (!WIN || j * BN + BN - 1 >= qw0 - W + 1)) {
          f32x16 sacc[C::NKB];
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb) sacc[kb] = (f32x16){};
#pragma unroll
          for (int s = 0; s < C::KSTEPS; ++s)
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
              Frag<OpBF16> kh, kl;
              kh.v = *(const u32x4*)(ks0 + k_rd + kb * 32 * C::K_STRIDE + 32 * s);
              kl.v = *(const u32x4*)(ks1 + k_rd + kb * 32 * C::K_STRIDE + 32 * s);
              sacc[kb] = mma32(kh, qh[s], sacc[kb]);
              sacc[kb] = mma32(kh, ql[s], sacc[kb]);
              sacc[kb] = mma32(kl, qh[s], sacc[kb]);
            }
          if constexpr (WIN)
            mask_window(j, sacc);
          else
            mask(j, sacc);
          const float m_new = fmaxf(m_run, rowmax(sacc));
          const float m_use = m_new == -INFINITY ? 0.f : m_new;
          const float alpha = fast_exp2(m_run - m_use);
          m_run = m_new;
          l_run *= alpha;
          softmax_pv(vs0, sacc, std::true_type{}, m_use, std::true_type{}, alpha);
        }
      }
      return m_run;
    };
    // After a fast pass: a unit out of the f16 range goes to wide_pass, one
    // whose row sums outgrew the fixed reference to rescale_pass (one barrier
    // when neither happened).
    auto finish_unit = [&](float m_ref, auto win_tag) -> float {
      const float l_chk = pair_sum(l_run);
      float o_chk = 0.f;  // inf or NaN if any accumulator is (or the sum overflows)
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o_chk += oacc[db][e];
      const bool overflow = !(l_chk < 0x1p126f) || !(fabsf(o_chk) <= 3.4028234663852886e38f);  // NaN-safe
      if (!__syncthreads_or(overflow)) return m_ref;
      if constexpr (F16OP) {
        if (__syncthreads_or(l_chk != l_chk)) return wide_pass(win_tag);
      }
      return rescale_pass(win_tag);
    };
    float m_fin;
    if (W > 0 && bm > BN) {
      // Q fragments straight from global memory, each lane its own row.
      load_q_direct();
      m_fin = rescale_pass(std::true_type{});
      if constexpr (F16OP) {
        const float l_chk = pair_sum(l_run);
        if (__syncthreads_or(l_chk != l_chk)) m_fin = wide_pass(std::true_type{});
      }
    } else if (W > 0) {
      // ---- Windowed fast path (units of at most one tile of rows, so every
      // row's own key lies in the unit's last tile jl). That tile goes first
      // and gives each row its reference m, the row's max over it; then the
      // window's tiles jb .. jl-1 in order, with S starting from -m. Tiles
      // below jl hold no key past any row (no causal mask); those starting
      // before the last row's window need the window's left edge.
      // Processing order i = 0, 1, ..: tile tl(i), LDS stages by i's parity.
      const int jl = n_tiles - 1, n_it = jl - j0 + 1;
      auto tl = [&](int i) { return i == 0 ? jl : j0 + i - 1; };
      auto wactive = [&](int tile) {
        return wave_has_rows && tile * BN <= wave_last && tile * BN + BN - 1 >= qw0 - W + 1;
      };
      const int lo_all = q_hi - 1 - W + 1;  // tiles starting at or after this need no edge mask
      float m_ref = 0.f;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) oacc[db] = (f32x16){};
      l_run = 0.f;
      u32x4 kw1[KI][2];
      f32x4 kc1[KI][2], ksn1[KI][2];
      // (Each workgroup runs one unit: its LDS has no earlier users to wait for.)
      load_k(jl * BN, ks0, kw, kc, ksn);
      load_v(jl * BN, vs0, vw);
      if (n_it > 1) load_k(tl(1) * BN, ks1, kw1, kc1, ksn1);
      issue_q();
      stage_q();
      store_k(jl * BN, ks0, kw, kc, ksn, vw);
      wait_vmem();
      __syncthreads();
      f32x16 s_cur[C::NKB];
      if (wave_has_rows) {
        scores(ks0, s_cur, (f32x16){});
        mask_window(jl, s_cur);
        m_ref = rowmax(s_cur);
        // Only lanes past the sequence end can see no key here; 0 keeps their
        // arithmetic finite (their rows are never stored).
        if (m_ref == -INFINITY) m_ref = 0.f;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) s_cur[kb] -= m_ref;
      }
      if (n_it > 1) store_k(tl(1) * BN, ks1, kw1, kc1, ksn1, vw);
      wait_vmem();
      __syncthreads();
      const f32x16 negm = (f32x16){} - m_ref;
      auto witer = [&](int i) {
        char* ki = stage_of(i, ks0, ks1);
        char* ki1 = stage_of(i + 1, ks0, ks1);
        char* vi = stage_of(i, vs0, vs1);
        char* vi1 = stage_of(i + 1, vs0, vs1);
        const int tc = tl(i);
        if (i + 1 < n_it) load_v(tl(i + 1) * BN, vi1, vw);
        if (i + 2 < n_it) load_k(tl(i + 2) * BN, ki, kw, kc, ksn);
        f32x16 s_next[C::NKB];
        if (i + 1 < n_it && wactive(tl(i + 1))) scores(ki1, s_next, negm);
        if (wactive(tc)) {
          if (i > 0 && tc * BN < lo_all) mask_window(tc, s_cur);
          softmax_pv(vi, s_cur, std::false_type{}, 0.f, std::false_type{}, 1.f);
        }
        if (i + 2 < n_it) store_k(tl(i + 2) * BN, ki, kw, kc, ksn, vw);
        wait_vmem();
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) s_cur[kb] = s_next[kb];
      };
      // Steady run: iterations whose tile needs no mask for any row and whose
      // two successors are window tiles too (consecutive keys), unrolled by
      // two with the stages fixed at compile time as in the causal path.
      f32x16 s_alt[C::NKB];
      auto wsteady = [&](int i, f32x16 (&s_in)[C::NKB], f32x16 (&s_out)[C::NKB], char* ki, char* ki1, char* vi,
                         char* vi1) {
        const int tc = tl(i);
        load_v((tc + 1) * BN, vi1, vw);
        load_k((tc + 2) * BN, ki, kw, kc, ksn);
        __builtin_amdgcn_sched_barrier(0);
        scores(ki1, s_out, negm);
        softmax_pv(vi, s_in, std::false_type{}, 0.f, std::false_type{}, 1.f);
        store_k((tc + 2) * BN, ki, kw, kc, ksn, vw);
        wait_vmem();
        __syncthreads();
      };
      // First steady iteration: tile tl(i) >= lo_all (i >= 1), rounded up to
      // an odd i so that the stage of iteration i is stage 1 (i odd).
      int i = 0;
      const int i_first = max(1, (max(lo_all, 0) + BN - 1) / BN - j0 + 1);
      for (; i < n_it && (i < i_first || (i & 1) == 0); ++i) witer(i);
      if (wave_has_rows) {
        for (; i + 3 < n_it; i += 2) {
          wsteady(i, s_cur, s_alt, ks1, ks0, vs1, vs0);
          wsteady(i + 1, s_alt, s_cur, ks0, ks1, vs0, vs1);
        }
      }
      for (; i < n_it; ++i) witer(i);
      m_fin = finish_unit(m_ref, std::true_type{});
    } else {
      float m_ref = 0.f;
      {
        auto active = [&](int t) { return wave_has_rows && (!C::CAUSAL || t * BN <= wave_last); };
        // Stage K_0, V_0 and K_1, with the loads of Q, K_0 and K_1 all in
        // flight before the first wait.
  #pragma unroll
        for (int db = 0; db < C::DB; ++db) oacc[db] = (f32x16){};
        l_run = 0.f;
        u32x4 kw1[KI][2];
        f32x4 kc1[KI][2], ksn1[KI][2];
        // (Each workgroup runs one unit: its LDS has no earlier users to wait for.)
        load_k(0, ks0, kw, kc, ksn);
        load_v(0, vs0, vw);
        if (n_tiles > 1) load_k(BN, ks1, kw1, kc1, ksn1);
        issue_q();
        stage_q();
        store_k(0, ks0, kw, kc, ksn, vw);
        wait_vmem();
        __syncthreads();
        // S_0 and the reference; K_1 into LDS.
        f32x16 s_cur[C::NKB];
        if (wave_has_rows) {
          scores(ks0, s_cur, (f32x16){});
          mask(0, s_cur);
          m_ref = rowmax(s_cur);
  #pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb) s_cur[kb] -= m_ref;
        }
        if (n_tiles > 1) store_k(BN, ks1, kw1, kc1, ksn1, vw);
        wait_vmem();
        __syncthreads();
        const f32x16 negm = (f32x16){} - m_ref;

        // kj/vj: the stages of tile j; kj1/vj1: those of tile j+1.
        auto iter = [&](int j, auto mask_tag, char* kj, char* kj1, char* vj, char* vj1) {
          constexpr bool MASK = decltype(mask_tag)::value;
          // Loads for V_{j+1} (LDS, stage (j+1)&1) and K_{j+2} (registers).
          if (j + 1 < n_tiles) load_v((j + 1) * BN, vj1, vw);
          if (j + 2 < n_tiles) load_k((j + 2) * BN, kj, kw, kc, ksn);
          f32x16 s_next[C::NKB];
          if (j + 1 < n_tiles && active(j + 1)) scores(kj1, s_next, negm);
          if (active(j)) {
            if constexpr (MASK) mask(j, s_cur);
            softmax_pv(vj, s_cur, std::false_type{}, 0.f, std::false_type{}, 1.f);
          }
          if (j + 2 < n_tiles) store_k((j + 2) * BN, kj, kw, kc, ksn, vw);
          wait_vmem();
          __syncthreads();
  #pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb) s_cur[kb] = s_next[kb];
        };
        // Steady state: tiles j+1 and j+2 exist, tile j needs no mask and the
        // wave has rows. Unrolled by two so every LDS stage is fixed at compile
        // time (the direct V load into one stage then needs no wait before the
        // reads of the others) and S alternates between two register sets; the
        // iteration is one straight-line block in which the matrix-core and
        // vector work of the two tiles can interleave.
        f32x16 s_alt[C::NKB];
        auto iter_steady = [&](int j, f32x16 (&s_in)[C::NKB], f32x16 (&s_out)[C::NKB], char* kj,
                               char* kj1, char* vj, char* vj1) {
          load_v((j + 1) * BN, vj1, vw);
          load_k((j + 2) * BN, kj, kw, kc, ksn);
          // Keep the global loads at the top of the block, a whole block ahead
          // of their use (left alone, the scheduler sinks them next to it).
          __builtin_amdgcn_sched_barrier(0);
          scores(kj1, s_out, negm);
          softmax_pv(vj, s_in, std::false_type{}, 0.f, std::false_type{}, 1.f);
          store_k((j + 2) * BN, kj, kw, kc, ksn, vw);
          wait_vmem();
          __syncthreads();
        };
        int j = 0;
        if (wave_has_rows) {
          const int n_steady = min(n_plain, n_tiles - 2);
          for (; j + 1 < n_steady; j += 2) {
            iter_steady(j, s_cur, s_alt, ks0, ks1, vs0, vs1);
            iter_steady(j + 1, s_alt, s_cur, ks1, ks0, vs1, vs0);
          }
        }
        for (; j < n_plain; ++j)
          iter(j, std::false_type{}, stage_of(j, ks0, ks1), stage_of(j + 1, ks0, ks1),
               stage_of(j, vs0, vs1), stage_of(j + 1, vs0, vs1));
        for (; j < n_tiles; ++j)
          iter(j, std::true_type{}, stage_of(j, ks0, ks1), stage_of(j + 1, ks0, ks1),
               stage_of(j, vs0, vs1), stage_of(j + 1, vs0, vs1));
      }
      m_fin = finish_unit(m_ref, std::false_type{});
    }

    // ---- Epilogue: O = O^T / l, rounded to bf16, goes through the wave's
    // staging area and leaves with whole rows per wave instruction; rows past
    // the sequence end fall outside the buffer range and are dropped.
    const float l_tot = pair_sum(l_run);
    const float inv = 1.f / l_tot;
    uint16_t* obase = (uint16_t*)a.o + (long)tok0 * qs + (long)head * D;
    const rsrc_t ro = make_rsrc(obase, (uint32_t)(((L - 1) * qs + D) * 2));
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = db * 32 + 8 * a4 + 4 * hh;
        const float o0 = oacc[db][4 * a4] * inv, o1 = oacc[db][4 * a4 + 1] * inv;
        const float o2 = oacc[db][4 * a4 + 2] * inv, o3 = oacc[db][4 * a4 + 3] * inv;
        *(u32x2*)(q_stage + l32 * C::Q_STRIDE + d * 2) =
            (u32x2){pack2(OpBF16{}, o0, o1), pack2(OpBF16{}, o2, o3)};
      }
    {
#pragma unroll
      for (int i = 0; i < 32 * QCH / 64; ++i) {
        const int flat = i * 64 + lane, r = flat / QCH, c = flat % QCH;
        const u32x4 row = *(const u32x4*)(q_stage + r * C::Q_STRIDE + c * 16);
        __builtin_amdgcn_raw_buffer_store_b128(row, ro, (qw0 + r) * qs * 2 + c * 16, 0, 0);
      }
    }
    if (a.lse != nullptr && hh == 0 && my_q < L)
      a.lse[lse_base + my_q] = (m_fin + log2f(l_tot)) * 0.69314718055994531f;
  }
};

// img0, img_kvs: the first K tile image of the unit's sequence (K/V head 0)
// and the images between consecutive K/V heads (used with once-rotated keys).
template <class C>
__device__ __forceinline__ void run_unit(const AttnArgs& a, int tok0, int L, int qb, int head0, long lse_b,
                                         long lse_h, long img0, long img_kvs, CGR_LDS_PARAMS) {
  if constexpr (C::F32)
    Unit<C>::run(a, tok0, L, qb, head0, lse_b, lse_h, ks0, ks1, vs0, vs1, qst);
  else
    UnitFast<C>::run(a, tok0, L, qb, head0, lse_b, lse_h, img0, img_kvs, ks0, ks1, vs0, vs1, qst);
}

// Ranks (query blocks, lightest first) of a causal dense call with once-
// rotated keys that are claimed at run time rather than placed by workgroup
// index: the lightest quarter.
__host__ __device__ constexpr int kfwd_dyn_ranks(int nQ) { return nQ / 4 > 1 ? nQ / 4 : 1; }
// The claim counter: the int after the tile images in the workspace.
template <class C>
__device__ __forceinline__ int* fwd_dyn_counter(const AttnArgs& a) {
  const long n_img = (long)a.B * a.KV * ((a.T + C::BN - 1) / C::BN);
  return (int*)((char*)a.krot + n_img * C::K_IMG);
}

// Dense batch: one workgroup per unit (entry, K/V group, hp heads of the
// group, query block). Heavy units (late query blocks, which see the most
// keys under the causal mask) are issued first, and when the (batch, kv-head)
// groups divide evenly over the 8 XCDs, each XCD takes whole groups so the
// query heads that share a K/V head share that XCD's L2.
template <class C>
__global__ __launch_bounds__(C::THREADS, C::WPS) void attn_fwd_dense_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char k0[C::K_BYTES], k1[C::K_BYTES];
  __shared__ __attribute__((aligned(16))) char v0[C::V_BYTES], v1[C::V_BYTES];
  extern __shared__ __attribute__((aligned(16))) char qst[];
  const int bm = 32 * C::NW / a.hp;
  const int nQ = (a.T + bm - 1) / bm;
  const int G = a.H / a.KV, GH = G / a.hp, groups = a.B * a.KV;
  const int u = blockIdx.x;
  int rank, g, hq;
  bool claimed = false;
  if constexpr (C::KPRE && C::CAUSAL && !C::WIN) {
    // The lightest quarter of the ranks goes to whichever XCD gets there
    // first: the XCDs run at different clocks (5-6 % apart under this load),
    // and with every unit placed by workgroup index (XCD u % 8) the slowest
    // one sets the kernel's end. The grid has two workgroups for each such
    // unit; each claims the next unit from a counter at the end of the
    // workspace (zeroed by krot_kernel) or exits when none is left, and the
    // last claimer sets the counter back to zero for the next call.
    const int per_rank = groups * GH, R0 = nQ - kfwd_dyn_ranks(nQ);
    const int S = R0 * per_rank, dyn = (nQ - R0) * per_rank;
    if (u >= S) {
      __shared__ int claim;
      if (threadIdx.x == 0) {
        int* ctr = fwd_dyn_counter<C>(a);
        const int d = atomicAdd(ctr, 1);
        if (d == 2 * dyn - 1) atomicExch(ctr, 0);
        claim = d;
      }
      __syncthreads();
      const int d = claim;
      if (d >= dyn) return;
      rank = R0 + d / per_rank;
      const int rem = d - (rank - R0) * per_rank;
      g = rem / GH;
      hq = rem - g * GH;
      claimed = true;
    }
  }
  // The items of a rank are rotated by the rank: an XCD deals its workgroups
  // out over its shader engines in turn, and a fixed order would hand one
  // engine the same (entry, heads) item rank after rank (all the long entry's
  // work, in a batch of mixed lengths).
  if (claimed) {
    // placed above
  } else if ((groups & 7) == 0) {
    const int x = u & 7, i = u >> 3, per = (groups >> 3) * GH;
    rank = i / per;
    const int rem = (i - rank * per + rank) % per;
    g = (rem / GH) * 8 + x;
    hq = rem % GH;
  } else {
    const int per = groups * GH;
    rank = u / per;
    const int rem = (u - rank * per + rank) % per;
    g = rem / GH;
    hq = rem % GH;
  }
  const int qb = C::CAUSAL ? nQ - 1 - rank : rank;
  const int b = g / a.KV, kvh = g - b * a.KV;
  const int head0 = kvh * G + hq * a.hp;
  // A padded entry is its first L tokens: the unit sees only those keys and
  // writes only those rows; units past them have nothing to do.
  const int L = a.seqlens == nullptr ? a.T : min(max(a.seqlens[b], 0), a.T);
  if (qb * bm >= L) return;
  // Images of a dense batch: per (entry, K/V head), ceil(T / BN) tiles.
  const long n_img = (a.T + C::BN - 1) / C::BN;
  run_unit<C>(a, b * a.T, L, qb, head0, (long)b * a.H * a.T, a.T, (long)b * a.KV * n_img, n_img, k0, k1, v0, v1,
              qst);
}

// Packed batch: one workgroup per unit (schedule item, head group of hp
// heads). The schedule lists items most expensive first, and the device hands
// out workgroups in index order as compute units free up, which balances the
// load (longest-processing-time-first) without a work queue. Workgroup u runs
// on XCD u % 8 and takes item (u / 8 / HG) * 8 + u % 8, head group
// (u / 8) % HG: the head groups of an item follow one another on one XCD,
// whose L2 then serves the item's K/V tiles to all of them. The grid covers
// the host's bound on the items, rounded up to 8, times HG; workgroups past
// the schedule's count exit at once.
template <class C>
__global__ __launch_bounds__(C::THREADS, C::WPS) void attn_fwd_varlen_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char k0[C::K_BYTES], k1[C::K_BYTES];
  __shared__ __attribute__((aligned(16))) char v0[C::V_BYTES], v1[C::V_BYTES];
  extern __shared__ __attribute__((aligned(16))) char qst[];
  const int HG = a.H / a.hp;  // head groups of hp heads
  const int j = blockIdx.x >> 3;
  const int it = (j / HG) * 8 + (blockIdx.x & 7), hg = j % HG;
  if (it >= a.sched[0]) return;
  const int2* items = (const int2*)(a.sched + kSchedHeaderInts);
  const int2 sq = items[it];
  const int tok0 = a.cu_seqlens[sq.x];
  const int L = a.cu_seqlens[sq.x + 1] - tok0;
  // Images of a packed batch: per K/V head, kimg_slots slots; sequence s's
  // tiles start at slot tok0 / BN + s (see varlen_prep_kernel).
  const long img0 = C::KPRE ? (long)(tok0 / C::BN + sq.x) : 0;
  run_unit<C>(a, tok0, L, sq.y, hg * a.hp, tok0, a.total_tokens, img0, a.kimg_slots, k0, k1, v0, v1, qst);
}

// K rotated once at its positions (token t of a dense batch entry is at
// position t) and rounded to the Q.K^T operand type, written as tile images:
// per (entry, K/V head, tile of BN keys), the tile exactly as the unit's LDS
// stage will hold it (rows of 2*D bytes, 16-byte chunks swizzled by tswz), so
// the unit copies each tile into LDS with 1-KiB direct loads. Keys past the
// entry's length are zeros. Item = (entry, image row, group g < D/16) carrying
// the chunk pair (g, g + D/16), as in the K loader, for every K/V head: the
// cos/sin values of the position are loaded once for all heads.
template <class C>
__global__ __launch_bounds__(256) void krot_kernel(AttnArgs a) {
  constexpr int D = C::D, BN = C::BN, IPR = D / 16;
  const int n_img = (a.T + BN - 1) / BN;
  const long tid = (long)blockIdx.x * 256 + threadIdx.x;
  const long item = tid / IPR;
  if (item >= (long)a.B * n_img * BN) return;
  const int g = (int)(tid % IPR), r = (int)(item % BN);
  const long bt = item / BN;  // b * n_img + tile
  const int tile = (int)(bt % n_img), b = (int)(bt / n_img);
  const int t = tile * BN + r;
  if (tid == 0) *fwd_dyn_counter<C>(a) = 0;  // the attention kernel's claim counter
  const int L = a.seqlens == nullptr ? a.T : min(max(a.seqlens[b], 0), a.T);
  const bool ok = t < L;
  f32x4 c[2], s[2];
  load_tab<D, C::STYLE>(a.rope_cos + (long)t * (D / 2), a.rope_sin + (long)t * (D / 2), g, ok, c, s);
  const uint16_t* kp = (const uint16_t*)a.k + ((long)b * a.T + t) * a.KV * D;
  for (int kv = 0; kv < a.KV; ++kv) {
    u32x4 w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
    if (ok) {
      const uint16_t* kh = kp + (long)kv * D;
      u32x4 i0[1] = {*(const u32x4*)(kh + 8 * g)}, i1[1] = {*(const u32x4*)(kh + 8 * g + D / 2)};
      float x0[8], x1[8];
      raw_to_f32<uint16_t>(i0, x0);
      raw_to_f32<uint16_t>(i1, x1);
      rope_pair<C::STYLE>(x0, x1, c, s);
      w0 = to_frag_or_nan<typename C::QK>(x0).v;
      w1 = to_frag_or_nan<typename C::QK>(x1).v;
    }
    const long img = ((long)b * a.KV + kv) * n_img + tile;
    char* row = (char*)a.krot + (long)img * C::K_IMG + r * 2 * D;
    *(u32x4*)(row + 16 * (g ^ tswz<D>(r))) = w0;
    *(u32x4*)(row + 16 * ((g + D / 16) ^ tswz<D>(r))) = w1;
  }
}

// Packed batch with the keys rotated once: workgroup 0 builds the work
// schedule (schedule_body) while the others write the K tile images, as for
// a dense batch, per K/V head in kimg_slots slots of one tile. Sequence s's
// tiles take the slots from floor(c_s / BN) + s on (c_s = cu_seqlens[s]): the
// next sequence starts past s's last tile (floor(c_s / BN) + ceil(L_s / BN)
// <= floor(c_{s+1} / BN) + 1), every slot stays below ceil(total / BN) +
// num_seqs, and the attention kernel finds a sequence's first slot from its
// first token, so the rotation needs nothing from the schedule and both run
// in one launch. A slot belongs to the last sequence whose first slot is at
// or before it; rows past that sequence's end, and slots between sequences,
// are zeros. With a malformed cu_seqlens the schedule sets the error word and
// schedules nothing, and the images (which then no unit reads) hold whatever
// the search finds; every read stays inside k and the tables regardless.
constexpr int kPrepThreads = kSchedThreads;
template <class C>
__global__ __launch_bounds__(kPrepThreads) void varlen_prep_kernel(AttnArgs a) {
  constexpr int D = C::D, BN = C::BN, IPR = D / 16, IPI = IPR * BN;  // items per image
  if (blockIdx.x == 0) {
    const int bm = 32 * C::NW / a.hp;
    schedule_body(a.cu_seqlens, a.B, a.total_tokens, a.T, __builtin_ctz(bm), __builtin_ctz(BN), C::CAUSAL,
                  a.sched, a.max_items, a.status_out);
    return;
  }
  const long tid = (long)(blockIdx.x - 1) * kPrepThreads + threadIdx.x;
  int img = (int)(tid / IPI);  // kv * kimg_slots + slot
  // A workgroup's items lie in one image when images are at least a
  // workgroup long: the search below is then uniform (scalar loads).
  if constexpr (IPI % kPrepThreads == 0) img = __builtin_amdgcn_readfirstlane(img);
  if (img >= a.KV * a.kimg_slots) return;
  const int within = (int)(tid % IPI);
  const int g = within % IPR, r = within / IPR;
  const int slot = img % a.kimg_slots, kv = img / a.kimg_slots;
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu_seqlens[mid] / BN + mid <= slot) lo = mid;
    else hi = mid - 1;
  }
  const int c0 = a.cu_seqlens[lo], L = a.cu_seqlens[lo + 1] - c0;
  const int t = (slot - (c0 / BN + lo)) * BN + r;
  u32x4 w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
  if (t >= 0 && t < L && t < a.T && c0 >= 0 && c0 + t < a.total_tokens) {
    const uint16_t* kp = (const uint16_t*)a.k + ((long)(c0 + t) * a.KV + kv) * D;
    u32x4 i0[1] = {*(const u32x4*)(kp + 8 * g)}, i1[1] = {*(const u32x4*)(kp + 8 * g + D / 2)};
    float x0[8], x1[8];
    raw_to_f32<uint16_t>(i0, x0);
    raw_to_f32<uint16_t>(i1, x1);
    f32x4 c[2], sn[2];
    load_tab<D, C::STYLE>(a.rope_cos + (long)t * (D / 2), a.rope_sin + (long)t * (D / 2), g, true, c, sn);
    rope_pair<C::STYLE>(x0, x1, c, sn);
    w0 = to_frag_or_nan<typename C::QK>(x0).v;
    w1 = to_frag_or_nan<typename C::QK>(x1).v;
  }
  char* row = (char*)a.krot + (long)img * C::K_IMG + r * 2 * D;
  *(u32x4*)(row + 16 * (g ^ tswz<D>(r))) = w0;
  *(u32x4*)(row + 16 * ((g + D / 16) ^ tswz<D>(r))) = w1;
}

// Launch one instance. Host-side, after the arguments are validated.
template <class C>
hipError_t launch_attn(const AttnArgs& a, bool varlen, int grid, hipStream_t stream) {
  if (varlen)
    hipLaunchKernelGGL(attn_fwd_varlen_kernel<C>, dim3(grid), dim3(C::THREADS), C::Q_STAGE_BYTES,
                       stream, a);
  else
    hipLaunchKernelGGL(attn_fwd_dense_kernel<C>, dim3(grid), dim3(C::THREADS), C::Q_STAGE_BYTES,
                       stream, a);
  return hipGetLastError();
}

// What a dense-batch launch with once-rotated keys (a.krot set) enqueues:
// the key rotation into the workspace, the attention kernel over it, or both.
enum { PHASE_ROTATE = 1, PHASE_ATTEND = 2, PHASE_ALL = 3 };

// Dense batch with the K rotation done once up front (a.krot set).
template <class C>
hipError_t launch_attn_kpre(const AttnArgs& a, int grid, hipStream_t stream, int phases) {
  if (C::CAUSAL && !C::WIN) {
    // Two workgroups for every claimed unit (see attn_fwd_dense_kernel: the
    // last of the 2 x dyn claims resets the counter, so the count is exact).
    const int bm = 32 * C::NW / a.hp, nQ = (a.T + bm - 1) / bm;
    const long more = (long)kfwd_dyn_ranks(nQ) * a.B * (a.H / a.hp);
    if (grid + more > 0x7fffffffL) return hipErrorInvalidValue;
    grid += (int)more;
  }
  if (phases & PHASE_ROTATE) {
    const long items = (long)a.B * ((a.T + C::BN - 1) / C::BN) * C::BN * (C::D / 16);
    hipLaunchKernelGGL((krot_kernel<C>), dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & PHASE_ATTEND)
    hipLaunchKernelGGL(attn_fwd_dense_kernel<C>, dim3(grid), dim3(C::THREADS), C::Q_STAGE_BYTES, stream, a);
  return hipGetLastError();
}

// Packed batch with the K rotation done once up front (a.krot set): the
// schedule and the rotation in one launch, then the attention kernel.
template <class C>
hipError_t launch_attn_kpre_varlen(const AttnArgs& a, int grid, hipStream_t stream) {
  const long items = (long)a.KV * a.kimg_slots * C::BN * (C::D / 16);
  hipLaunchKernelGGL((varlen_prep_kernel<C>), dim3((unsigned)(1 + (items + kPrepThreads - 1) / kPrepThreads)),
                     dim3(kPrepThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_fwd_varlen_kernel<C>, dim3(grid), dim3(C::THREADS), C::Q_STAGE_BYTES, stream, a);
  return hipGetLastError();
}

#ifndef CGR_MAX_HP
#define CGR_MAX_HP 8
#endif
// Waves per workgroup, query heads per unit (the largest power of two that
// divides both the waves and the group size G), query rows per unit and keys
// per tile of the forward instances of a head_dim.
// nw: the waves of an instance built with a count of its own (0: the default).
constexpr int fwd_waves(int head_dim, int nw = 0) { return head_dim == 256 ? 4 : nw > 0 ? nw : CGR_NW; }
constexpr int fwd_heads_per_unit(int head_dim, int G, int nw = 0) {
  int hp = 1;
  while (2 * hp <= fwd_waves(head_dim, nw) && 2 * hp <= CGR_MAX_HP && G % (2 * hp) == 0) hp *= 2;
  return hp;
}
constexpr int fwd_block_rows(int head_dim, int hp, int nw = 0) { return 32 * fwd_waves(head_dim, nw) / hp; }
// Waves of the dense instances for grids that would leave compute units idle
// (bf16 I/O, keys rotated on every tile, no window): twice the units of the
// default, each half as long.
constexpr int kSmallNW = 4;
constexpr int fwd_tile_keys(int head_dim) { return head_dim == 256 ? 32 : CGR_BN; }
constexpr int kMinBM = 32;  // smallest query block of any unit
// Bytes of one K tile image of the once-rotated keys (16-bit operands).
constexpr long fwd_kimg_bytes(int head_dim) { return (long)fwd_tile_keys(head_dim) * 2 * head_dim; }

template <class C>
hipError_t launch_attn_dense(const AttnArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(attn_fwd_dense_kernel<C>, dim3(grid), dim3(C::THREADS), C::Q_STAGE_BYTES, stream, a);
  return hipGetLastError();
}

// phases (dense batches with a.krot set): PHASE_ROTATE, PHASE_ATTEND or both.
// small: a dense bf16 call without window or once-rotated keys, on the
// kSmallNW-wave instances.
template <int D>
hipError_t launch_attn_d(const AttnArgs& a, int f32_io, int qk_bf16, int style, int causal,
                         bool varlen, int grid, hipStream_t stream, int phases, bool small) {
  if (small) {
    if (f32_io || varlen || a.window > 0 || a.krot != nullptr || D == 256) return hipErrorInvalidValue;
    if constexpr (D != 256) {
#define CGR_SMALL(QK, CAU)                                                                                  \
  return style == STYLE_HALF                                                                                \
      ? launch_attn_dense<Cfg<D, uint16_t, QK, CAU, STYLE_HALF, false, false, kSmallNW>>(a, grid, stream) \
      : launch_attn_dense<Cfg<D, uint16_t, QK, CAU, STYLE_INTERLEAVED, false, false, kSmallNW>>(a, grid, stream)
      if (qk_bf16) {
        if (causal) CGR_SMALL(OpBF16, true);
        CGR_SMALL(OpBF16, false);
      }
      if (causal) CGR_SMALL(OpF16, true);
      CGR_SMALL(OpF16, false);
#undef CGR_SMALL
    }
  }
#define CGR_LAUNCH(IO, QK, CAU, STY, WIN)                                                       \
  if constexpr (!std::is_same<IO, float>::value) {                                               \
    if (a.krot != nullptr)                                                                        \
      return varlen ? launch_attn_kpre_varlen<Cfg<D, IO, QK, CAU, STY, WIN, true>>(a, grid, stream) \
                    : launch_attn_kpre<Cfg<D, IO, QK, CAU, STY, WIN, true>>(a, grid, stream, phases); \
  }                                                                                               \
  return launch_attn<Cfg<D, IO, QK, CAU, STY, WIN>>(a, varlen, grid, stream)
#define CGR_BY_STYLE(IO, QK, CAU, WIN) \
  if (style == STYLE_HALF) { CGR_LAUNCH(IO, QK, CAU, STYLE_HALF, WIN); } else { CGR_LAUNCH(IO, QK, CAU, STYLE_INTERLEAVED, WIN); }
#define CGR_BY_MASK(IO, QK)                                                                           \
  if (causal && a.window > 0) { CGR_BY_STYLE(IO, QK, true, true) }                                   \
  else if (causal) { CGR_BY_STYLE(IO, QK, true, false) } else { CGR_BY_STYLE(IO, QK, false, false) }
  if (f32_io) {
    if constexpr (D == 256) return hipErrorInvalidValue;  // rejected by the host checks first
    else { CGR_BY_MASK(float, OpF32) }
  } else if (qk_bf16) {
    CGR_BY_MASK(uint16_t, OpBF16)
  } else {
    CGR_BY_MASK(uint16_t, OpF16)
  }
#undef CGR_BY_MASK
#undef CGR_BY_STYLE
#undef CGR_LAUNCH
}

}  // namespace cgr
