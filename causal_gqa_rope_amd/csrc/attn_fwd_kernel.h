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
// Work unit: one (sequence, query head, block of BM = 128 query rows). A
// workgroup of four waves runs it; wave w owns query rows 32w..32w+31.
//
// Per unit:
//   * Q rows are loaded once, rotated in f32 at their positions, multiplied by
//     scale*log2(e) and rounded once to the Q.K^T operand type; they stay in
//     registers as the B operand of S^T = K Q^T.
//   * Key/value tiles of BN = 64 rows stream through LDS, double-buffered:
//     while tile j is multiplied, tile j+1 is already loading into registers
//     (16-byte global loads); K is rotated at the key positions and rounded to
//     the operand type on its way into LDS; V goes in unchanged, row-major.
//   * S^T (keys x queries) comes out of 32x32x16 MFMAs with each lane holding
//     one query column, so the row max / row sum need only one exchange with
//     the partner lane (lane ^ 32) and the probabilities P feed the next
//     product straight from registers: O^T += V^T P^T, where V^T fragments are
//     read from the row-major V tile with transposing LDS reads.
//   * Causal: tiles entirely above the diagonal are never visited; only tiles
//     that straddle the diagonal (or the ragged end of a sequence) evaluate
//     the mask.
//   * Epilogue: O = O^T / l, rounded to the I/O type; lse = ln2 * (m + log2 l).
#pragma once

#include <type_traits>

#include "device_common.h"

namespace cgr {

enum { STYLE_INTERLEAVED = 0, STYLE_HALF = 1 };

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* rope_cos;  // [P, D/2]
  const float* rope_sin;
  const int32_t* cu_seqlens;  // packed batches
  int32_t* sched;             // packed batches: [0] items, [1] queue counter, [2] error, then items
  int B, T, H, KV;
  int total_tokens;
  float qscale;  // softmax_scale * log2(e), folded into Q
};

constexpr int kSchedHeaderInts = 4;

// Row stride (dwords) of the V tile in LDS: the transposing reads of one
// half-wave touch 4 rows x 64 bytes, which land on disjoint banks when the
// stride is 16 or 48 (mod 64) dwords.
constexpr int v_stride_dwords(int row_dwords) {
  int s = row_dwords;
  while ((s % 64) != 16 && (s % 64) != 48) ++s;
  return s;
}

template <int D_, typename IO_, typename QK_, bool CAUSAL_, int STYLE_>
struct Cfg {
  static constexpr int D = D_;
  using IO = IO_;  // float, or uint16_t holding bf16 bits
  using QK = QK_;  // OpF16 / OpBF16 / OpF32
  static constexpr bool F32 = std::is_same<IO, float>::value;
  using PV = typename std::conditional<F32, OpF32, OpBF16>::type;
  static constexpr bool CAUSAL = CAUSAL_;
  static constexpr int STYLE = STYLE_;

  static constexpr int NW = 4;
  static constexpr int THREADS = 64 * NW;
  static constexpr int BM = 32 * NW;  // query rows per unit
  static constexpr int BN = 64;       // keys per tile
  static constexpr int ESZ = F32 ? 4 : 2;
  static constexpr int KSTEPS = D / 16;  // 32x32x16 k-steps over the head dim
  static constexpr int DB = D / 32;      // 32-wide blocks of the head dim
  static constexpr int NKB = BN / 32;    // 32-key blocks per tile

  static constexpr int K_STRIDE = D * ESZ + 16;  // bytes per K row in LDS
  static constexpr int V_STRIDE = F32 ? D * 4 + 16 : 4 * v_stride_dwords(D / 2);
  static constexpr int K_BYTES = BN * K_STRIDE;
  static constexpr int V_BYTES = BN * V_STRIDE;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int SMEM = 2 * STAGE;

  // Loader work items. K: (row, 8-element group g < D/16), which carries the
  // group pair (g, g + D/16) so that both RoPE pairings find their partners.
  static constexpr int K_ITEMS = BN * (D / 16);
  static constexpr int KU = (K_ITEMS + THREADS - 1) / THREADS;
  static constexpr int KW = F32 ? 2 : 1;  // 16-byte words per 8-element group
  // V: 16-byte chunks.
  static constexpr int V_CHUNKS = D * ESZ / 16;
  static constexpr int V_ITEMS = BN * V_CHUNKS;
  static constexpr int VU = (V_ITEMS + THREADS - 1) / THREADS;

  static_assert(D == 32 || D == 64 || D == 128, "head_dim");
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
template <int STYLE>
__device__ __forceinline__ void rope_pair(float (&x0)[8], float (&x1)[8], const f32x4 (&c)[2],
                                          const f32x4 (&s)[2]) {
  if constexpr (STYLE == STYLE_INTERLEAVED) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float a = x0[2 * m], b = x0[2 * m + 1];
      x0[2 * m] = a * c[0][m] - b * s[0][m];
      x0[2 * m + 1] = a * s[0][m] + b * c[0][m];
      a = x1[2 * m];
      b = x1[2 * m + 1];
      x1[2 * m] = a * c[1][m] - b * s[1][m];
      x1[2 * m + 1] = a * s[1][m] + b * c[1][m];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float cj = c[j >> 2][j & 3], sj = s[j >> 2][j & 3];
      const float a = x0[j], b = x1[j];
      x0[j] = a * cj - b * sj;
      x1[j] = a * sj + b * cj;
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

  // One work unit: query rows qb*BM .. of a sequence of L tokens starting at
  // token tok0, query head `head`. lse_base indexes lse[] for local row 0.
  static __device__ __forceinline__ void run(const AttnArgs& a, int tok0, int L, int qb, int head,
                                             long lse_base, char* smem) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int G = a.H / a.KV, kvh = head / G;
    const long qs = (long)a.H * D, ks = (long)a.KV * D;
    const IO* qp = (const IO*)a.q + (long)tok0 * qs + (long)head * D;
    const IO* kp = (const IO*)a.k + (long)tok0 * ks + (long)kvh * D;
    const IO* vp = (const IO*)a.v + (long)tok0 * ks + (long)kvh * D;

    const int q0 = qb * C::BM;
    const int qw0 = q0 + wave * 32;
    const int my_q = qw0 + l32;
    const bool wave_has_rows = qw0 < L;
    const int wave_last = min(qw0 + 31, L - 1);
    const int q_hi = min(q0 + C::BM, L);
    const int n_tiles = C::CAUSAL ? (q_hi + BN - 1) / BN : (L + BN - 1) / BN;

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
    load_tile(regs, kp, vp, ks, 0, L, a.rope_cos, a.rope_sin);
    store_tile(regs, smem, smem + C::K_BYTES);
    __syncthreads();

    for (int j = 0; j < n_tiles; ++j) {
      const int kt0 = j * BN;
      if (j + 1 < n_tiles) load_tile(regs, kp, vp, ks, kt0 + BN, L, a.rope_cos, a.rope_sin);
      const char* Ks = smem + (j & 1) * C::STAGE;
      const char* Vs = Ks + C::K_BYTES;
      const bool active = wave_has_rows && (!C::CAUSAL || kt0 <= wave_last);
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
        // Mask: only tiles that straddle the diagonal or the sequence end.
        const bool need_mask = C::CAUSAL ? (kt0 + BN - 1 > qw0) : (kt0 + BN > L);
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kt0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
              if ((C::CAUSAL && key > my_q) || key >= L) sacc[kb][i] = -INFINITY;
            }
        }
        // Online softmax. Tile 0 always holds key 0, which every row may see,
        // so m_new is finite from the first tile on.
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        mx = pair_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(sacc[kb][i] - m_new);
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
      if (j + 1 < n_tiles) {
        char* nK = smem + ((j + 1) & 1) * C::STAGE;
        store_tile(regs, nK, nK + C::K_BYTES);
      }
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

// Dense batch: one workgroup per unit. Heavy units (late query blocks, which
// see the most keys under the causal mask) are issued first, and when the
// (batch, kv-head) groups divide evenly over the 8 XCDs, each XCD takes whole
// groups so the query heads that share a K/V head share that XCD's L2.
template <class C>
__global__ __launch_bounds__(C::THREADS, 2) void attn_fwd_dense_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  const int nQ = (a.T + C::BM - 1) / C::BM;
  const int G = a.H / a.KV, groups = a.B * a.KV;
  const int u = blockIdx.x;
  int rank, g, hq;
  if ((groups & 7) == 0) {
    const int x = u & 7, i = u >> 3, per = (groups >> 3) * G;
    rank = i / per;
    const int rem = i - rank * per;
    g = (rem / G) * 8 + x;
    hq = rem % G;
  } else {
    const int per = groups * G;
    rank = u / per;
    const int rem = u - rank * per;
    g = rem / G;
    hq = rem % G;
  }
  const int qb = C::CAUSAL ? nQ - 1 - rank : rank;
  const int b = g / a.KV, kvh = g - b * a.KV;
  const int head = kvh * G + hq;
  Unit<C>::run(a, b * a.T, a.T, qb, head, ((long)b * a.H + head) * a.T, smem);
}

// Packed batch: a persistent grid pulls (sequence, query block) items from the
// schedule in order (most expensive first); each item expands to all heads.
template <class C>
__global__ __launch_bounds__(C::THREADS, 2) void attn_fwd_varlen_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ int s_unit;
  const int n_units = a.sched[0] * a.H;
  int* counter = a.sched + 1;
  const int2* items = (const int2*)(a.sched + kSchedHeaderInts);
  for (;;) {
    if (threadIdx.x == 0) s_unit = atomicAdd(counter, 1);
    __syncthreads();
    const int u = s_unit;
    __syncthreads();
    if (u >= n_units) break;
    const int it = u / a.H, head = u - it * a.H;
    const int2 sq = items[it];
    const int tok0 = a.cu_seqlens[sq.x];
    const int L = a.cu_seqlens[sq.x + 1] - tok0;
    Unit<C>::run(a, tok0, L, sq.y, head, (long)head * a.total_tokens + tok0, smem);
  }
}

// Launch one instance. Host-side, after the arguments are validated.
template <class C>
hipError_t launch_attn(const AttnArgs& a, bool varlen, int grid, hipStream_t stream) {
  if (varlen)
    hipLaunchKernelGGL(attn_fwd_varlen_kernel<C>, dim3(grid), dim3(C::THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_fwd_dense_kernel<C>, dim3(grid), dim3(C::THREADS), 0, stream, a);
  return hipGetLastError();
}

constexpr int kBM = 128;  // query rows per unit (all instances)
constexpr int kBN = 64;   // keys per tile (all instances)

template <int D>
hipError_t launch_attn_d(const AttnArgs& a, int f32_io, int qk_bf16, int style, int causal,
                         bool varlen, int grid, hipStream_t stream) {
#define CGR_LAUNCH(IO, QK, CAU, STY) return launch_attn<Cfg<D, IO, QK, CAU, STY>>(a, varlen, grid, stream)
#define CGR_BY_STYLE(IO, QK, CAU) \
  if (style == STYLE_HALF) { CGR_LAUNCH(IO, QK, CAU, STYLE_HALF); } else { CGR_LAUNCH(IO, QK, CAU, STYLE_INTERLEAVED); }
#define CGR_BY_MASK(IO, QK) \
  if (causal) { CGR_BY_STYLE(IO, QK, true) } else { CGR_BY_STYLE(IO, QK, false) }
  if (f32_io) {
    CGR_BY_MASK(float, OpF32)
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
