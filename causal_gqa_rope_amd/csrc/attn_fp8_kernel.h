// Fused causal GQA + RoPE attention forward with fp8 (OCP e4m3) operands on
// the gfx950 matrix cores (internal to libcgr).
//
// What is computed is the attention of the bf16 forward ("Attention from
// Scratch", section "Attention, the math"; RoPE from "Embeddings & the
// Residual Stream", "Positional information: RoPE") on inputs given in fp8:
// the real q, k, v are the e4m3 values times a per-tensor descale each. Both
// products run on v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, f32
// accumulation, twice the bf16 rate):
//   * Q.K^T: the keys, rotated once in f32 by fp8_prep_kernel and halved (the
//     rotation can grow a component by up to sqrt 2), are rounded back to
//     e4m3; the queries, rotated in the unit's prologue, are scaled by gamma
//     in [1/4, 1/2) and rounded to e4m3. The remaining factor of the softmax
//     scale, log2(e) and the descales is a power of two 2^E, applied by the
//     instruction's block scale, so the accumulator holds the score in log2
//     units directly.
//   * P.V: p = 2^(s - m) rounded to e4m3 (2^-9 .. 448; above 464 it rounds
//     to NaN), against V
//     as given; the row sum adds the unrounded p in f32; O is scaled by the V
//     descale / row sum once at the end.
// The row reference m is the row's max over the first key tile (as in the
// bf16 fast path); a unit whose later scores exceed it by so much that some
// p leaves e4m3's range (which turns into NaN) is recomputed with the
// classic rescaling online softmax, where p <= 1.
//
// Operand layouts (32x32x64, fp8): lane l holds row / column l % 32 and 32
// consecutive k-slots 32 (l / 32) .. +31, 8 registers. The S accumulator of a
// 64-key tile holds, in lane (query l32, half hh), keys 32 kb + 8 (i / 4) +
// 4 hh + i % 4 for kb < 2, i < 16; the P.V product takes those 32 values as
// its B operand in register order, i.e. k-slot 32 hh + 16 kb + i stands for
// that key. fp8_prep_kernel writes each V tile transposed (rows = head dim)
// with its keys in that slot order, so the A operand is 32 contiguous bytes.
// K tiles, V^T tiles and the Q staging use XOR-swizzled 16-byte chunks so the
// 16 lanes of a bank cycle read distinct bank slots.
#pragma once

#include "attn_fwd_kernel.h"

namespace cgr {

typedef int i32x8 __attribute__((ext_vector_type(8)));

struct Fp8Args {
  const uint8_t* q;  // [B, T, H, D] e4m3
  const uint8_t* k;  // [B, T, KV, D] e4m3
  const uint8_t* v;  // [B, T, KV, D] e4m3
  uint8_t* kimg;     // [B, KV, NT] tile images of the rotated keys (64 x D bytes)
  uint8_t* vimg;     // [B, KV, NT] tile images of V^T in slot order (D x 64 bytes)
  void* o;           // [B, T, H, D] bf16
  float* lse;        // [B, H, T] or null
  const float* rope_cos;
  const float* rope_sin;
  const int32_t* seqlens;  // valid tokens per entry (right padding), or null: T
  int B, T, H, KV, NT;
  float qgamma;      // rotated q (in e4m3 units) times this is the Q operand
  int kscale;        // e8m0 block scale 2^E of the K operand, in every byte
  float vdescale;
};

constexpr int kFp8D = 128;   // head_dim of the fp8 instances
constexpr int kFp8BN = 64;   // keys per tile
#ifndef CGR_FP8_NW
#define CGR_FP8_NW 4
#endif
constexpr int kFp8NW = CGR_FP8_NW;  // waves per workgroup (4: two workgroups per CU, measured 2.5 % over 8)
constexpr int kFp8BM = 32 * kFp8NW;
constexpr int kFp8Tile = kFp8BN * kFp8D;  // bytes of one K or V^T tile image

// 16-byte chunk swizzles: K / Q rows of 128 bytes, V^T rows of 64 bytes.
__device__ __forceinline__ int swz128(int r) {
  return (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1);
}
__device__ __forceinline__ int swz64(int r) { return (r >> 2) & 3; }

// Two e4m3 bytes <-> two floats.
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}
template <bool HI>
__device__ __forceinline__ uint32_t f32x2_to_fp8(float a, float b, uint32_t old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}
// 8 e4m3 bytes (two dwords) -> 8 floats, and back.
__device__ __forceinline__ void fp8x8_to_f32(uint32_t w0, uint32_t w1, float (&x)[8]) {
  const f32x2 a = fp8x2_to_f32<false>(w0), b = fp8x2_to_f32<true>(w0);
  const f32x2 c = fp8x2_to_f32<false>(w1), d = fp8x2_to_f32<true>(w1);
  x[0] = a[0]; x[1] = a[1]; x[2] = b[0]; x[3] = b[1];
  x[4] = c[0]; x[5] = c[1]; x[6] = d[0]; x[7] = d[1];
}
__device__ __forceinline__ u32x2 f32x8_to_fp8(const float (&x)[8]) {
  uint32_t w0 = f32x2_to_fp8<false>(x[0], x[1], 0u);
  w0 = f32x2_to_fp8<true>(x[2], x[3], w0);
  uint32_t w1 = f32x2_to_fp8<false>(x[4], x[5], 0u);
  w1 = f32x2_to_fp8<true>(x[6], x[7], w1);
  return (u32x2){w0, w1};
}

// ---- Key rotation and tile images. One workgroup of 256 threads per
// (batch entry, K/V head, 64-key tile).
//   K: item (row, group g < D/16) = elements 8g..8g+7 and their partners
//   8g+D/2.. (both pairings find their partners inside the item); rotated in
//   f32 at the row's position, halved, rounded to e4m3, written swizzled.
//   Rows past the sequence are zeros.
//   V^T: the tile is staged in LDS, then each thread gathers 16-key chunks of
//   one head-dim row in slot order.
template <int STYLE>
__global__ __launch_bounds__(256) void fp8_prep_kernel(Fp8Args a) {
  constexpr int D = kFp8D, BN = kFp8BN;
  __shared__ __attribute__((aligned(16))) uint8_t vt[BN * D];
  const int tile = blockIdx.x % a.NT, bk = blockIdx.x / a.NT;  // bk = b * KV + kv
  const int b = bk / a.KV, kv = bk % a.KV;
  const int t0 = tile * BN;
  const int tid = threadIdx.x;
  uint8_t* kimg = a.kimg + (long)blockIdx.x * kFp8Tile;
  uint8_t* vimg = a.vimg + (long)blockIdx.x * kFp8Tile;
  const long ks = (long)a.KV * D;  // token stride
  const uint8_t* kb = a.k + ((long)b * a.T) * ks + (long)kv * D;
  const uint8_t* vb = a.v + ((long)b * a.T) * ks + (long)kv * D;
  const int L = a.seqlens == nullptr ? a.T : min(max(a.seqlens[b], 0), a.T);
  // K: BN rows x D/16 items, 2 per thread.
  for (int it = tid; it < BN * (D / 16); it += 256) {
    const int r = it / (D / 16), g = it % (D / 16), t = t0 + r;
    u32x2 w0 = {0u, 0u}, w1 = {0u, 0u};
    if (t < L) {
      const uint8_t* src = kb + (long)t * ks;
      const u32x2 i0 = *(const u32x2*)(src + 8 * g), i1 = *(const u32x2*)(src + 8 * g + D / 2);
      float x0[8], x1[8];
      fp8x8_to_f32(i0[0], i0[1], x0);
      fp8x8_to_f32(i1[0], i1[1], x1);
      f32x4 c[2], s[2];
      load_tab<D, STYLE>(a.rope_cos + (long)t * (D / 2), a.rope_sin + (long)t * (D / 2), g, true, c, s);
      rope_pair<STYLE>(x0, x1, c, s);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x0[j] *= 0.5f;
        x1[j] *= 0.5f;
      }
      w0 = f32x8_to_fp8(x0);
      w1 = f32x8_to_fp8(x1);
    }
    // element e of row r sits at chunk e/16 (swizzled), byte e%16
    const int e0 = 8 * g, e1 = 8 * g + D / 2;
    *(u32x2*)(kimg + r * D + 16 * ((e0 >> 4) ^ swz128(r)) + (e0 & 15)) = w0;
    *(u32x2*)(kimg + r * D + 16 * ((e1 >> 4) ^ swz128(r)) + (e1 & 15)) = w1;
  }
  // V: stage the tile (rows past the sequence as zeros).
  for (int it = tid; it < BN * D / 16; it += 256) {
    const int r = it / (D / 16), c = it % (D / 16), t = t0 + r;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (t < L) w = *(const u32x4*)(vb + (long)t * ks + 16 * c);
    *(u32x4*)(vt + r * D + 16 * c) = w;
  }
  __syncthreads();
  // V^T: D rows x 4 chunks of 16 slots; slot 32hh + 16kb + i holds key
  // 32kb + 8(i/4) + 4hh + i%4.
  for (int it = tid; it < D * 4; it += 256) {
    const int d = it / 4, c = it % 4;
    uint32_t w[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      uint32_t x = 0;
#pragma unroll
      for (int by = 0; by < 4; ++by) {
        const int slot = 16 * c + 4 * q4 + by;
        const int hh = slot >> 5, kbk = (slot >> 4) & 1, i = slot & 15;
        const int key = 32 * kbk + 8 * (i >> 2) + 4 * hh + (i & 3);
        x |= (uint32_t)vt[key * D + d] << (8 * by);
      }
      w[q4] = x;
    }
    *(u32x4*)(vimg + d * BN + 16 * (c ^ swz64(d))) = (u32x4){w[0], w[1], w[2], w[3]};
  }
}

__device__ __forceinline__ f32x16 mma_fp8(i32x8 a, i32x8 b, f32x16 c, int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, 0x7f7f7f7f);
}
__device__ __forceinline__ i32x8 lds32(const char* p0, const char* p1) {
  const u32x4 x = *(const u32x4*)p0, y = *(const u32x4*)p1;
  return (i32x8){(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
}

#define CGR_FP8_LDS char *ks0, char *ks1, char *vs0, char *vs1, char *qst

template <bool CAUSAL, int STYLE>
struct UnitFp8 {
  static constexpr int D = kFp8D, BN = kFp8BN, NW = kFp8NW, BM = kFp8BM;
  static constexpr int NKB = BN / 32, DB = D / 32;

  // Entry b's first L tokens (L <= T, the entry stride).
  static __device__ __forceinline__ void run(const Fp8Args& a, int b, int L, int qb, int head, CGR_FP8_LDS) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int T = a.T;
    const int G = a.H / a.KV, kvh = head / G;
    const int qs = a.H * D;  // token stride of q and o (elements)
    const uint8_t* qbase = a.q + ((long)b * T) * qs + (long)head * D;
    const long img0 = ((long)b * a.KV + kvh) * a.NT * kFp8Tile;
    const rsrc_t rk = make_rsrc(a.kimg + img0, (uint32_t)(a.NT * kFp8Tile));
    const rsrc_t rv = make_rsrc(a.vimg + img0, (uint32_t)(a.NT * kFp8Tile));

    const int q0 = qb * BM, qw0 = q0 + wave * 32, my_q = qw0 + l32;
    const bool wave_has_rows = qw0 < L;
    const int wave_last = min(qw0 + 31, L - 1);
    const int q_hi = min(q0 + BM, L);
    const int n_tiles = CAUSAL ? (q_hi + BN - 1) / BN : (L + BN - 1) / BN;
    const int n_plain = CAUSAL ? min(n_tiles, (q0 + 1) / BN) : L / BN;
    auto active = [&](int t) { return wave_has_rows && (!CAUSAL || t * BN <= wave_last); };

    // Tile images: 8 KiB = 8 direct loads of 1 KiB, spread over the waves.
    auto load_k = [&](int j, char* kst) {
#pragma unroll
      for (int u = 0; u < 8 / NW; ++u)
        buf_load16_lds(rk, kst + (wave + u * NW) * 1024, lane * 16, j * kFp8Tile + (wave + u * NW) * 1024);
    };
    auto load_v = [&](int j, char* vst) {
#pragma unroll
      for (int u = 0; u < 8 / NW; ++u)
        buf_load16_lds(rv, vst + (wave + u * NW) * 1024, lane * 16, j * kFp8Tile + (wave + u * NW) * 1024);
    };

    // ---- Q: rotate this wave's 32 rows at their positions, scale by gamma,
    // round to e4m3, stage (swizzled) and read back as B fragments. Item =
    // (row, chunk pair c, c + 4): 16 elements and their partners D/2 on.
    char* const q_stage = qst + wave * 32 * D;
    i32x8 qf[2];
    auto stage_q = [&]() {
      const rsrc_t rq = make_rsrc(qbase, (uint32_t)((L - 1) * qs + D));
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2) {
        const int item = i2 * 64 + lane, r = item / 4, c = item % 4;
        const int row = qw0 + r, pos = row < L ? row : 0;
        const u32x4 w0 = buf_load16(rq, row * qs + 16 * c, 0);
        const u32x4 w1 = buf_load16(rq, row * qs + 16 * c + D / 2, 0);
        const float* cs = a.rope_cos + (long)pos * (D / 2);
        const float* sn = a.rope_sin + (long)pos * (D / 2);
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {  // 8 elements at a time: group g = 2c + h8
          const int g = 2 * c + h8;
          float x0[8], x1[8];
          fp8x8_to_f32(w0[2 * h8], w0[2 * h8 + 1], x0);
          fp8x8_to_f32(w1[2 * h8], w1[2 * h8 + 1], x1);
          f32x4 tc[2], ts[2];
          load_tab<D, STYLE>(cs, sn, g, true, tc, ts);
          rope_pair<STYLE>(x0, x1, tc, ts);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            x0[j] *= a.qgamma;
            x1[j] *= a.qgamma;
          }
          const int e0 = 8 * g, e1 = 8 * g + D / 2;
          *(u32x2*)(q_stage + r * D + 16 * ((e0 >> 4) ^ swz128(r)) + (e0 & 15)) = f32x8_to_fp8(x0);
          *(u32x2*)(q_stage + r * D + 16 * ((e1 >> 4) ^ swz128(r)) + (e1 & 15)) = f32x8_to_fp8(x1);
        }
      }
      // k-step s: bytes 64s + 32hh .. +31 of row l32 = chunks 4s + 2hh, +1.
#pragma unroll
      for (int s = 0; s < 2; ++s)
        qf[s] = lds32(q_stage + l32 * D + 16 * ((4 * s + 2 * hh) ^ swz128(l32)),
                      q_stage + l32 * D + 16 * ((4 * s + 2 * hh + 1) ^ swz128(l32)));
    };

    // ---- Products.
    const int ksc = a.kscale;
    auto scores = [&](const char* Ks, f32x16 (&sacc)[NKB], const f32x16& cinit) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int r = kb * 32 + l32;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const i32x8 kf = lds32(Ks + r * D + 16 * ((4 * s + 2 * hh) ^ swz128(r)),
                                 Ks + r * D + 16 * ((4 * s + 2 * hh + 1) ^ swz128(r)));
          sacc[kb] = mma_fp8(kf, qf[s], s == 0 ? cinit : sacc[kb], ksc);
        }
      }
    };
    auto mask = [&](int j, f32x16 (&sacc)[NKB]) {
      const int lim = (CAUSAL ? min(my_q, L - 1) : L - 1) - j * BN - 4 * hh;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 8 * (i >> 2) + (i & 3) > lim) sacc[kb][i] = -INFINITY;
    };
    auto rowmax = [&](const f32x16 (&sacc)[NKB]) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      return pair_max(mx);
    };
    f32x16 oacc[DB];
    float l_run = 0.f;
    // p = 2^(s - shift) -> e4m3 B fragment (slot order = register order);
    // the row sum adds the unrounded p.
    auto probs = [&](const f32x16 (&sacc)[NKB], float shift, i32x8& pf) {
      float l0 = 0.f, l1 = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kb = j >> 2, i = 4 * (j & 3);
        const float p0 = fast_exp2(sacc[kb][i] - shift), p1 = fast_exp2(sacc[kb][i + 1] - shift);
        const float p2 = fast_exp2(sacc[kb][i + 2] - shift), p3 = fast_exp2(sacc[kb][i + 3] - shift);
        l0 += p0 + p1;
        l1 += p2 + p3;
        const uint32_t w = f32x2_to_fp8<false>(p0, p1, 0u);
        pf[j] = (int)f32x2_to_fp8<true>(p2, p3, w);
      }
      l_run += l0 + l1;
    };
    auto pv = [&](const char* Vs, const i32x8& pf) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int r = db * 32 + l32;
        const i32x8 vf = lds32(Vs + r * BN + 16 * ((2 * hh) ^ swz64(r)),
                               Vs + r * BN + 16 * ((2 * hh + 1) ^ swz64(r)));
        oacc[db] = mma_fp8(vf, pf, oacc[db], 0x7f7f7f7f);
      }
    };

    // ---- Fast path: the reference m of each row is its max over tile 0; S
    // of later tiles starts from -m. Software-pipelined by one tile: iteration
    // j computes S_{j+1} while P_j V_j runs. LDS holds K one tile ahead of V.
    float m_ref = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){};
    __syncthreads();  // earlier users of this workgroup's LDS are done
    load_k(0, ks0);
    load_v(0, vs0);
    if (n_tiles > 1) load_k(1, ks1);
    stage_q();
    wait_vmem();
    __syncthreads();
    f32x16 s_cur[NKB];
    if (wave_has_rows) {
      scores(ks0, s_cur, (f32x16){});
      mask(0, s_cur);
      m_ref = rowmax(s_cur);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s_cur[kb] -= m_ref;
    }
    __syncthreads();  // every wave is done with K_0 before iteration 0 loads K_2 over it
    const f32x16 negm = (f32x16){} - m_ref;
    auto iter = [&](int j, auto mask_tag, char* kj, char* kj1, char* vj, char* vj1) {
      constexpr bool MASK = decltype(mask_tag)::value;
      if (j + 1 < n_tiles) load_v(j + 1, vj1);
      if (j + 2 < n_tiles) load_k(j + 2, kj);
      f32x16 s_next[NKB];
      if (j + 1 < n_tiles && active(j + 1)) scores(kj1, s_next, negm);
      if (active(j)) {
        if constexpr (MASK) mask(j, s_cur);
        i32x8 pf;
        probs(s_cur, 0.f, pf);
        pv(vj, pf);
      }
      wait_vmem();
      __syncthreads();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s_cur[kb] = s_next[kb];
    };
    // Steady state (tiles j+1 and j+2 exist, tile j needs no mask, the wave
    // has rows): straight-line code with the stages fixed at compile time,
    // S alternating between two register sets.
    f32x16 s_alt[NKB];
    auto iter_steady = [&](int j, f32x16 (&s_in)[NKB], f32x16 (&s_out)[NKB], char* kj, char* kj1, char* vj,
                           char* vj1) {
      load_v(j + 1, vj1);
      load_k(j + 2, kj);
      // Keep the loads at the top, a whole tile ahead of their use.
      __builtin_amdgcn_sched_barrier(0);
      scores(kj1, s_out, negm);
      i32x8 pf;
      probs(s_in, 0.f, pf);
      pv(vj, pf);
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
    for (; j < n_tiles; ++j) {
      if (j < n_plain)
        iter(j, std::false_type{}, stage_of(j, ks0, ks1), stage_of(j + 1, ks0, ks1), stage_of(j, vs0, vs1),
             stage_of(j + 1, vs0, vs1));
      else
        iter(j, std::true_type{}, stage_of(j, ks0, ks1), stage_of(j + 1, ks0, ks1), stage_of(j, vs0, vs1),
             stage_of(j + 1, vs0, vs1));
    }
    float m_fin = m_ref;
    // A p above 464 rounds to NaN in e4m3 (and poisons O); 0 * NaN/inf is
    // NaN, so one sum over the accumulators finds it.
    float chk = l_run * 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) chk += oacc[db][i] * 0.f;
    const bool bad = !(chk == 0.f) || !(pair_sum(l_run) <= 1.099511627776e12f);
    if (__syncthreads_or(bad)) {
      // ---- Rescaling path (classic online softmax, p <= 1), not pipelined.
      float m_run = -INFINITY;
      l_run = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){};
      for (int t = 0; t < n_tiles; ++t) {
        __syncthreads();
        load_k(t, ks0);
        load_v(t, vs0);
        wait_vmem();
        __syncthreads();
        if (active(t)) {
          f32x16 sacc[NKB];
          scores(ks0, sacc, (f32x16){});
          mask(t, sacc);
          const float m_new = fmaxf(m_run, rowmax(sacc));
          const float alpha = fast_exp2(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
          i32x8 pf;
          probs(sacc, m_new, pf);
          pv(vs0, pf);
        }
      }
      m_fin = m_run;
    }

    // ---- Epilogue: O = O^T * vdescale / l in bf16, 8-byte stores straight
    // from the accumulators (rows past the sequence fall outside the range).
    const float l_tot = pair_sum(l_run);
    const float inv = a.vdescale / l_tot;
    uint16_t* obase = (uint16_t*)a.o + ((long)b * T) * qs + (long)head * D;
    const rsrc_t ro = make_rsrc(obase, (uint32_t)(((L - 1) * qs + D) * 2));
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d = db * 32 + 8 * a4 + 4 * hh;
        const u32x2 ov = (u32x2){pack2(OpBF16{}, oacc[db][4 * a4] * inv, oacc[db][4 * a4 + 1] * inv),
                                 pack2(OpBF16{}, oacc[db][4 * a4 + 2] * inv, oacc[db][4 * a4 + 3] * inv)};
        __builtin_amdgcn_raw_buffer_store_b64(ov, ro, (my_q * qs + d) * 2, 0, 0);
      }
    if (a.lse != nullptr && hh == 0 && my_q < L)
      a.lse[((long)b * a.H + head) * T + my_q] = (m_fin + log2f(l_tot)) * 0.69314718055994531f;
  }
};

// Dense batch, one workgroup per (entry, query head, 32 * kFp8NW-row block),
// two workgroups per CU (each wave has 256 registers): heavy
// blocks first; when the (entry, K/V head) groups divide over the 8 XCDs, each
// XCD takes whole groups (their query heads share the XCD's L2).
template <bool CAUSAL, int STYLE>
__global__ __launch_bounds__(64 * kFp8NW, 2) void attn_fwd_fp8_kernel(Fp8Args a) {
  __shared__ __attribute__((aligned(16))) char k0[kFp8Tile], k1[kFp8Tile];
  __shared__ __attribute__((aligned(16))) char v0[kFp8Tile], v1[kFp8Tile];
  __shared__ __attribute__((aligned(16))) char qst[kFp8NW * 32 * kFp8D];
  const int nQ = (a.T + kFp8BM - 1) / kFp8BM;
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
  const int qb = CAUSAL ? nQ - 1 - rank : rank;
  const int b = g / a.KV, kvh = g - b * a.KV;
  // A padded entry is its first L tokens; units past them have nothing to do.
  const int L = a.seqlens == nullptr ? a.T : min(max(a.seqlens[b], 0), a.T);
  if (qb * kFp8BM >= L) return;
  UnitFp8<CAUSAL, STYLE>::run(a, b, L, qb, kvh * G + hq, k0, k1, v0, v1, qst);
}

template <bool CAUSAL, int STYLE>
hipError_t launch_fp8_inst(const Fp8Args& a, hipStream_t stream) {
  hipLaunchKernelGGL((fp8_prep_kernel<STYLE>), dim3((unsigned)(a.B * a.KV * a.NT)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long grid = (long)((a.T + kFp8BM - 1) / kFp8BM) * a.B * a.H;
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<CAUSAL, STYLE>), dim3((unsigned)grid), dim3(64 * kFp8NW), 0, stream, a);
  return hipGetLastError();
}

}  // namespace cgr
