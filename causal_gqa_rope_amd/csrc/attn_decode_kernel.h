// Decode against a KV cache, and RoPE applied to rows at given positions, for
// gfx950 (internal to libcgr).
//
// Decode: the Tq newest tokens of each sequence attend to its cache of L keys
// and values (their own included as the last Tq rows): query i sits at
// position L - Tq + i and sees keys j <= L - Tq + i ("Attention from
// Scratch", "Attention, the math"; GQA exists so that this cache shrinks by
// n_head / n_kv_head). The cache holds keys already rotated at their
// positions (rope_rotate_kernel below does that when rows are appended); the
// queries are rotated here at their offset positions.
//
// Work: the G * Tq query rows of one (sequence, K/V head) are the 32 columns
// of one matrix-core block (in groups of 32 when there are more), so the K/V
// rows are read once for all the heads that share them. The key range is cut
// into chunks (split-KV): one single-wave workgroup per (sequence, K/V head,
// row group, chunk) streams its chunk's K/V tiles one tile ahead (K into
// registers, V into LDS with direct loads) and keeps a classic online softmax
// per query column.
// It leaves a partial O (normalised) and its log-sum-exp; decode_combine_kernel
// merges the chunks of a row: lse = log sum_s exp(lse_s), O = sum_s
// exp(lse_s - lse) O_s. The whole path is bound by reading the cache from HBM.
#pragma once

#include "tile_common.h"

namespace cgr {

struct DecodeArgs {
  const void* q;            // [B, Tq, H, D] bf16
  const void* kc;           // bf16 rotated keys, entry (b, t, kv) at b*sb + t*st + kv*sh
  const void* vc;           // bf16 values, same layout
  const int32_t* seqlens;   // [B] cache lengths
  void* o;                  // [B, Tq, H, D] bf16
  float* lse;               // [B, H, Tq] natural log, or null
  const float* rope_cos;    // [P, D/2]
  const float* rope_sin;
  float* part_o;            // [B, H, Tq, NS, D] f32, normalised partial outputs
  float* part_lse;          // [B, H, Tq, NS] f32, log2 units
  int32_t* status;          // device error word
  long sb, st, sh;          // cache strides (elements): batch entry, token, K/V head
  int B, Tq, S, H, KV, NS, CH, RG, M;  // M: the largest cache length the call allows
  int window;               // > 0: keys 0 <= position - j < window; 0: none
  float qscale;             // scale * log2(e)
};

constexpr int kDecodeBN = 32;  // keys per tile

template <int D, int STYLE>
__global__ __launch_bounds__(64) void attn_decode_kernel(DecodeArgs a) {
  constexpr int BN = kDecodeBN, KSTEPS = D / 16, DB = D / 32;
  constexpr int TILE = BN * 2 * D;
  constexpr int LOADS = TILE / 1024 + KSTEPS;  // vector loads per tile (V to LDS, K to registers)
  // K needs no transpose: its tile goes straight into registers as the A
  // operand of S^T (lane = key row, k-step s = 16-byte chunk 2s + hh). Only V,
  // read transposed, passes through LDS, in two stages (separate arrays, so
  // the compiler sees which one a direct load writes). 16 KiB of LDS per
  // workgroup lets 8 of them share a CU, each with the next tile's 16 KiB in
  // flight while it works on the current one.
  __shared__ __attribute__((aligned(16))) char vs0[TILE], vs1[TILE];
  const int lane = threadIdx.x, l32 = lane & 31, hh = lane >> 5;
  int u = blockIdx.x;
  const int split = u % a.NS;
  u /= a.NS;
  const int rg = u % a.RG;
  u /= a.RG;
  const int kvh = u % a.KV, b = u / a.KV;
  const int L = __builtin_amdgcn_readfirstlane(a.seqlens[b]);
  // Entries with an invalid length are left alone (the combine step reports them).
  if (L < a.Tq || L > a.M) return;
  const int k0 = split * a.CH;
  if (k0 >= L) return;
  const int k1 = min(L, k0 + a.CH);
  // Sliding window: a chunk that ends before every query's window starts has
  // nothing to do (the merge skips the same chunks).
  if (a.window > 0 && k1 <= L - a.Tq - a.window + 1) return;
  const int G = a.H / a.KV;
  const int r = rg * 32 + l32;
  const bool row_ok = r < G * a.Tq;
  const int qi = row_ok ? r / G : 0, g = row_ok ? r - qi * G : 0;
  const int head = kvh * G + g, pos = L - a.Tq + qi;

  // Query row r (lane l32) as the B operand of S^T = K Q^T: k-step s of lane
  // half hh holds elements 16s + 8hh .. +7, i.e. 16-byte chunk 2s + hh. The
  // pairs of both pairings stay inside the lane (chunk c pairs with itself
  // for adjacent pairs, with chunk c + NCH/2 for the half pairing). The cache
  // is bf16, so the product is a bf16 one; the rotated, scaled query is
  // carried as two bf16 parts (hi + lo, 16 mantissa bits together) and the
  // scores take two products per k-step: their error is then the cache's own
  // rounding. The extra products are free in a kernel bound by HBM.
  u32x4 qhi[KSTEPS], qlo[KSTEPS];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + (((long)b * a.Tq + qi) * a.H + head) * D;
    float x[KSTEPS][8];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const u32x4 w[1] = {row_ok ? *(const u32x4*)(qrow + (2 * s + hh) * 8) : (u32x4){0, 0, 0, 0}};
      raw_to_f32<uint16_t>(w, x[s]);
    }
    const float* cs = a.rope_cos + (long)pos * (D / 2);
    const float* sn = a.rope_sin + (long)pos * (D / 2);
    if constexpr (STYLE == STYLE_INTERLEAVED) {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const int c = 2 * s + hh;
        const f32x4 cc = *(const f32x4*)(cs + 4 * c), ss = *(const f32x4*)(sn + 4 * c);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float x0 = x[s][2 * m], x1 = x[s][2 * m + 1];
          x[s][2 * m] = x0 * cc[m] - x1 * ss[m];
          x[s][2 * m + 1] = x0 * ss[m] + x1 * cc[m];
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < KSTEPS / 2; ++s) {
        const int c = 2 * s + hh;  // element 8c + j pairs with 8c + j + D/2 (step s + KSTEPS/2)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const f32x4 cc = *(const f32x4*)(cs + 8 * c + 4 * h2), ss = *(const f32x4*)(sn + 8 * c + 4 * h2);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int j = 4 * h2 + m;
            const float x0 = x[s][j], x1 = x[s + KSTEPS / 2][j];
            x[s][j] = x0 * cc[m] - x1 * ss[m];
            x[s + KSTEPS / 2][j] = x0 * ss[m] + x1 * cc[m];
          }
        }
      }
    }
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      float lo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[s][j] *= a.qscale;
        lo[j] = x[s][j] - (float)(__bf16)x[s][j];
      }
      qhi[s] = to_frag<OpBF16>(x[s]).v;
      qlo[s] = to_frag<OpBF16>(lo).v;
    }
  }

  // The cache of this (sequence, K/V head): rows past L read as zeros.
  const int ks = (int)a.st;  // token stride (elements)
  const long cbase = (long)b * a.sb + (long)kvh * a.sh;
  const rsrc_t rk = make_rsrc((const uint16_t*)a.kc + cbase, (uint32_t)(((L - 1) * ks + D) * 2));
  const rsrc_t rv = make_rsrc((const uint16_t*)a.vc + cbase, (uint32_t)(((L - 1) * ks + D) * 2));
  const int n_tiles = (k1 - k0 + BN - 1) / BN;
  auto issue = [&](int j, u32x4 (&kf)[KSTEPS], char* vt) {
    const int so = (k0 + j * BN) * ks * 2;
    tile_to_lds<D, BN>(rv, vt, ks * 2, so, 0, 1, lane);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) kf[s] = buf_load16(rk, l32 * ks * 2 + (2 * s + hh) * 16, so);
  };

  const TrOffsets<D> tro(lane);
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;
  const uint32_t ones_bf16 = 0x3f803f80u;
  // Key of accumulator register i: tile start + 8(i/4) + 4hh + i%4; visible
  // to this column iff below k1 and at or before the query's position.
  const int lim_all = min(k1 - 1, pos) - 4 * hh;
  const int lo_all = a.window > 0 ? pos - a.window + 1 - 4 * hh : -(1 << 30);  // and from here on

  auto tile = [&](int j, const u32x4 (&kt)[KSTEPS], const char* Vt) {
    f32x16 sacc = (f32x16){};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const Frag<OpBF16> kf = frag<OpBF16>(kt[s]);
      sacc = mma32(kf, frag<OpBF16>(qhi[s]), sacc);
      sacc = mma32(kf, frag<OpBF16>(qlo[s]), sacc);
    }
    const int lim = lim_all - (k0 + j * BN), lo = lo_all - (k0 + j * BN);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int off = 8 * (i >> 2) + (i & 3);
      if (off > lim || off < lo) sacc[i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
    const float m_new = fmaxf(m_run, pair_max(mx));
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // no visible key yet: p = 0, alpha = 1
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
    u32x4 pf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t pk = pack2(OpBF16{}, fast_exp2(sacc[8 * t + 2 * q] - m_use),
                                  fast_exp2(sacc[8 * t + 2 * q + 1] - m_use));
        pf[t][q] = pk;
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                                __builtin_bit_cast(bf16x2, ones_bf16), l_run, false);
      }
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        oacc[db] = mma32(frag<OpBF16>(tr_frag<D>(Vt, 16 * t, db, tro)), frag<OpBF16>(pf[t]), oacc[db]);
  };

  // Tile j uses V stage j % 2 and K register set j % 2; each step issues
  // the loads of tile j + 1 before waiting for tile j.
  u32x4 ka[KSTEPS], kb[KSTEPS];
  issue(0, ka, vs0);
  int j = 0;
  for (; j + 1 < n_tiles; j += 2) {
    issue(j + 1, kb, vs1);
    wait_vmem_le<LOADS>();
    tile(j, ka, vs0);
    if (j + 2 < n_tiles) {
      issue(j + 2, ka, vs0);
      wait_vmem_le<LOADS>();
    } else {
      wait_vmem_le<0>();
    }
    tile(j + 1, kb, vs1);
  }
  if (j < n_tiles) {
    wait_vmem_le<0>();
    tile(j, ka, vs0);
  }

  if (!row_ok) return;
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const long prow = (((long)b * a.H + head) * a.Tq + qi) * a.NS + split;
  float* po = a.part_o + prow * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *(f32x4*)(po + 32 * db + 8 * g4 + 4 * hh) =
          (f32x4){oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv, oacc[db][4 * g4 + 2] * inv,
                  oacc[db][4 * g4 + 3] * inv};
  if (hh == 0) a.part_lse[prow] = l_tot > 0.f ? m_run + log2f(l_tot) : -INFINITY;
}

// Merge the chunks of every (sequence, head, query) row. D/4 threads per row,
// 4 elements each. Block 0's first thread also writes the error word: 0, or 1
// when some cache length lies outside [Tq, M] (those rows are left unwritten;
// the host has checked M against the cache capacity and the tables).
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  constexpr int TPR = D / 4;
  const long t = (long)blockIdx.x * 64 + threadIdx.x;
  auto bad = [&](int L) { return L < a.Tq || L > a.M; };
  if (t == 0) {
    int code = 0;
    for (int b = 0; b < a.B; ++b)
      if (bad(a.seqlens[b])) code = 1;
    a.status[0] = code;
  }
  const long row = t / TPR;  // ((b * H + h) * Tq + i)
  const int c = (int)(t % TPR);
  if (row >= (long)a.B * a.H * a.Tq) return;
  const int i = (int)(row % a.Tq);
  const long bh = row / a.Tq;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int L = a.seqlens[b];
  if (bad(L)) return;
  const int ns = (L + a.CH - 1) / a.CH;
  // The chunks the decode kernel skipped under a sliding window.
  const int s0 = a.window > 0 ? max(0, L - a.Tq - a.window + 1) / a.CH : 0;
  const float* pl = a.part_lse + row * a.NS;
  float mx = -INFINITY;
  for (int s = s0; s < ns; ++s) mx = fmaxf(mx, pl[s]);
  float den = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const f32x4* po = (const f32x4*)(a.part_o + row * a.NS * D) + c;
#pragma unroll 4
  for (int s = s0; s < ns; ++s) {
    const float w = fast_exp2(pl[s] - mx);  // chunks with no visible key have lse -inf: w = 0
    den += w;
    acc += w * po[s * (D / 4)];
  }
  acc *= 1.f / den;
  uint16_t* orow = (uint16_t*)a.o + (((long)b * a.Tq + i) * a.H + h) * D;
  *(u32x2*)(orow + 4 * c) = (u32x2){pack2(OpBF16{}, acc[0], acc[1]), pack2(OpBF16{}, acc[2], acc[3])};
  if (a.lse != nullptr && c == 0) a.lse[((long)b * a.H + h) * a.Tq + i] = (mx + log2f(den)) * 0.69314718055994531f;
}

// RoPE on rows at given positions: out[t, h] = R(positions[t]) x[t, h] for
// x [N, nh, D]. Item = (row, group g < D/16) carrying the chunk pair
// (g, g + D/16), as in the forward's K loader. Rows whose position lies
// outside [0, P) are left unwritten and set the error word to 1 (the word is
// only ever raised here; the caller clears it).
template <int D, typename IO, int STYLE>
__global__ __launch_bounds__(256) void rope_rotate_kernel(const IO* x, IO* out, const int32_t* positions,
                                                          long n_rows, int nh, const float* cs,
                                                          const float* sn, int P, int32_t* status) {
  constexpr int IPR = D / 16;
  constexpr int W = std::is_same<IO, float>::value ? 2 : 1;
  const long tid = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = tid / IPR;
  if (row >= n_rows) return;
  const int g = (int)(tid % IPR);
  const int p = positions[row / nh];
  if (p < 0 || p >= P) {
    if (status != nullptr) status[0] = 1;
    return;
  }
  const IO* xp = x + row * D;
  u32x4 w0[W], w1[W];
#pragma unroll
  for (int k = 0; k < W; ++k) {
    w0[k] = *((const u32x4*)(xp + 8 * g) + k);
    w1[k] = *((const u32x4*)(xp + 8 * g + D / 2) + k);
  }
  float x0[8], x1[8];
  raw_to_f32<IO>(w0, x0);
  raw_to_f32<IO>(w1, x1);
  f32x4 c[2], s[2];
  load_tab<D, STYLE>(cs + (long)p * (D / 2), sn + (long)p * (D / 2), g, true, c, s);
  rope_pair<STYLE>(x0, x1, c, s);
  IO* op = out + row * D;
  if constexpr (std::is_same<IO, float>::value) {
    *(f32x4*)(op + 8 * g) = (f32x4){x0[0], x0[1], x0[2], x0[3]};
    *(f32x4*)(op + 8 * g + 4) = (f32x4){x0[4], x0[5], x0[6], x0[7]};
    *(f32x4*)(op + 8 * g + D / 2) = (f32x4){x1[0], x1[1], x1[2], x1[3]};
    *(f32x4*)(op + 8 * g + D / 2 + 4) = (f32x4){x1[4], x1[5], x1[6], x1[7]};
  } else {
    *(u32x4*)(op + 8 * g) = to_frag<OpBF16>(x0).v;
    *(u32x4*)(op + 8 * g + D / 2) = to_frag<OpBF16>(x1).v;
  }
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, int style, hipStream_t stream) {
  const unsigned grid = (unsigned)((long)a.B * a.KV * a.RG * a.NS);
  if (style == STYLE_HALF)
    hipLaunchKernelGGL((attn_decode_kernel<D, STYLE_HALF>), dim3(grid), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_decode_kernel<D, STYLE_INTERLEAVED>), dim3(grid), dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long threads = (long)a.B * a.H * a.Tq * (D / 4);
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3((unsigned)((threads + 63) / 64)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_rope_rotate_d(const void* x, void* out, const int32_t* positions, long n_rows, int nh,
                                int f32_io, const float* cs, const float* sn, int P, int style,
                                int32_t* status, hipStream_t stream) {
  const unsigned grid = (unsigned)((n_rows * (D / 16) + 255) / 256);
#define CGR_RR(IO, STY)                                                                             \
  hipLaunchKernelGGL((rope_rotate_kernel<D, IO, STY>), dim3(grid), dim3(256), 0, stream, (const IO*)x, \
                     (IO*)out, positions, n_rows, nh, cs, sn, P, status)
  if (f32_io) {
    if (style == STYLE_HALF) CGR_RR(float, STYLE_HALF); else CGR_RR(float, STYLE_INTERLEAVED);
  } else {
    if (style == STYLE_HALF) CGR_RR(uint16_t, STYLE_HALF); else CGR_RR(uint16_t, STYLE_INTERLEAVED);
  }
#undef CGR_RR
  return hipGetLastError();
}

}  // namespace cgr
