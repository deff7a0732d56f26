// The block's steps before attention, fused, for gfx950 (internal to libcgr):
// pre-norm RMSNorm ("The Transformer Block & the Model", section "RMSNorm:
// normalizing before every sub-layer": x / sqrt(mean(x^2) + eps) * weight),
// the bias-free q, k, v projections and RoPE on q and k ("Attention from
// Scratch", "Attention, the math": project, then rotate).
//
//   y[t, o] = rstd[t] * sum_c W[o, c] w[c] x[t, c],  rstd[t] = 1 / sqrt(mean_c x[t, c]^2 + eps)
//   q, k, v = the W_q, W_k, W_v rows of y; q and k rotated at positions[t].
//
// Two kernels:
//   * qkv_prep_kernel: rstd per token (one read of x), and W' = W diag(w)
//     rounded once to bf16 (the norm's weight folded into the projection).
//   * qkv_gemm_kernel: Y^T = W' X^T on 32x32x16 bf16 MFMAs, one lane column per
//     token, so the epilogue finds each RoPE pair inside a lane; it scales by
//     rstd, rotates, rounds once to bf16 and writes q, k, v. The normalised
//     activations never reach memory.
#pragma once

#include "tile_common.h"

namespace cgr {

struct QkvArgs {
  const void* x;             // [N, C] bf16
  const void* norm_w;        // [C] bf16
  const void* w;             // [O, C] bf16: rows of W_q, then W_k, then W_v
  const int32_t* positions;  // [N]
  void* q;                   // [N, H, D] bf16
  void* k;                   // [N, KV, D] bf16
  void* v;                   // [N, KV, D] bf16
  const float* rope_cos;     // [P, D/2]
  const float* rope_sin;
  float* rstd;               // workspace [N]
  void* wn;                  // workspace [O, C] bf16: W diag(w)
  int32_t* status;           // device error word: 1 when a position is outside [0, P)
  int N, C, H, KV, O, P;
  int rot_q, rot_k;
  float eps;
};

// rstd: one wave per token (blocks 0 .. ceil(N/4)-1); then W': 8 elements per
// thread. Block 0's first thread clears the error word (the GEMM only raises it).
template <int D>
__global__ __launch_bounds__(256) void qkv_prep_kernel(QkvArgs a) {
  const int nrb = (a.N + 3) / 4;
  if ((int)blockIdx.x < nrb) {
    if (blockIdx.x == 0 && threadIdx.x == 0) a.status[0] = 0;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= a.N) return;
    const uint16_t* row = (const uint16_t*)a.x + (long)t * a.C;
    float s = 0.f;
    for (int c = 8 * lane; c < a.C; c += 512) {
      const u32x4 w[1] = {*(const u32x4*)(row + c)};
      float f[8];
      raw_to_f32<uint16_t>(w, f);
#pragma unroll
      for (int j = 0; j < 8; ++j) s += f[j] * f[j];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
    if (lane == 0) a.rstd[t] = 1.f / sqrtf(s / (float)a.C + a.eps);
    return;
  }
  const long i8 = ((long)(blockIdx.x - nrb) * 256 + threadIdx.x) * 8;
  if (i8 >= (long)a.O * a.C) return;
  const int c = (int)(i8 % a.C);
  const u32x4 ww[1] = {*(const u32x4*)((const uint16_t*)a.w + i8)};
  const u32x4 gw[1] = {*(const u32x4*)((const uint16_t*)a.norm_w + c)};
  float f[8], g[8];
  raw_to_f32<uint16_t>(ww, f);
  raw_to_f32<uint16_t>(gw, g);
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] *= g[j];
  *(u32x4*)((uint16_t*)a.wn + i8) = to_frag<OpBF16>(f).v;
}

// RoPE on the accumulator blocks of one head (lane column = one token at
// position `pos`; block b holds the head's features 32b + 8(i/4) + 4hh + i%4):
// pair (a, b) with angle t becomes (a cos t - b sin t, a sin t + b cos t).
// Adjacent pairs sit in registers (i, i+1); half pairs (d, d + D/2) in the
// same register of block b + D/64 (or, for D = 32, of row group i/4 + 2).
template <int D, int STYLE>
__device__ __forceinline__ void rope_head(f32x16* const (&blk)[D / 32], const float* c, const float* s,
                                          int hh) {
  if constexpr (STYLE == STYLE_INTERLEAVED) {
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int p = (32 * b + 8 * g + 4 * hh) / 2;
        const f32x2 cc = *(const f32x2*)(c + p), ss = *(const f32x2*)(s + p);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const float x0 = (*blk[b])[4 * g + 2 * m], x1 = (*blk[b])[4 * g + 2 * m + 1];
          (*blk[b])[4 * g + 2 * m] = x0 * cc[m] - x1 * ss[m];
          (*blk[b])[4 * g + 2 * m + 1] = x0 * ss[m] + x1 * cc[m];
        }
      }
  } else {
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * b + 8 * g + 4 * hh;
        if (d >= D / 2) continue;
        const int b2 = D >= 64 ? b + D / 64 : b, g2 = D >= 64 ? g : g + 2;
        const f32x4 cc = *(const f32x4*)(c + d), ss = *(const f32x4*)(s + d);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float x0 = (*blk[b])[4 * g + m], x1 = (*blk[b2])[4 * g2 + m];
          (*blk[b])[4 * g + m] = x0 * cc[m] - x1 * ss[m];
          (*blk[b2])[4 * g2 + m] = x0 * ss[m] + x1 * cc[m];
        }
      }
  }
}

// Workgroup tile: 256 output features (whole heads) x 256 tokens, 8 waves of
// 128 features x 64 tokens (one workgroup per CU); K steps of KB features of x
// through LDS (direct loads, rows of 2 * KB bytes with the swizzle of
// tile_common.h): KB = 64 with two stages when the width allows (half the
// barriers of KB = 32: +6 %), else KB = 32 with three.
template <int D, int STYLE, int KB>
__global__ __launch_bounds__(512, 1) void qkv_gemm_kernel(QkvArgs a) {
  constexpr int BO = 256, BT = 256, NWV = 8;
  constexpr int NS = KB == 64 ? 2 : 3;  // LDS stages
  constexpr int AT = BO * KB * 2, BTB = BT * KB * 2;
  static_assert(128 % D == 0, "whole heads per wave");
  static_assert(KB == 32 || KB == 64, "K step");
  // Stages as separate arrays, named at compile time in the unrolled loop:
  // tile j + NS - 1 loads while tile j is multiplied.
  __shared__ __attribute__((aligned(16))) char a0[AT], a1[AT], a2[NS == 3 ? AT : 16];
  __shared__ __attribute__((aligned(16))) char b0[BTB], b1[BTB], b2[NS == 3 ? BTB : 16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int fh = wave >> 2, tw = wave & 3;  // this wave: features 128 fh .., tokens 64 tw ..
  // Tile order: consecutive workgroups go to the 8 XCDs in turn. When the
  // token tiles split evenly over the XCDs, XCD x takes token tiles
  // [x n_tt/8, (x+1) n_tt/8), walked token-fastest, so the workgroups it runs
  // at once share both their weight rows and their token rows through its L2
  // (each weight tile is fetched once per n_tt/8 token tiles instead of once
  // per token tile).
  const int n_ot = (a.O + BO - 1) / BO, n_tt = (a.N + BT - 1) / BT;
  int ot, tt;
  if ((n_tt & 7) == 0) {
    const int x = blockIdx.x & 7, kk = blockIdx.x >> 3, per = n_tt >> 3;
    ot = kk / per;
    tt = x * per + kk % per;
  } else {
    ot = blockIdx.x % n_ot;
    tt = blockIdx.x / n_ot;
  }
  const int o0 = ot * BO, t0 = tt * BT;
  const rsrc_t rw = make_rsrc(a.wn, (uint32_t)((long)a.O * a.C * 2));
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)((long)a.N * a.C * 2));
  const int nk = a.C / KB;
  auto issue = [&](int j, char* at, char* bt) {
    tile_to_lds<KB, BO>(rw, at, a.C * 2, (o0 * a.C + j * KB) * 2, wave, NWV, lane);
    tile_to_lds<KB, BT>(rx, bt, a.C * 2, (t0 * a.C + j * KB) * 2, wave, NWV, lane);
  };
  f32x16 acc[4][2];
#pragma unroll
  for (int ob = 0; ob < 4; ++ob) acc[ob][0] = acc[ob][1] = (f32x16){};
  auto compute = [&](const char* at, const char* bt) {
#pragma unroll
    for (int s = 0; s < KB / 16; ++s) {
      Frag<OpBF16> af[4], bf[2];
#pragma unroll
      for (int ob = 0; ob < 4; ++ob) af[ob] = frag<OpBF16>(row_frag<KB>(at, 128 * fh + 32 * ob + l32, s, hh));
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) bf[tb] = frag<OpBF16>(row_frag<KB>(bt, 64 * tw + 32 * tb + l32, s, hh));
#pragma unroll
      for (int ob = 0; ob < 4; ++ob)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) acc[ob][tb] = mma32(af[ob], bf[tb], acc[ob][tb]);
    }
  };
  // Step j: wait for this wave's loads of tile j (later tiles' may still be in
  // flight), barrier (tile j complete in LDS, and every wave done with tile
  // j - 1, whose stage tile j + NS - 1 then takes), issue that tile, multiply j.
  constexpr int LOADS = (AT / 1024 + BTB / 1024) / NWV;  // this wave's loads per tile
  auto step = [&](int j, const char* at, const char* bt, char* an, char* bn) {
    if (NS == 3 && j + 1 < nk)
      wait_vmem_le<LOADS>();
    else
      wait_vmem_le<0>();
    __syncthreads();
    if (j + NS - 1 < nk) issue(j + NS - 1, an, bn);
    compute(at, bt);
  };
  issue(0, a0, b0);
  if constexpr (NS == 3) {
    if (1 < nk) issue(1, a1, b1);
    for (int j = 0; j < nk; j += 3) {
      step(j, a0, b0, a2, b2);
      if (j + 1 < nk) step(j + 1, a1, b1, a0, b0);
      if (j + 2 < nk) step(j + 2, a2, b2, a1, b1);
    }
  } else {
    for (int j = 0; j < nk; j += 2) {
      step(j, a0, b0, a1, b1);
      if (j + 1 < nk) step(j + 1, a1, b1, a0, b0);
    }
  }

  // Epilogue: lane column = token; block ob = features o0 + 32 ob ...
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int t = t0 + 64 * tw + 32 * tb + l32;
    if (t >= a.N) continue;
    const int p = a.positions[t];
    if (p < 0 || p >= a.P) {
      a.status[0] = 1;
      continue;
    }
    const float r = a.rstd[t];
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) acc[ob][tb] *= r;
    const float* cs = a.rope_cos + (long)p * (D / 2);
    const float* sn = a.rope_sin + (long)p * (D / 2);
#pragma unroll
    for (int hb = 0; hb < 128 / D; ++hb) {  // heads in this wave's 128 features
      const int head = (o0 + 128 * fh + hb * D) / D;
      if (head >= a.H + 2 * a.KV) break;
      const bool is_q = head < a.H, is_k = !is_q && head < a.H + a.KV;
      if ((is_q && a.rot_q) || (is_k && a.rot_k)) {
        f32x16* blk[D / 32];
#pragma unroll
        for (int b = 0; b < D / 32; ++b) blk[b] = &acc[hb * (D / 32) + b][tb];
        rope_head<D, STYLE>(blk, cs, sn, hh);
      }
      uint16_t* dst;
      if (is_q)
        dst = (uint16_t*)a.q + ((long)t * a.H + head) * D;
      else if (is_k)
        dst = (uint16_t*)a.k + ((long)t * a.KV + head - a.H) * D;
      else
        dst = (uint16_t*)a.v + ((long)t * a.KV + head - a.H - a.KV) * D;
#pragma unroll
      for (int b = 0; b < D / 32; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& x = acc[hb * (D / 32) + b][tb];
          *(u32x2*)(dst + 32 * b + 8 * g + 4 * hh) =
              (u32x2){pack2(OpBF16{}, x[4 * g], x[4 * g + 1]), pack2(OpBF16{}, x[4 * g + 2], x[4 * g + 3])};
        }
    }
  }
}

template <int D>
hipError_t launch_qkv_d(const QkvArgs& a, int style, hipStream_t stream) {
  const long nrb = (a.N + 3) / 4, nwb = ((long)a.O * a.C / 8 + 255) / 256;
  hipLaunchKernelGGL(qkv_prep_kernel<D>, dim3((unsigned)(nrb + nwb)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)(((a.O + 255) / 256) * (long)((a.N + 255) / 256));
  const bool k64 = a.C % 64 == 0;
  if (style == STYLE_HALF) {
    if (k64)
      hipLaunchKernelGGL((qkv_gemm_kernel<D, STYLE_HALF, 64>), dim3(grid), dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((qkv_gemm_kernel<D, STYLE_HALF, 32>), dim3(grid), dim3(512), 0, stream, a);
  } else {
    if (k64)
      hipLaunchKernelGGL((qkv_gemm_kernel<D, STYLE_INTERLEAVED, 64>), dim3(grid), dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((qkv_gemm_kernel<D, STYLE_INTERLEAVED, 32>), dim3(grid), dim3(512), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace cgr
