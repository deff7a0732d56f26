// Shared device helpers of the backward and decode kernels (internal to
// libcgr): 16-bit operand tiles in LDS written by direct global->LDS loads and
// read both row-wise and transposed, and the accumulator epilogues (transposed
// rotation, bf16 stores).
#pragma once

#include "attn_fwd_kernel.h"

namespace cgr {

// Load `rows` rows (row r of the tile at global byte offset r * gstride + soff)
// into an LDS tile, by the `nw` waves of a group; `wig` is this wave's index in
// the group. Rows past the buffer's range read as zeros.
template <int D, int ROWS>
__device__ __forceinline__ void tile_to_lds(rsrc_t rs, char* lds, int gstride, int soff, int wig,
                                            int nw, int lane) {
  constexpr int NCH = D / 8;
  constexpr int NI = ROWS * NCH / 64;  // 1 KiB wave loads
  static_assert(ROWS * NCH % 64 == 0, "whole wave loads");
  for (int u = wig; u < NI; u += nw) {
    const int slot = u * 64 + lane, r = slot / NCH, pc = slot % NCH;
    buf_load16_lds(rs, lds + u * 1024, r * gstride + 16 * (pc ^ tswz<D>(r)), soff);
  }
}

// The same copy for a group of NWG waves with its per-lane global offsets
// worked out once (they depend on the lane, the wave's index in the group and
// the row stride only): a loop that copies tile after tile then issues just
// the loads, each with the tile's scalar offset.
template <int D, int ROWS, int NWG>
struct TileCopy {
  static constexpr int NCH = D / 8;
  static constexpr int NI = ROWS * NCH / 64;         // 1 KiB wave loads
  static constexpr int PER = (NI + NWG - 1) / NWG;   // loads per wave, at most
  static_assert(ROWS * NCH % 64 == 0, "whole wave loads");
  int wig;
  int voff[PER];
  __device__ __forceinline__ bool has(int k) const { return NI % NWG == 0 || wig + k * NWG < NI; }
  __device__ __forceinline__ TileCopy(int wig_, int gstride, int lane) : wig(wig_) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int slot = (wig + k * NWG) * 64 + lane, r = slot / NCH, pc = slot % NCH;
      voff[k] = r * gstride + 16 * (pc ^ tswz<D>(r));
    }
  }
  __device__ __forceinline__ void operator()(rsrc_t rs, char* lds, int soff) const {
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (has(k)) buf_load16_lds(rs, lds + (wig + k * NWG) * 1024, voff[k], soff);
  }
};

// Operand fragment k-step s of row r (lane half hh): elements 16s + 8hh .. +7.
template <int D>
__device__ __forceinline__ u32x4 row_frag(const char* tile, int r, int s, int hh) {
  return *(const u32x4*)(tile + toff<D>(r, 2 * s + hh));
}

// Per-lane offsets of the transposing reads. For 16 tile rows starting at a
// multiple of 16 and the 32-wide column block db, lane (hh, gi, li) reads row
// 4hh + li/4 (first half) and 8 rows further (second half), 8 bytes at logical
// chunk 4db + 2(gi&1) + (li&3)/2, half li&1. The pair of reads is the
// operand fragment A[m][k] = X[row(k)][32db + m]: with k-slot 8hh + j it
// holds row 8(j/4) + 4hh + j%4 of the 16, the row order of the accumulator
// registers 8t..8t+7 that the B operand comes from.
template <int D>
struct TrOffsets {
  int a[D / 32], b[D / 32];
  __device__ __forceinline__ TrOffsets(int lane) {
    const int hh = lane >> 5, gi = lane >> 4, li = lane & 15;
    const int ra = 4 * hh + (li >> 2), rb = ra + 8;
    const int cs = 2 * (gi & 1) + ((li & 3) >> 1), half = 8 * (li & 1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      a[db] = ra * 2 * D + 16 * ((4 * db + cs) ^ tswz<D>(ra)) + half;
      b[db] = rb * 2 * D + 16 * ((4 * db + cs) ^ tswz<D>(rb)) + half;
    }
  }
};
template <int D>
__device__ __forceinline__ u32x4 tr_frag(const char* tile, int row16, int db, const TrOffsets<D>& o) {
  const char* p = tile + row16 * 2 * D;
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + o.a[db]));
  const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + o.b[db]));
  const u32x2 ux = __builtin_bit_cast(u32x2, x), uy = __builtin_bit_cast(u32x2, y);
  return (u32x4){ux[0], ux[1], uy[0], uy[1]};
}

template <typename Op>
__device__ __forceinline__ Frag<Op> frag(u32x4 v) {
  Frag<Op> f;
  f.v = v;
  return f;
}

// The transposed rotation applied to an accumulator whose lane column sits at
// position `pos` and whose registers hold rows d = 32db + 8(i/4) + 4hh + i%4:
// pair (a, b) with angle t becomes (a cos t + b sin t, -a sin t + b cos t).
// Pairs lie inside the lane for both pairings: (d, d+1) are registers i, i+1;
// (d, d + D/2) are the same register of block db + D/64 (or, for D = 32, of
// row group i/4 + 2).
template <int D, int STYLE>
__device__ __forceinline__ void rope_transpose_acc(f32x16 (&acc)[D / 32], const float* cs,
                                                   const float* sn, int pos, int hh) {
  const float* c = cs + (long)pos * (D / 2);
  const float* s = sn + (long)pos * (D / 2);
  if constexpr (STYLE == STYLE_INTERLEAVED) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int p = (32 * db + 8 * g + 4 * hh) / 2;
        const f32x2 cc = *(const f32x2*)(c + p), ss = *(const f32x2*)(s + p);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const float a = acc[db][4 * g + 2 * m], b = acc[db][4 * g + 2 * m + 1];
          acc[db][4 * g + 2 * m] = a * cc[m] + b * ss[m];
          acc[db][4 * g + 2 * m + 1] = -a * ss[m] + b * cc[m];
        }
      }
  } else {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * db + 8 * g + 4 * hh;
        if (d >= D / 2) continue;  // compile-time per (db, g) up to hh
        const int db2 = D >= 64 ? db + D / 64 : db, g2 = D >= 64 ? g : g + 2;
        const f32x4 cc = *(const f32x4*)(c + d), ss = *(const f32x4*)(s + d);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float a = acc[db][4 * g + m], b = acc[db2][4 * g2 + m];
          acc[db][4 * g + m] = a * cc[m] + b * ss[m];
          acc[db2][4 * g2 + m] = -a * ss[m] + b * cc[m];
        }
      }
  }
}

// Round an accumulator (lane column = row `pos` of a [.., D] bf16 tensor) to
// bf16 and store it: 8 bytes (4 consecutive elements) per (db, row group).
template <int D>
__device__ __forceinline__ void store_acc_bf16(const f32x16 (&acc)[D / 32], float mul, rsrc_t r,
                                               int row_off, int hh) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * db + 8 * g + 4 * hh;
      const u32x2 w = {pack2(OpBF16{}, acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul),
                       pack2(OpBF16{}, acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul)};
      __builtin_amdgcn_raw_buffer_store_b64(w, r, row_off + d * 2, 0, 0);
    }
}

// Store an accumulator as f32 (lane column = row `pos` of a [.., D] f32
// tensor): 16 bytes (4 consecutive elements) per (db, row group).
template <int D>
__device__ __forceinline__ void store_acc_f32(const f32x16 (&acc)[D / 32], rsrc_t r, int row_off, int hh) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * db + 8 * g + 4 * hh;
      const f32x4 w = {acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), r, row_off + d * 4, 0, 0);
    }
}

}  // namespace cgr
