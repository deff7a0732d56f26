// Device-side building blocks for gfx950 (CDNA4): vector types, MFMA wrappers,
// conversions and cross-lane reductions. Internal to libcgr.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace cgr {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Element tags for the matrix-product operand types.
struct OpBF16 {};
struct OpF16 {};
struct OpF32 {};

// Eight operand values of one lane for a 32x32x16 product (hardware k-slots
// 8*(lane/32) .. +7). 16-bit types are four packed dwords; f32 is eight floats.
template <typename Op>
struct Frag {
  u32x4 v;
};
template <>
struct Frag<OpF32> {
  f32x8 v;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to one packed pair of the operand type (round to nearest even).
__device__ __forceinline__ uint32_t pack2(OpBF16, float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pack2(OpF16, float a, float b) {
  f16x2 r = __builtin_convertvector((f32x2){a, b}, f16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// Eight floats -> one fragment.
template <typename Op>
__device__ __forceinline__ Frag<Op> to_frag(const float (&x)[8]) {
  Frag<Op> f;
  f.v = (u32x4){pack2(Op{}, x[0], x[1]), pack2(Op{}, x[2], x[3]), pack2(Op{}, x[4], x[5]),
                pack2(Op{}, x[6], x[7])};
  return f;
}
template <>
__device__ __forceinline__ Frag<OpF32> to_frag<OpF32>(const float (&x)[8]) {
  Frag<OpF32> f;
  f.v = (f32x8){x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return f;
}

// Range of the f16 operand: the largest finite f16 is 65504, and values of
// magnitude 65520 or more round to infinity.
constexpr float kF16Limit = 65520.f;

// max |x_i| over eight values.
__device__ __forceinline__ float absmax8(const float (&x)[8]) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
  return m;
}

// Eight floats -> one fragment; for f16, a value outside its range becomes NaN
// (not infinity), so that every score it enters is NaN whatever it is
// multiplied by, and a row that sees it ends with a NaN row sum.
template <typename Op>
__device__ __forceinline__ Frag<Op> to_frag_or_nan(const float (&x)[8]) {
  if constexpr (std::is_same<Op, OpF16>::value) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = fabsf(x[i]) < kF16Limit ? x[i] : __builtin_nanf("");
    return to_frag<Op>(y);
  } else {
    return to_frag<Op>(x);
  }
}

// bf16 hi + lo parts of eight floats: hi = x rounded to bf16, lo = (x - hi)
// rounded to bf16, so hi + lo carries 16 significant bits and f32's range.
__device__ __forceinline__ void split_bf16(const float (&x)[8], Frag<OpBF16>& hi, Frag<OpBF16>& lo) {
  float r[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t h = pack2(OpBF16{}, x[2 * i], x[2 * i + 1]);
    hi.v[i] = h;
    r[2 * i] = x[2 * i] - bf16_lo(h);
    r[2 * i + 1] = x[2 * i + 1] - bf16_hi(h);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) lo.v[i] = pack2(OpBF16{}, r[2 * i], r[2 * i + 1]);
}

// D = A(32x16) * B(16x32) + C on the matrix cores. Lane l supplies row/column
// l%32 and k-slots 8*(l/32)..+7 of A and B; the accumulator register i of lane
// l holds row 8*(i/4) + 4*(l/32) + i%4, column l%32.
__device__ __forceinline__ f32x16 mma32(const Frag<OpBF16>& a, const Frag<OpBF16>& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                 __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma32(const Frag<OpF16>& a, const Frag<OpF16>& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a.v),
                                                __builtin_bit_cast(f16x8, b.v), c, 0, 0, 0);
}
// f32: eight 32x32x2 steps; step j takes k-slot j of lanes 0-31 (k = 0) and of
// lanes 32-63 (k = 1), so the eight steps cover the same sixteen k-slots.
__device__ __forceinline__ f32x16 mma32(const Frag<OpF32>& a, const Frag<OpF32>& b, f32x16 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}

// Lanes l and l^32 exchange: returns the value of the lower-half lane and of
// the upper-half lane of the pair (same in both lanes).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Operand tiles in LDS: rows of 2*D bytes (16-bit elements), 16-byte chunks
// XOR-swizzled per row. The swizzle serves both ways the tiles are read:
//   * row reads (operand row m = lane%32, 16 bytes): the 16 lanes that share a
//     bank cycle read 16 consecutive rows at one logical chunk, which the
//     swizzle spreads over all 16 bank slots of a 256-byte line;
//   * transposing reads (ds_read_b64_tr_b16): a half-wave reads 4 consecutive
//     rows x 64 bytes, which the swizzle puts on 4 distinct 64-byte windows.
// Tiles are written by direct global->LDS loads (16 bytes per lane, lane order),
// so the swizzle is applied to the global address each lane fetches.
template <int D>
__device__ __forceinline__ int tswz(int r) {
  if constexpr (D >= 128)
    return (((r >> 1) & 1) << 3) | ((r & 1) << 2) | (((r >> 2) & 1) << 1) | (((r >> 1) ^ (r >> 3)) & 1);
  else if constexpr (D == 64)
    return (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1);
  else
    return (r >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int toff(int r, int c) {
  return r * 2 * D + 16 * (c ^ tswz<D>(r));
}


}  // namespace cgr
