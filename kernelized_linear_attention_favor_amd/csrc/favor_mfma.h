// gfx950 register-level helpers for the MFMA kernels.
//
// Lane layouts of v_mfma_f32_32x32x16_{bf16,f16} (wave64), D = A (32x16) * B (16x32):
//   A: lane l holds A[l % 32][8 * (l / 32) + s], s = 0..7
//   B: lane l holds B[8 * (l / 32) + s][l % 32], s = 0..7
//   D: lane l holds D[8 * (i / 4) + 4 * (l / 32) + (i % 4)][l % 32], i = 0..15
// The contraction index k may be permuted freely as long as A and B use the
// same permutation; the kernels use that to feed one MFMA's output registers
// straight into the next MFMA as an operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace favor {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
// Two floats -> packed fp16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2 v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo_as_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_as_f32(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// Split fp32 pair (a, b) into hi = bf16(a, b) and lo = bf16(a - hi_a, b - hi_b):
// hi + lo carries about 16 significant bits.
__device__ __forceinline__ void split_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(a, b);
  lo = pack_bf16(a - bf16_lo_as_f32(hi), b - bf16_hi_as_f32(hi));
}

// Same split with hi = truncation of (a, b) to bf16 (exact, no rounding step):
// lo = a - hi_a is exact in fp32 and is then rounded to bf16.
__device__ __forceinline__ void split_bf16_trunc(float a, float b, uint32_t& hi, uint32_t& lo) {
  const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  hi = __builtin_amdgcn_perm(ub, ua, 0x07060302u);  // upper halves of (a, b)
  lo = pack_bf16(a - __uint_as_float(ua & 0xffff0000u), b - __uint_as_float(ub & 0xffff0000u));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// Two packed fp16 values times (s.x, s.y), rounded to fp16.  The word comes in
// by value: bit-casting a vector element in place (v[i]) reads element 0
// with this compiler.
__device__ __forceinline__ uint32_t mul_f16x2(uint32_t u, f16x2 s) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, u) * s);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Cross-lane helpers without LDS traffic (VALU permutes).
// Combine x of lane l with x of lane l ^ 32 (v_permlane32_swap): every lane
// gets the same result for the pair, computed in the same operand order.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// DPP row shift right by n within each 16-lane row; lanes shifted in get `fill`.
template <int N>
__device__ __forceinline__ float dpp_shr(float x, float fill) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), 0x110 + N,
                                                    0xf, 0xf, false));
}
// Inclusive prefix maximum over lanes 0..31 and, separately, 32..63.
__device__ __forceinline__ float prefix_max32(float x, int lane) {
  const float ninf = -__builtin_huge_valf();
  x = fmaxf(x, dpp_shr<1>(x, ninf));
  x = fmaxf(x, dpp_shr<2>(x, ninf));
  x = fmaxf(x, dpp_shr<4>(x, ninf));
  x = fmaxf(x, dpp_shr<8>(x, ninf));
  const float r15 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
  const float r47 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
  if (lane & 16) x = fmaxf(x, (lane & 32) ? r47 : r15);
  return x;
}
// Maximum over lanes 0..31, returned to every lane (a wave-uniform value);
// lanes 32..63 are assumed to hold the same values as lanes 0..31.
__device__ __forceinline__ float max32_uniform(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false)));   // lane ^ 1
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false)));   // lane ^ 2
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false)));  // 7 - lane
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xf, 0xf, false)));  // 15 - lane
  return fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)),
               __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16)));
}
// Sum over each aligned group of 8 lanes (quad swaps, then the half-row mirror).
__device__ __forceinline__ float sum8(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, false));  // lane ^ 1
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xf, 0xf, false));  // lane ^ 2
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false)); // 7 - lane
  return x;
}

// Position of feature offset f (0..15) inside a 16-wide MFMA k-block when the
// A operand comes from a 32x32 MFMA output: slots 0-3 of lane half 0 hold
// features 0-3, slots 4-7 hold 8-11; lane half 1 holds 4-7 and 12-15.
// Swapping bits 2 and 3 maps feature offset <-> slot position (an involution).
__host__ __device__ constexpr int kblock_pos(int f) {
  return (f & ~0xC) | ((f & 4) << 1) | ((f & 8) >> 1);
}

}  // namespace favor
