// Device helpers shared by the bf16-input MFMA kernels (non-causal and causal).
#pragma once

#include <math.h>

#include "favor_internal.h"
#include "favor_mfma.h"

namespace favor {
namespace bf16k {

constexpr int kD = 64;          // head dimension supported by the MFMA path
constexpr int kKT = 64;         // key tokens staged per iteration (two 32-token MFMA tiles)
constexpr uint32_t kBf16One = 0x3f80u;
constexpr uint32_t kF16OnePair = 0x3c003c00u;   // fp16 (1.0, 1.0)
constexpr float kFInf = __builtin_huge_valf();

// Waves per SIMD the state kernel is compiled for (register budget 512 / this).
#ifndef FAVOR_KV_WAVES_PER_EU
#define FAVOR_KV_WAVES_PER_EU 2
#endif

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Three bf16 parts whose sum carries x to about 24 bits.
__device__ __forceinline__ void split3_bf16(float x, uint32_t& w01, uint32_t& w23) {
  const uint32_t p0 = pack_bf16(x, 0.f);
  const float r1 = x - bf16_lo_as_f32(p0);
  const uint32_t p1 = pack_bf16(r1, 0.f);
  const float r2 = r1 - bf16_lo_as_f32(p1);
  const uint32_t p2 = pack_bf16(r2, 0.f);
  w01 = (p0 & 0xffffu) | (p1 << 16);
  w23 = p2 & 0xffffu;
}

// Staged tiles are dense 64 x 64 bf16 (128 B rows) with the 16-byte chunks of
// row r stored at chunk position (c ^ (r & 7)), which spreads the rows of a
// column of chunks over the LDS banks.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
// Generic pointer into __shared__ memory -> LDS address space (addrspacecast).
__device__ __forceinline__ lds_void* as_lds(const void* p) { return (lds_void*)(p); }

// Workgroup barrier for LDS hand-off only: waits for this wave's LDS accesses,
// then s_barrier.  Unlike __syncthreads() it carries no memory fence, so
// global loads still in flight (the next tile's prefetch) are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maximum
  __builtin_amdgcn_s_barrier();
}

// B operand (k = key slot, n = value column) for a 16-key k-block, read with
// the LDS transpose instruction from the row-major tile: within each group of
// 16 lanes, lane 4v+q supplies 4 consecutive columns of key slot v, and lane
// 4q+j receives column 4q+j of the 4 keys.  Two reads give the 8 slots.
__device__ __forceinline__ u32x4 v_operand(const uint16_t* vt, int key0, int dt, int lane) {
  const int g = lane >> 4, v = (lane >> 2) & 3, q = lane & 3, h = lane >> 5;
  const int chunk = 4 * dt + 2 * (g & 1) + (q >> 1);
  const int ka = key0 + 4 * h + v, kb = ka + 8;
  const uint16_t* pa = vt + swz(ka, chunk) + 4 * (q & 1);
  const uint16_t* pb = vt + swz(kb, chunk) + 4 * (q & 1);
  const v4i16 ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)as_lds(pa));
  const v4i16 rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)as_lds(pb));
  const u32x2 a = __builtin_bit_cast(u32x2, ra), b = __builtin_bit_cast(u32x2, rb);
  return u32x4{a[0], a[1], b[0], b[1]};
}

constexpr int kWStride = 80;   // bf16 per staged W' row: 64 d + 8 beta parts + 8 zero

// Projection of one 32-feature tile: D[feature, query] = w_f.q + beta_f.
__device__ __forceinline__ f32x16 out_proj(const uint16_t* wsh, int ft, int col, int half,
                                           const u32x4 (&qB)[4], const u32x4 augB) {
  f32x16 acc = {};
  const uint16_t* wr = &wsh[(32 * ft + col) * kWStride + 8 * half];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    acc = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(wr + 16 * kb)), as_bf16x8(qB[kb]),
                    acc);
  return mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(wr + 64)), as_bf16x8(augB), acc);
}

// Softmax weights of one feature tile -> fp16 A operand -> numerator and
// denominator MFMAs.  tmax tracks the largest exponent used (log2 units).
__device__ __forceinline__ void out_accumulate(const f32x16& pa, float off, int ft,
                                               const uint16_t* ysh, int YS, int col, int half,
                                               const u32x4 onesB, f32x16& yacc0, f32x16& yacc1,
                                               f32x16& dacc, float& tmax) {
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
    u32x4 a;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float e0 = fmaf(pa[8 * kb2 + 2 * w], kLog2e, off);
      const float e1 = fmaf(pa[8 * kb2 + 2 * w + 1], kLog2e, off);
      tmax = fmaxf(tmax, fmaxf(e0, e1));
      a[w] = pack_f16(fast_exp2(e0), fast_exp2(e1));
    }
    const int kpos = 32 * ft + 16 * kb2 + 8 * half;
    const u32x4 b0 = *reinterpret_cast<const u32x4*>(&ysh[col * YS + kpos]);
    const u32x4 b1 = *reinterpret_cast<const u32x4*>(&ysh[(32 + col) * YS + kpos]);
    yacc0 = mfma_f16(as_f16x8(a), as_f16x8(b0), yacc0);
    yacc1 = mfma_f16(as_f16x8(a), as_f16x8(b1), yacc1);
    dacc = mfma_f16(as_f16x8(a), as_f16x8(onesB), dacc);
  }
}

}  // namespace bf16k
}  // namespace favor
