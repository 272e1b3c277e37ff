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
// row r stored at chunk position (c ^ ((r >> 1) & 7)).  Rows 2j and 2j + 1 are
// 32 banks apart and the eight XOR patterns shift the rest, so one chunk
// column of 16 consecutive rows covers all 64 LDS banks once (a conflict-free
// phase of a 16-byte read).  Rows 16 apart share the pattern.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3); }

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

// Lane offsets of v_operand's two reads for the key rows of a 16-key group
// starting at a multiple of 16 (rows 16 apart share the swizzle pattern, so
// the group start is an immediate offset): [dt][0] keys 0..7, [dt][1] keys 8..15.
struct VOpAddr {
  int a[2][2];
};
__device__ __forceinline__ VOpAddr vop_addr(int lane) {
  const int g = lane >> 4, v = (lane >> 2) & 3, q = lane & 3, h = lane >> 5;
  VOpAddr r;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    const int chunk = 4 * dt + 2 * (g & 1) + (q >> 1);
    r.a[dt][0] = swz(4 * h + v, chunk) + 4 * (q & 1);
    r.a[dt][1] = swz(4 * h + v + 8, chunk) + 4 * (q & 1);
  }
  return r;
}
// v_operand with precomputed lane offsets; key0 a multiple of 16.
__device__ __forceinline__ u32x4 v_operand_at(const uint16_t* vt, int key0, int dt, const VOpAddr& va) {
  const v4i16 ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)as_lds(vt + key0 * 64 + va.a[dt][0]));
  const v4i16 rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)as_lds(vt + key0 * 64 + va.a[dt][1]));
  const u32x2 a = __builtin_bit_cast(u32x2, ra), b = __builtin_bit_cast(u32x2, rb);
  return u32x4{a[0], a[1], b[0], b[1]};
}

constexpr int kWStride = 72;   // bf16 per staged W' row: 64 d + 8 beta parts (36 banks: 16 rows conflict-free)

// The chip deals a launch's workgroups to its 8 XCDs round-robin by index, and
// each XCD has its own L2.  This maps launch index b of a G-workgroup grid to a
// logical index such that every XCD gets one contiguous run of logical indices
// (the first G % 8 XCDs one more than the rest); a bijection on [0, G).  With
// the (b, h) pair as the slow part of the logical index, the workgroups of one
// sequence share an L2, and what they all read (its earlier segments' states,
// its W rows, its normalised state table) is fetched from HBM once per XCD
// instead of once per XCD that holds any of them.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_contiguous(int b, int G) {
  const int x = b % kXcds, q = G / kXcds, r = G - q * kXcds;
  return x * q + min(x, r) + b / kXcds;
}

}  // namespace bf16k
}  // namespace favor
