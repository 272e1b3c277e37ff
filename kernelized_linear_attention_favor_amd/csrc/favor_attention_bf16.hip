// bf16-input FAVOR+ attention on gfx950 MFMA (non-causal), three kernels:
//
//   k_kv_state  : per (key-range split, b, h): Phi(K)^T [V | 1] partial sums.
//   k_merge     : per (b, h, 16 features): combine splits in fixed order,
//                 form yhat_f = S_f / z_f and beta_f = log z_f.
//   k_output    : per query tile: y_i = sum_f softmax_f(w_f.q_i + beta_f) yhat_f.
//
// The method (Performer notes: Kernel Attention View, Normalization, FAVOR+):
//   phi(x) = exp(W x - |x|^2/2) / sqrt(m);  S = Phi(K)^T V;  z = Phi(K)^T 1;
//   y_i = phi(q_i)^T S / phi(q_i)^T z.
// Exact rewrites used here (shifts that cancel in the ratio):
//   * key side: every key of a (b, h) shares the per-feature shift c_f, so
//     S_f and z_f are both carried as 2^{-c_f}-scaled sums plus c_f; the
//     1/sqrt(m) factors cancel and are dropped.
//   * query side: exp(-|q|^2/2) is a per-row constant and cancels.  Folding
//     z_f into the exponent, phi(q_i)_f z_f = exp(w_f.q_i + beta_f), so
//         y_i = sum_f exp(w_f.q_i + beta_f - M_i) yhat_f / sum_f exp(... - M_i)
//     with M_i the row maximum: a softmax over the m features.
//
// Precision plan (worst-case |y - y_ref| / max|y_ref| per (b, h) below 5e-4 on
// the measured workloads, against a 2e-3 budget):
//   * key features exp(e - c) are rounded to fp16 (11 significant bits) for
//     the S = Phi(K)^T V MFMA, with V scaled by a power of two into fp16 range
//     (exact for bf16 values); z sums the same rounded features (fp32, v_dot2),
//     so each yhat_f = S_f / z_f is an exact weighted average of the values.
//   * query softmax weights (at most 2^16, the shift being the first feature
//     tile's row maximum) go to fp16; yhat is scaled by one power of two per
//     (b, h) into (-1, 1) and goes to fp16; the denominator sums the same fp16
//     weights in fp32, so rounding of a weight moves numerator and
//     denominator together.
//   * projections w.x (+ the -|k|^2/2 or beta term, carried as three bf16
//     parts in an extra k-block) accumulate in fp32.
#include <math.h>

#include <algorithm>

#include "favor_bf16_common.h"
#include "favor_internal.h"
#include "favor_mfma.h"
#include "favor_walk.h"

namespace favor {
namespace {

using namespace bf16k;

// ---------------------------------------------------------------------------
// k_kv_state: one workgroup = NW waves, one 32-feature tile per wave, of one
// (b, h) over one contiguous key range.
//
// Per 32-key block and feature tile:
//   proj (32x32 MFMA, k = 64 d + 1 aug block) -> D[key, feature] =
//        w_f.k_j - |k_j|^2/2                    (lane = feature column)
//   phi  = exp2(D log2e - c_f) -> fp16           (c_f: per feature, the first
//                                                 tile's maximum + 8)
//   S_f += phi^T (V / sigma_v)                   (fp16 MFMA; output registers
//                                                 reused as the A operand)
//   z_f += phi                                   (the same rounded values,
//                                                 summed in fp32 by v_dot2)
// A staged 64-key tile is two blocks, software-pipelined inside the wave: the
// projection of block 1 has no dependence on block 0's exponentials, nor
// block 0's S MFMAs on block 1's, so the matrix and vector pipes of one wave
// can work side by side instead of in turn.
// sigma_v is a power of two above the first tile's largest |v|.  If anything
// overflowed (a later key or value far above the first tile's), the range is
// recomputed with c_f and sigma_v from an exact max-only pass.
// ---------------------------------------------------------------------------
constexpr int kKBuf = 2;   // staged key/value tiles (double buffering)
constexpr float kBetaNone = -1.0e30f;   // beta of a feature without keys (finite: it is split into bf16 parts)
// Per staged tile: two words per key (bf16 parts of -|k|^2/2), then one sink
// word per lane for the lanes that hold no key's norm, so that staging has no
// branch.
constexpr int kAugWords = 2 * kKT + 64;

template <int NW>
struct KvSmem {
  uint16_t k[kKBuf][kKT * kD];     // keys, bf16
  uint16_t v[kKBuf][kKT * kD];     // values / sigma_v, fp16
  uint32_t aug[kKBuf][kAugWords];  // per key: (p0 | p1 << 16, p2), the bf16 parts of -|k|^2/2
  float vred[NW];
  float zinv[NW][32];              // per wave: 1 / z_f of its features (single-range epilogue)
  int flag;
};

// 16-byte chunks of one 64-key tile (64 keys x 8 chunks) held per thread.
template <int NW>
struct KvRegs {
  static constexpr int R = (kKT * 8) / (NW * 64);
  u32x4 k[R], v[R];
};

// Global -> registers for one tile.  Keys past the end of the range are
// clamped to the last key (finite data; their weights are masked later).
// Rows are d bf16 wide (d = 32 or 64); the tile keeps 64 columns.  The
// chunks past d re-read the row's first chunk and are zeroed when staged:
// no load is predicated and nothing reads the registers before the stage, so
// the loads stay in flight for the whole step in between.
template <int NW>
__device__ __forceinline__ void load_kv(KvRegs<NW>& r, const uint16_t* Kb, const uint16_t* Vb,
                                        int tile0, int ntok, int d, int tid) {
#pragma unroll
  for (int i = 0; i < KvRegs<NW>::R; ++i) {
    const int c = tid + NW * 64 * i;
    const int tok = min(tile0 + (c >> 3), ntok - 1), ch = c & 7;
    const size_t o = static_cast<size_t>(tok) * d + (8 * ch < d ? ch * 8 : 0);
    r.k[i] = *reinterpret_cast<const u32x4*>(Kb + o);
    r.v[i] = *reinterpret_cast<const u32x4*>(Vb + o);
  }
}

// Largest |v| among the 8 bf16 values of a chunk.
__device__ __forceinline__ float chunk_absmax(const u32x4& c) {
  float m = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    m = fmaxf(m, fmaxf(fabsf(bf16_lo_as_f32(c[w])), fabsf(bf16_hi_as_f32(c[w]))));
  return m;
}

// Registers -> swizzled LDS tile: keys as given (bf16), values times vinv (a
// power of two) as fp16, plus -|k|^2/2 of each key as three bf16 parts (the 8
// threads holding a key's 8 chunks are adjacent lanes; the first two store
// the key's two words, the others their sink word).  vmx tracks the largest
// |v| staged.
template <int NW>
__device__ __forceinline__ void stage_kv(KvSmem<NW>& sm, int buf, const KvRegs<NW>& r, int tid, int d,
                                         float vinv, float& vmx) {
#pragma unroll
  for (int i = 0; i < KvRegs<NW>::R; ++i) {
    const int c = tid + NW * 64 * i;
    const int key = c >> 3, ch = c & 7;
    const bool live = 8 * ch < d;   // columns past d are zero
    const u32x4 kx = live ? r.k[i] : u32x4{0u, 0u, 0u, 0u};
    const u32x4 vx = live ? r.v[i] : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(&sm.k[buf][swz(key, ch)]) = kx;
    u32x4 vh;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      vh[w] = pack_f16(bf16_lo_as_f32(vx[w]) * vinv, bf16_hi_as_f32(vx[w]) * vinv);
    *reinterpret_cast<u32x4*>(&sm.v[buf][swz(key, ch)]) = vh;
    vmx = fmaxf(vmx, chunk_absmax(vx));
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = bf16_lo_as_f32(kx[w]), b = bf16_hi_as_f32(kx[w]);
      s = fmaf(a, a, s);
      s = fmaf(b, b, s);
    }
    s = sum8(s);
    uint32_t w01, w23;
    split3_bf16(-0.5f * s, w01, w23);
    const int slot = ch < 2 ? 2 * key + ch : 2 * kKT + (tid & 63);
    sm.aug[buf][slot] = ch == 0 ? w01 : w23;
  }
}

// Workgroup maximum of x (one barrier).  Every thread gets the result.
template <int NW>
__device__ __forceinline__ float block_max(KvSmem<NW>& sm, float x, int tid) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  if ((tid & 63) == 0) sm.vred[tid >> 6] = x;
  __syncthreads();
  float m = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) m = fmaxf(m, sm.vred[w]);
  return m;
}

// 1 / (smallest power of two above m); 1 for m = 0.
__device__ __forceinline__ float inv_pow2_above(float m) {
  int ex = 0;
  if (m > 0.f && m <= 3.0e38f) frexpf(m, &ex);
  return ldexpf(1.0f, -ex);
}

// Per-wave state of one 32-feature tile: W operand (B, lane = feature), the
// shift c_f, the running S_f (D layout, rows = features) and this lane's
// share of z_f (the keys of its half of every block; the two lanes of a
// feature column are added at the end).
struct KvFeat {
  u32x4 wB[4];
  float c;
  f32x16 sacc[2];
  float z;
};

// Lane offsets (bf16 elements from a staged tile's start) of the MFMA
// operands for the first rows; rows 16 apart share the swizzle pattern, so
// every other 16-row group is a constant offset away and the per-tile
// addresses reduce to immediates.
struct KvAddr {
  int k[4];   // projection A operand: key row `col`, chunk 2 kb + half
  int v[4];   // value B operand [2 dt + j]: key slots 8 j + 4 half + (0..3)
};

__device__ __forceinline__ KvAddr kv_addr(int lane) {
  KvAddr a;
  const int col = lane & 31, half = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) a.k[kb] = swz(col, 2 * kb + half);
  // ds_read_tr16_b64 layout (as v_operand): lane 4v+q of each 16-lane group
  // supplies 4 consecutive columns of key slot v
  const int g = lane >> 4, v = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    const int chunk = 4 * dt + 2 * (g & 1) + (q >> 1);
    a.v[2 * dt] = swz(4 * half + v, chunk) + 4 * (q & 1);
    a.v[2 * dt + 1] = swz(4 * half + v + 8, chunk) + 4 * (q & 1);
  }
  return a;
}

// Projection of the 32 keys row0 .. row0 + 31 of a staged tile on the wave's
// features: D[key, feature] = w_f.k_j - |k_j|^2/2 (lane = feature column).
__device__ __forceinline__ f32x16 kv_proj(const uint16_t* kt, const uint32_t* at, int row0, const KvAddr& ad,
                                          int col, int half, const u32x4 (&wB)[4], const u32x4 augB) {
  f32x16 acc = {};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    acc = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(kt + row0 * 64 + ad.k[kb])), as_bf16x8(wB[kb]),
                    acc);
  // the upper lane half's copy meets the zero half of augB (finite values
  // times zero add nothing), so it needs no zeroing
  const u32x2 a = *reinterpret_cast<const u32x2*>(at + 2 * (row0 + col));
  return mfma_bf16(as_bf16x8(u32x4{a[0], a[1], 0u, 0u}), as_bf16x8(augB), acc);
}

// phi = 2^(D log2e - c) of the 16 keys in registers 8 kb2 .. 8 kb2 + 7 of a
// projection, rounded to fp16 and packed as an A operand; z gets their sum.
__device__ __forceinline__ u32x4 kv_phi(const f32x16& p, int kb2, float nc, float& z) {
  const f16x2 ones = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
  u32x4 a;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t h = pack_f16(fast_exp2(fmaf(p[8 * kb2 + 2 * w], kLog2e, nc)),
                                fast_exp2(fmaf(p[8 * kb2 + 2 * w + 1], kLog2e, nc)));
    z = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, h), ones, z, false);
    a[w] = h;
  }
  return a;
}

// S += phi^T (V / sigma_v) for the 16-key group starting at key0 (a multiple
// of 16) of a staged tile; the value operand is read with the LDS transpose.
__device__ __forceinline__ void kv_sv(const uint16_t* vt, int key0, const u32x4& a, const KvAddr& ad,
                                      f32x16 (&sacc)[2]) {
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    const v4i16 ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)as_lds(vt + key0 * 64 + ad.v[2 * dt]));
    const v4i16 rb =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)as_lds(vt + key0 * 64 + ad.v[2 * dt + 1]));
    const u32x2 x = __builtin_bit_cast(u32x2, ra), y = __builtin_bit_cast(u32x2, rb);
    sacc[dt] = mfma_f16(as_f16x8(a), as_f16x8(u32x4{x[0], x[1], y[0], y[1]}), sacc[dt]);
  }
}

// Largest D log2e over 32 keys (keys at or past ntok excluded) into c.
__device__ __forceinline__ void kv_max(const f32x16& pacc, int tok_base, int ntok, int half,
                                       bool partial, float& c) {
  float mx = -kFInf;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 8 * (i >> 2) + 4 * half + (i & 3);
    if (!partial || tok_base + r < ntok) mx = fmaxf(mx, pacc[i]);
  }
  mx = pair_max(mx);
  c = fmaxf(c, mx * kLog2e);
}

// Projections of the 32 keys row0 .. row0 + 31 on FT feature tiles, the key
// operand read once for all of them.
template <int FT>
__device__ __forceinline__ void kv_proj_n(const uint16_t* kt, const uint32_t* at, int row0, const KvAddr& ad,
                                          int col, int half, const KvFeat (&fs)[FT], const u32x4 augB,
                                          f32x16 (&p)[FT]) {
  u32x4 kop[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) kop[kb] = *reinterpret_cast<const u32x4*>(kt + row0 * 64 + ad.k[kb]);
  const u32x2 a = *reinterpret_cast<const u32x2*>(at + 2 * (row0 + col));
  const u32x4 ka4 = u32x4{a[0], a[1], 0u, 0u};   // (upper half: times augB's zeros)
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    f32x16 acc = {};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) acc = mfma_bf16(as_bf16x8(kop[kb]), as_bf16x8(fs[ft].wB[kb]), acc);
    p[ft] = mfma_bf16(as_bf16x8(ka4), as_bf16x8(augB), acc);
  }
}

// S += phi^T (V / sigma_v) of FT feature tiles for the 16-key group at key0,
// the value operand read once for all of them.
template <int FT>
__device__ __forceinline__ void kv_sv_n(const uint16_t* vt, int key0, const u32x4 (&a)[FT], const KvAddr& ad,
                                        KvFeat (&fs)[FT]) {
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    const v4i16 ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)as_lds(vt + key0 * 64 + ad.v[2 * dt]));
    const v4i16 rb =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)as_lds(vt + key0 * 64 + ad.v[2 * dt + 1]));
    const u32x2 x = __builtin_bit_cast(u32x2, ra), y = __builtin_bit_cast(u32x2, rb);
    const u32x4 vop = u32x4{x[0], x[1], y[0], y[1]};
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) fs[ft].sacc[dt] = mfma_f16(as_f16x8(a[ft]), as_f16x8(vop), fs[ft].sacc[dt]);
  }
}

// One full 64-key tile, accumulating with c fixed.  One feature tile: both
// projections first, then each block's features and S update (the next
// block's projection overlaps this block's exponentials).  Two feature
// tiles: block by block, the two tiles' chains interleaving.
template <int NW, int FT>
__device__ __forceinline__ void kv_tile_acc(const KvSmem<NW>& sm, int buf, const KvAddr& ad, const u32x4 augB,
                                            KvFeat (&fs)[FT], int col, int half) {
  const uint16_t* kt = sm.k[buf];
  const uint16_t* vt = sm.v[buf];
  const uint32_t* at = sm.aug[buf];
  if constexpr (FT == 1) {
    const float nc = -fs[0].c;
    const f32x16 p0 = kv_proj(kt, at, 0, ad, col, half, fs[0].wB, augB);
    const f32x16 p1 = kv_proj(kt, at, 32, ad, col, half, fs[0].wB, augB);
    const u32x4 a0 = kv_phi(p0, 0, nc, fs[0].z);
    const u32x4 a1 = kv_phi(p0, 1, nc, fs[0].z);
    kv_sv(vt, 0, a0, ad, fs[0].sacc);
    kv_sv(vt, 16, a1, ad, fs[0].sacc);
    const u32x4 a2 = kv_phi(p1, 0, nc, fs[0].z);
    const u32x4 a3 = kv_phi(p1, 1, nc, fs[0].z);
    kv_sv(vt, 32, a2, ad, fs[0].sacc);
    kv_sv(vt, 48, a3, ad, fs[0].sacc);
  } else {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x16 p[FT];
      kv_proj_n<FT>(kt, at, 32 * st, ad, col, half, fs, augB, p);
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        u32x4 a[FT];
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) a[ft] = kv_phi(p[ft], kb2, -fs[ft].c, fs[ft].z);
        kv_sv_n<FT>(vt, 32 * st + 16 * kb2, a, ad, fs);
      }
    }
  }
}

// One 64-key tile, block by block.  MAX: only raise c.  ACC: accumulate with
// c fixed.  PARTIAL: the tile runs past the end of the key range; tail keys
// are masked.
enum { kModeMax = 1, kModeAcc = 2 };
template <int NW, int FT, int MODE, bool PARTIAL>
__device__ __forceinline__ void kv_tile(const KvSmem<NW>& sm, int buf, int tile0, int ntok, const KvAddr& ad,
                                        const u32x4 augB, KvFeat (&fs)[FT], int col, int half) {
  const uint16_t* kt = sm.k[buf];
  const uint16_t* vt = sm.v[buf];
  const uint32_t* at = sm.aug[buf];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int tok_base = tile0 + 32 * st;
    if (PARTIAL && tok_base >= ntok) break;
    f32x16 p[FT];
    kv_proj_n<FT>(kt, at, 32 * st, ad, col, half, fs, augB, p);
    if (MODE == kModeMax) {
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) kv_max(p[ft], tok_base, ntok, half, PARTIAL, fs[ft].c);
      continue;
    }
    if (PARTIAL) {
#pragma unroll
      for (int ft = 0; ft < FT; ++ft)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + 4 * half + (i & 3);
          if (tok_base + r >= ntok) p[ft][i] = -kFInf;
        }
    }
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      u32x4 a[FT];
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) a[ft] = kv_phi(p[ft], kb2, -fs[ft].c, fs[ft].z);
      kv_sv_n<FT>(vt, 32 * st + 16 * kb2, a, ad, fs);
    }
  }
}

// One step over a full tile t.  Tiles are loaded into a ring of P register
// sets, P + 1 tiles ahead of use (the loads of several tiles are in flight
// while one computes), staged into the LDS buffer the next tile reads, and
// computed from LDS.  The step stages and loads unconditionally: past the last
// tile r holds clamped copies of the last key, staged into the free buffer and
// never read.
template <int NW, int FT, int MODE, int P>
__device__ __forceinline__ void kv_step(KvSmem<NW>& sm, int t, int ntok, int d, KvRegs<NW>& r,
                                        const uint16_t* Kb, const uint16_t* Vb, const KvAddr& ad,
                                        const u32x4 augB, KvFeat (&fs)[FT], float vinv, float& vmx, int tid,
                                        int col, int half) {
  if (MODE == kModeAcc)
    kv_tile_acc<NW, FT>(sm, t & 1, ad, augB, fs, col, half);
  else
    kv_tile<NW, FT, MODE, false>(sm, t & 1, t * kKT, ntok, ad, augB, fs, col, half);
  stage_kv<NW>(sm, (t + 1) & 1, r, tid, d, vinv, vmx);
  load_kv<NW>(r, Kb, Vb, (t + P + 1) * kKT, ntok, d, tid);
  lds_barrier();
}

// Register sets in the prefetch ring (two: a deeper ring measured no faster,
// the loads of two tiles in flight already cover the compute of one).
constexpr int kKvRing = 2;

// FIRST: c is first set from tile 0 alone (a max over its keys) and the value
// scale from tile 0's largest |v|, then the range is accumulated with both
// fixed; otherwise MODE applies to every tile with the given vinv.  vmx
// returns the largest |v| of the range (MAX passes).
template <int NW, int FT, int MODE, bool FIRST>
__device__ __forceinline__ void kv_range(KvSmem<NW>& sm, const uint16_t* Kb, const uint16_t* Vb, int ntok,
                                         int d, const KvAddr& ad, const u32x4 augB, KvFeat (&fs)[FT],
                                         float& vinv, float& vmx, int tid, int lane) {
  const int ntiles = (ntok + kKT - 1) / kKT;
  if (ntiles == 0) return;   // uniform over the workgroup
  const int col = lane & 31, half = lane >> 5;
  constexpr int P = kKvRing;
  KvRegs<NW> r[P];
  load_kv<NW>(r[0], Kb, Vb, 0, ntok, d, tid);
  if (FIRST) {
    // values are staged as fp16 after scaling by 1 / sigma_v, a power of two
    // above tile 0's largest |v| (a later tile over 2^15 larger overflows
    // and sends the range to the exact pass)
    float m0 = 0.f;
#pragma unroll
    for (int i = 0; i < KvRegs<NW>::R; ++i) m0 = fmaxf(m0, chunk_absmax(r[0].v[i]));
    vinv = inv_pow2_above(block_max<NW>(sm, m0, tid));
  }
  stage_kv<NW>(sm, 0, r[0], tid, d, vinv, vmx);
#pragma unroll
  for (int j = 0; j < P; ++j) load_kv<NW>(r[j], Kb, Vb, (j + 1) * kKT, ntok, d, tid);
  lds_barrier();
  if (FIRST) {
    if (kKT <= ntok)
      kv_tile<NW, FT, kModeMax, false>(sm, 0, 0, ntok, ad, augB, fs, col, half);
    else
      kv_tile<NW, FT, kModeMax, true>(sm, 0, 0, ntok, ad, augB, fs, col, half);
    // 2^8 of headroom: fp16 features of later keys overflow only 2^24 above
    // tile 0's largest
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) fs[ft].c += 8.0f;
  }
  // full tiles P at a time (set j holds tile t + 1 + j), then the remaining
  // full tiles and the partial last tile
  const int nfull = ntok / kKT;
  int t = 0;
  for (; t + P <= nfull; t += P) {
#pragma unroll
    for (int j = 0; j < P; ++j)
      kv_step<NW, FT, MODE, P>(sm, t + j, ntok, d, r[j], Kb, Vb, ad, augB, fs, vinv, vmx, tid, col, half);
  }
#pragma unroll
  for (int j = 0; j + 1 < P; ++j) {
    if (t < nfull) {
      kv_step<NW, FT, MODE, P>(sm, t, ntok, d, r[j], Kb, Vb, ad, augB, fs, vinv, vmx, tid, col, half);
      ++t;
    }
  }
  if (t < ntiles) kv_tile<NW, FT, MODE, true>(sm, t & 1, t * kKT, ntok, ad, augB, fs, col, half);
}

// Where the state pass writes when a (b, h) has a single key range: the
// merge's outputs (yhat, beta, sigma), which need no merge then.  yhat null:
// the pass writes partial states for k_merge.
struct KvFinal {
  uint16_t* yhat;
  float* beta;
  float* sigma;
};

// Single-range epilogue: what k_merge computes from one partial, with the same
// operations in the same order (so the two routes agree bit for bit):
// sigma = the power of two above the range's largest |v|, yhat_f = S_f / z_f /
// sigma (fp16, k-block slot order), beta_f = (c_f + log2 z_f) ln 2; a masked
// feature gets yhat = 0 and the empty beta.
template <int NW, int FT>
__device__ __forceinline__ void kv_final(KvSmem<NW>& sm, const KvFeat (&fs)[FT], const KvFinal& fin, float vm,
                                         float sig, int bh, int fo, int fo0, int m, int ma, int wave, int lane,
                                         int tid) {
  const int col = lane & 31, half = lane >> 5;
  int ex = 0;
  if (vm > 0.f && vm <= 3.0e38f) frexpf(vm, &ex);
  const float sg = ldexpf(1.0f, ex);
  if (fo0 == 0 && blockIdx.y == 0 && tid < kD) fin.sigma[static_cast<size_t>(bh) * kD + tid] = sg;
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    const int f0 = fo + 32 * (FT * wave + ft);
    const float zf = pair_sum(fs[ft].z);
    const bool live = f0 + col < m && fs[ft].c != -kFInf;
    const float zt = live ? zf : 0.f;
    if (half == 0) {
      fin.beta[static_cast<size_t>(bh) * ma + f0 + col] = zt > 0.f ? (fs[ft].c + log2f(zt)) * kLn2 : kBetaNone;
      sm.zinv[wave][col] = zt > 0.f ? 1.0f / zt : 0.f;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // this wave's LDS writes (lgkmcnt(0))
    __builtin_amdgcn_wave_barrier();
    // register 4 g + j holds feature f0 + 8 g + 4 half + j; its yhat slot in
    // the 16-feature block is 8 half + 4 (g & 1) + j, so the four registers
    // of a group are four adjacent slots
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      uint16_t* yrow = fin.yhat + (static_cast<size_t>(bh) * kD + 32 * dt + col) * ma + f0 + 8 * half;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 iz = *reinterpret_cast<const f32x4*>(&sm.zinv[wave][8 * g + 4 * half]);
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int fr = f0 + 8 * g + 4 * half + j;
          // (a feature with z = 0 contributes exactly 0, as in the merge)
          const float acc = fr < m && iz[j] != 0.f ? fs[ft].sacc[dt][4 * g + j] * sig : 0.f;
          y[j] = (acc * iz[j]) / sg;
        }
        *reinterpret_cast<u32x2*>(yrow + 16 * (g >> 1) + 4 * (g & 1)) =
            u32x2{pack_f16(y[0], y[1]), pack_f16(y[2], y[3])};
      }
    }
  }
}

// NW waves of FT 32-feature tiles each cover the 32 NW FT features fo .. of a
// piece (blockIdx.y selects the piece: fo = fo0 + blockIdx.y * 32 NW FT);
// features at or past m are masked (their range state is written empty).
// The library launches FT = 1.  D is the head dimension (32 or 64): with it
// known, the staging needs no selects for dead 16-byte chunks at D = 64.
template <int NW, int FT, int D>
__global__ __launch_bounds__(NW * 64, FAVOR_KV_WAVES_PER_EU) void k_kv_state(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, const uint16_t* __restrict__ W,
    float* __restrict__ part_S, float* __restrict__ part_zc, float* __restrict__ part_vmax, KvFinal fin,
    int H, int n, int m, int ma, int fo0, int splits, int span) {
  constexpr int d = D;
  constexpr int MP = NW * 32 * FT;   // features of the piece
  __shared__ __attribute__((aligned(16))) KvSmem<NW> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int bh = blockIdx.x / splits;
  const int split = blockIdx.x - bh * splits;
  const int hh = bh % H;
  const int fo = fo0 + blockIdx.y * MP;
  const int j0 = split * span;
  const int ntok = max(0, min(n, j0 + span) - j0);
  const uint16_t* Kb = K + (static_cast<size_t>(bh) * n + j0) * d;
  const uint16_t* Vb = V + (static_cast<size_t>(bh) * n + j0) * d;
  const KvAddr ad = kv_addr(lane);

  KvFeat fs[FT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    const int f = fo + 32 * (FT * wave + ft) + col;   // B operand column of the projection
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bool live = f < m && 16 * kb + 8 * half < d;
      fs[ft].wB[kb] = live ? *reinterpret_cast<const u32x4*>(W + (static_cast<size_t>(hh) * m + f) * d +
                                                             16 * kb + 8 * half)
                           : u32x4{0u, 0u, 0u, 0u};
      // Keep W resident: an opaque definition stops the compiler from re-loading
      // it inside the key loop (whose vmcnt waits would also stall on the prefetch).
      asm volatile("" : "+v"(fs[ft].wB[kb]));
    }
    fs[ft].c = -kFInf;
    fs[ft].z = 0.f;
    fs[ft].sacc[0] = f32x16{};
    fs[ft].sacc[1] = f32x16{};
  }
  const u32x4 augB = half == 0 ? u32x4{kBf16One | (kBf16One << 16), kBf16One, 0u, 0u}
                               : u32x4{0u, 0u, 0u, 0u};

  // Pass 0 accumulates with c fixed from the first tile.  If a later key sat
  // far above that tile's maximum, phi, z or S overflowed: then a max-only
  // pass finds the exact maximum over the range and the range is accumulated
  // again with it.
  float vinv = 1.0f, vmx = 0.f;
  kv_range<NW, FT, kModeAcc, true>(sm, Kb, Vb, ntok, d, ad, augB, fs, vinv, vmx, tid, lane);
  bool bad = false;
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    bad |= !(fabsf(fs[ft].z) <= 3.0e38f);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) bad |= !(fabsf(fs[ft].sacc[dt][i]) <= 3.0e38f);
  }
  if (tid == 0) sm.flag = 0;
  __syncthreads();
  if (bad) sm.flag = 1;
  __syncthreads();
  if (sm.flag) {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      fs[ft].c = -kFInf;
      fs[ft].z = 0.f;
      fs[ft].sacc[0] = f32x16{};
      fs[ft].sacc[1] = f32x16{};
    }
    vmx = 0.f;
    kv_range<NW, FT, kModeMax, false>(sm, Kb, Vb, ntok, d, ad, augB, fs, vinv, vmx, tid, lane);
    vinv = inv_pow2_above(block_max<NW>(sm, vmx, tid));
    kv_range<NW, FT, kModeAcc, false>(sm, Kb, Vb, ntok, d, ad, augB, fs, vinv, vmx, tid, lane);
  }

  const float sig = 1.0f / vinv;
  const float vm = block_max<NW>(sm, vmx, tid);
  if (fin.yhat != nullptr) {
    kv_final<NW, FT>(sm, fs, fin, vm, sig, bh, fo, fo0, m, ma, wave, lane, tid);
    return;
  }
  // write this range's partial state (S back in value units) and its largest
  // |v|; masked features (at or past m) are written as an empty state
  const size_t base = static_cast<size_t>(bh) * splits + split;
  if (tid == 0 && blockIdx.y == 0) part_vmax[base] = vm;
  float* zc = part_zc + base * 2 * ma;
  float* Sb = part_S + base * ma * kD;
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    const int f0 = fo + 32 * (FT * wave + ft);
    const float zf = pair_sum(fs[ft].z);   // the column's two halves, in a fixed order
    if (half == 0) {
      zc[f0 + col] = f0 + col < m ? zf : 0.f;
      zc[ma + f0 + col] = f0 + col < m ? fs[ft].c : -kFInf;
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int fr = f0 + 8 * (i >> 2) + 4 * half + (i & 3);
        Sb[static_cast<size_t>(fr) * kD + 32 * dt + col] = fr < m ? fs[ft].sacc[dt][i] * sig : 0.f;
      }
  }
}

// ---------------------------------------------------------------------------
// k_merge: one workgroup per (b, h, block of 16 features); thread = (feature,
// group of 4 value columns), so 16 adjacent lanes read one 256-byte partial
// row.  Splits are combined in index order (deterministic):
//   c_f = max_s c_fs;  z_f = sum_s 2^{c_fs - c_f} z_fs;  S_f likewise;
//   yhat_f = S_f / z_f;  beta_f = (c_f + log2 z_f) ln 2  (natural-log units).
// Every yhat_f is a weighted average of the (b, h)'s values, so |yhat_f| stays
// below sigma, the power of two above the largest |v| of the (b, h) (from the
// state pass's per-range maxima).  yhat / sigma is stored as fp16, transposed
// to [dv][slot] in the slot order the output kernel's B operand reads; sigma
// goes to every column of the output kernel's per-column scale.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_merge(const float* __restrict__ part_S,
                                               const float* __restrict__ part_zc,
                                               const float* __restrict__ part_vmax,
                                               uint16_t* __restrict__ yhat,
                                               float* __restrict__ beta,
                                               float* __restrict__ sigma, int m, int splits) {
  __shared__ __attribute__((aligned(16))) uint16_t ys[kD][16];
  const int nfb = m >> 4;
  const int bh = blockIdx.x / nfb;
  const int fb = blockIdx.x - bh * nfb;
  const int t = threadIdx.x;
  const int f = 16 * fb + (t >> 4), cq = t & 15;
  const float* zc0 = part_zc + static_cast<size_t>(bh) * splits * 2 * m;
  const float* S0 = part_S + (static_cast<size_t>(bh) * splits * m + f) * kD + 4 * cq;
  float vm = 0.f, cm = -kFInf, zt = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (splits <= 8) {
    // every split's values read at once, then combined in index order
    float vs[8], cs[8], zs[8];
    f32x4 r[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s < splits) {
        vs[s] = part_vmax[static_cast<size_t>(bh) * splits + s];
        cs[s] = zc0[static_cast<size_t>(s) * 2 * m + m + f];
        zs[s] = zc0[static_cast<size_t>(s) * 2 * m + f];
        r[s] = *reinterpret_cast<const f32x4*>(S0 + static_cast<size_t>(s) * m * kD);
      } else {
        vs[s] = 0.f;
        cs[s] = -kFInf;
        zs[s] = 0.f;
        r[s] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      vm = fmaxf(vm, vs[s]);
      cm = fmaxf(cm, cs[s]);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      // an empty range (or a slot past the splits) has c = -inf and contributes nothing
      const float a = (cs[s] == -kFInf) ? 0.f : exp2f(cs[s] - cm);
      zt = fmaf(a, zs[s], zt);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) acc[cc] = fmaf(a, r[s][cc], acc[cc]);
    }
  } else {
    for (int s = 0; s < splits; ++s) {
      vm = fmaxf(vm, part_vmax[static_cast<size_t>(bh) * splits + s]);
      cm = fmaxf(cm, zc0[static_cast<size_t>(s) * 2 * m + m + f]);
    }
#pragma unroll 8
    for (int s = 0; s < splits; ++s) {
      const float cs = zc0[static_cast<size_t>(s) * 2 * m + m + f];
      const float zs = zc0[static_cast<size_t>(s) * 2 * m + f];
      const f32x4 r = *reinterpret_cast<const f32x4*>(S0 + static_cast<size_t>(s) * m * kD);
      const float a = (cs == -kFInf) ? 0.f : exp2f(cs - cm);
      zt = fmaf(a, zs, zt);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) acc[cc] = fmaf(a, r[cc], acc[cc]);
    }
  }
  int ex = 0;   // smallest power of two strictly above vm (1 for all-zero values)
  if (vm > 0.f && vm <= 3.0e38f) frexpf(vm, &ex);
  const float sg = ldexpf(1.0f, ex);
  // a feature no key reaches (masked past the feature count) gets yhat = 0 and
  // a beta so far below every other that its softmax weight is 0
  const float inv = zt > 0.f ? 1.0f / zt : 0.f;
  const int pos = kblock_pos(f & 15);
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const _Float16 hv = static_cast<_Float16>((acc[cc] * inv) / sg);
    ys[4 * cq + cc][pos] = __builtin_bit_cast(uint16_t, hv);
  }
  if (cq == 0) beta[static_cast<size_t>(bh) * m + f] = zt > 0.f ? (cm + log2f(zt)) * kLn2 : kBetaNone;
  __syncthreads();
  {
    const int c = t >> 2, q = t & 3;   // 4 slots of one column per thread
    *reinterpret_cast<u32x2*>(yhat + (static_cast<size_t>(bh) * kD + c) * m + 16 * fb + 4 * q) =
        *reinterpret_cast<const u32x2*>(&ys[c][4 * q]);
  }
  if (fb == 0 && t < kD) sigma[static_cast<size_t>(bh) * kD + t] = sg;
}

// ---------------------------------------------------------------------------
// k_state_merge: the splits of one (b, h) merged in index order into a decode
// state (same workgroup layout as k_merge): c_f = max_s c_fs, z_f and S_f the
// sums rescaled to it (S in value units).  State layout: S [BH][m][64], then
// z [BH][m], then c [BH][m], then one zero word per (b, h) (the decode
// kernel's finish counter).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_state_merge(const float* __restrict__ part_S,
                                                     const float* __restrict__ part_zc,
                                                     float* __restrict__ state, int BH, int m,
                                                     int splits) {
  const int nfb = m >> 4;
  const int bh = blockIdx.x / nfb;
  const int fb = blockIdx.x - bh * nfb;
  const int t = threadIdx.x;
  const int f = 16 * fb + (t >> 4), cq = t & 15;
  const float* zc0 = part_zc + static_cast<size_t>(bh) * splits * 2 * m;
  float cm = -kFInf;
  for (int s = 0; s < splits; ++s) cm = fmaxf(cm, zc0[static_cast<size_t>(s) * 2 * m + m + f]);
  float zt = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const float* S0 = part_S + (static_cast<size_t>(bh) * splits * m + f) * kD + 4 * cq;
#pragma unroll 8
  for (int s = 0; s < splits; ++s) {
    const float cs = zc0[static_cast<size_t>(s) * 2 * m + m + f];
    const float zs = zc0[static_cast<size_t>(s) * 2 * m + f];
    const f32x4 r = *reinterpret_cast<const f32x4*>(S0 + static_cast<size_t>(s) * m * kD);
    const float a = (cs == -kFInf) ? 0.f : exp2f(cs - cm);
    zt = fmaf(a, zs, zt);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) acc[cc] = fmaf(a, r[cc], acc[cc]);
  }
  const size_t row = static_cast<size_t>(bh) * m + f;
  *reinterpret_cast<f32x4*>(state + row * kD + 4 * cq) = acc;
  if (cq == 0) {
    state[static_cast<size_t>(BH) * m * kD + row] = zt;
    state[static_cast<size_t>(BH) * m * kD + static_cast<size_t>(BH) * m + row] = cm;
  }
  if (fb == 0 && t == 0)
    reinterpret_cast<uint32_t*>(state + static_cast<size_t>(BH) * m * (kD + 2))[bh] = 0u;
}

// ---------------------------------------------------------------------------
// k_output: 8 waves; each wave handles 32 queries at a time with all ma
// features (MT = ma / 32 tiles).  While two workgroups' LDS fit a CU (ma <=
// 288) the kernel runs at 128 VGPRs, four waves per SIMD; beyond, one
// workgroup per CU, two waves per SIMD, and each wave takes two 32-query tiles
// at a time (the W' and yhat operands read once for both).  LDS holds W' = [W |
// beta parts] (A operand of the projection; rows past m zero, their beta far
// below every other) and yhat^T (B operand of the output product) for the
// workgroup's (b, h).
//   proj: D[feature, query] = w_f.q + beta_f           (lane = query column)
//   M_i  = max_f D;  u = exp2((D - M_i) log2e) -> fp16 (A operand, k = feature)
//   num = u yhat'                                      (fp16 MFMA, fp32 acc)
//   den = sum_f u                                      (same rounded u, v_dot2)
//   y = sigma * num / den                              (the first d columns)
// The feature tiles are software-pipelined: tile ft + 1's projection is
// issued before tile ft's exponentials, which do not depend on it.
// ---------------------------------------------------------------------------
// LDS of the output kernel for MT feature tiles (W' table with its padding,
// yhat^T), and whether two workgroups fit a CU's 160 KB.
// A raw buffer over `bytes` bytes at p (stride 0: byte offsets, a store whose
// lane offset lies at or past the size is not performed; the gfx9 word-3
// format bits), and a nontemporal 4-byte store through it at a lane offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rows_rsrc(float* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, bytes, 0x00020000);
}
__device__ __forceinline__ void buffer_store_nt(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, voff, 0, 2 /* nt */);
}

constexpr int out_lds_bytes(int mt) { return (32 * mt * kWStride + 8) * 2 + kD * (32 * mt + 8) * 2 + 8 * 64 * 4; }
constexpr bool out_two_per_cu(int mt) { return 2 * out_lds_bytes(mt) <= 160 * 1024; }
constexpr int kOutWaves = 8;

template <int MT, int D>
__global__ __launch_bounds__(kOutWaves * 64, out_two_per_cu(MT) ? 4 : 2) void k_output(const uint16_t* __restrict__ Q,
                                                   const uint16_t* __restrict__ W,
                                                   const uint16_t* __restrict__ yhat,
                                                   const float* __restrict__ beta,
                                                   const float* __restrict__ sigma,
                                                   float* __restrict__ out, int H, int n,
                                                   int m, int span) {
  constexpr int mt = MT, ma = 32 * MT, d = D;
  constexpr int NWO = kOutWaves;
  constexpr int QT = out_two_per_cu(MT) ? 1 : 2;   // 32-query tiles per wave
  constexpr int YS = ma + 8;  // fp16 per staged yhat^T row
  __shared__ __attribute__((aligned(16))) uint16_t wsh[ma * kWStride + 8];   // + padding read by the last row
  __shared__ __attribute__((aligned(16))) uint16_t ysh[kD * YS];
  __shared__ __attribute__((aligned(16))) float rsh[NWO][64];   // per wave: its queries' output scales
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int nblk = (n + span - 1) / span;
  const int wg = xcd_contiguous(blockIdx.x, gridDim.x);   // the runs of one (b, h) share an L2
  const int bh = wg / nblk;
  const int blk = wg - bh * nblk;
  const int hh = bh % H;
  const int t0 = blk * span;
  const int t1 = min(n, t0 + span);

  const uint16_t* Qb = Q + static_cast<size_t>(bh) * n * d;
  float* Ob = out + static_cast<size_t>(bh) * n * d;
  const __amdgpu_buffer_rsrc_t orsrc = out_rows_rsrc(Ob + static_cast<size_t>(t0) * d, (t1 - t0) * d * 4);

  // This lane's queries (B operand column of each tile), loaded without
  // predication: rows past the end re-read the last row, and with d = 32 the
  // upper k-blocks are zero at compile time.  Everything below is per query,
  // so a row past the end computes exactly the last row's output and is
  // stored there (the same value to the same address): loads and stores carry
  // no branches, and the wait for a prefetched tile leaves the stores issued
  // after it in flight.
  auto load_q = [&](int tb, u32x4 (&qB)[QT][4]) {
#pragma unroll
    for (int q = 0; q < QT; ++q) {
      const int qt = min(tb + 32 * q + col, t1 - 1);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        qB[q][kb] = 16 * kb < D
                        ? *reinterpret_cast<const u32x4*>(Qb + static_cast<size_t>(qt) * d + 16 * kb + 8 * half)
                        : u32x4{0u, 0u, 0u, 0u};
    }
  };
  u32x4 qB[QT][4], qN[QT][4];
  int tb = t0 + 32 * QT * wave;
  if (tb < t1) load_q(tb, qB);   // the first queries, in flight during the staging below

  // stage W' and yhat^T
  for (int c = tid; c < ma * 8; c += NWO * 64) {
    const int f = c >> 3, ch = c & 7;
    *reinterpret_cast<u32x4*>(&wsh[f * kWStride + ch * 8]) =
        (f < m && 8 * ch < d) ? *reinterpret_cast<const u32x4*>(W + (static_cast<size_t>(hh) * m + f) * d + ch * 8)
                              : u32x4{0u, 0u, 0u, 0u};
  }
  for (int f = tid; f < ma; f += NWO * 64) {
    uint32_t w01, w23;
    split3_bf16(beta[static_cast<size_t>(bh) * ma + f], w01, w23);
    *reinterpret_cast<u32x4*>(&wsh[f * kWStride + 64]) = u32x4{w01, w23, 0u, 0u};
  }
  if (tid == 0) *reinterpret_cast<u32x4*>(&wsh[ma * kWStride]) = u32x4{0u, 0u, 0u, 0u};   // the padding
  for (int c = tid; c < kD * (ma / 8); c += NWO * 64) {
    const int dv = c / (ma / 8), ch = c - dv * (ma / 8);
    *reinterpret_cast<u32x4*>(&ysh[dv * YS + ch * 8]) =
        *reinterpret_cast<const u32x4*>(yhat + (static_cast<size_t>(bh) * kD + dv) * ma + ch * 8);
  }
  const float sg = sigma[static_cast<size_t>(bh) * kD];   // one value scale per (b, h)
  __syncthreads();

  const u32x4 augB = half == 0 ? u32x4{kBf16One | (kBf16One << 16), kBf16One, 0u, 0u}
                               : u32x4{0u, 0u, 0u, 0u};
  // projections of feature tile ft for the wave's query tiles: the W' operand
  // (4 k-blocks and the beta block) is read once for all of them
  auto proj = [&](int ft, const u32x4 (&qB)[QT][4], f32x16 (&pr)[QT]) {
    const uint16_t* wr = &wsh[(32 * ft + col) * kWStride + 8 * half];
    u32x4 wa[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) wa[kb] = *reinterpret_cast<const u32x4*>(wr + 16 * kb);
    // read by every lane: the upper half reads the next row's first W
    // values (the last row's, the zeroed padding past the table), finite
    // values that meet the zero half of augB and add nothing
    const u32x4 aug = *reinterpret_cast<const u32x4*>(wr + 64);
#pragma unroll
    for (int q = 0; q < QT; ++q) {
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) acc = mfma_bf16(as_bf16x8(wa[kb]), as_bf16x8(qB[q][kb]), acc);
      pr[q] = mfma_bf16(as_bf16x8(aug), as_bf16x8(augB), acc);
    }
  };
  // weights of feature tile ft -> numerators (the yhat operand read once for
  // all query tiles) and the denominators (v_dot2 over the same fp16 weights)
  const f16x2 ones2 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
  auto accumulate = [&](int ft, const f32x16 (&pr)[QT], const float (&off)[QT], f32x16 (&y0)[QT],
                        f32x16 (&y1)[QT], float (&den)[QT]) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      u32x4 a[QT];
#pragma unroll
      for (int q = 0; q < QT; ++q)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t h = pack_f16(fast_exp2(fmaf(pr[q][8 * kb2 + 2 * w], kLog2e, off[q])),
                                      fast_exp2(fmaf(pr[q][8 * kb2 + 2 * w + 1], kLog2e, off[q])));
          den[q] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, h), ones2, den[q], false);
          a[q][w] = h;
        }
      const int kpos = 32 * ft + 16 * kb2 + 8 * half;
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(&ysh[col * YS + kpos]);
#pragma unroll
      for (int q = 0; q < QT; ++q) y0[q] = mfma_f16(as_f16x8(a[q]), as_f16x8(b0), y0[q]);
      if (D > 32) {
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(&ysh[(32 + col) * YS + kpos]);
#pragma unroll
        for (int q = 0; q < QT; ++q) y1[q] = mfma_f16(as_f16x8(a[q]), as_f16x8(b1), y1[q]);
      }
    }
  };

  for (; tb < t1; tb += 32 * QT * NWO) {
    // Shift: the first feature tile's row maximum (log2 units), so the largest
    // weights sit near 1 with the whole fp16 normal range below them.  A later
    // feature more than 2^16 above it overflows fp16 and makes the
    // denominator infinite; then the tiles are redone with the exact row maxima.
    f32x16 pr[QT];
    proj(0, qB, pr);
    load_q(tb + 32 * QT * NWO, qN);  // next tiles' queries, in flight during these
    float off[QT], den[QT];
    f32x16 y0[QT], y1[QT];
#pragma unroll
    for (int q = 0; q < QT; ++q) {
      float mx = pr[q][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, pr[q][i]);
      off[q] = -pair_max(mx) * kLog2e;
      den[q] = 0.f;
      y0[q] = f32x16{};
      y1[q] = f32x16{};
    }
    accumulate(0, pr, off, y0, y1, den);
    // an opaque trip count keeps the loop rolled (fully unrolled, the
    // compiler hoists every tile's operand reads and runs out of registers)
    int nft = mt;
    asm volatile("" : "+s"(nft));
    for (int ft = 1; ft < nft; ++ft) {
      proj(ft, qB, pr);
      accumulate(ft, pr, off, y0, y1, den);
    }
    bool over = false;
#pragma unroll
    for (int q = 0; q < QT; ++q) over |= !(den[q] <= 3.0e38f);
    if (__ballot(over) != 0) {
      // exact row maxima, then redo the tiles
      float mx[QT];
#pragma unroll
      for (int q = 0; q < QT; ++q) mx[q] = -kFInf;
#pragma unroll 1
      for (int ft = 0; ft < mt; ++ft) {
        proj(ft, qB, pr);
#pragma unroll
        for (int q = 0; q < QT; ++q)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx[q] = fmaxf(mx[q], pr[q][i]);
      }
#pragma unroll
      for (int q = 0; q < QT; ++q) {
        off[q] = -pair_max(mx[q]) * kLog2e;
        den[q] = 0.f;
        y0[q] = f32x16{};
        y1[q] = f32x16{};
      }
#pragma unroll 1
      for (int ft = 0; ft < mt; ++ft) {
        proj(ft, qB, pr);
        accumulate(ft, pr, off, y0, y1, den);
      }
    }
    // each query's denominator (both lanes of its column, in a fixed order)
    // and output scale, then moved to the rows of the output layout: query r
    // sits in lane r.
    // Each store writes 128 contiguous bytes per row from 32 lanes.
#pragma unroll
    for (int q = 0; q < QT; ++q) {
      const float rq = sg * fast_rcp(pair_sum(den[q]));   // query col's output scale
      if (half == 0) rsh[wave][32 * q + col] = rq;
    }
    // (the wave's own LDS write, read back by its other lanes: in order)
    // The run's rows t0 .. t1-1 as a raw buffer: the lane's byte offset (row
    // and column) goes in the checked offset, so the stores of a partial last
    // tile's rows at or past t1 fall outside the buffer and are dropped by the
    // hardware.  The lane part is formed once per tile; a register's row
    // offset is a constant added to it.
    const uint32_t vo = static_cast<uint32_t>((tb - t0 + 4 * half) * d + col) * 4u;
#pragma unroll
    for (int q = 0; q < QT; ++q)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 sc4 = *reinterpret_cast<const f32x4*>(&rsh[wave][32 * q + 8 * g + 4 * half]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * g + j;
          const uint32_t o = vo + static_cast<uint32_t>((32 * q + 8 * g + j) * d * 4);
          buffer_store_nt(y0[q][i] * sc4[j], orsrc, o);
          if (D > 32) buffer_store_nt(y1[q][i] * sc4[j], orsrc, o + 128);
        }
      }
#pragma unroll
    for (int q = 0; q < QT; ++q)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) qB[q][kb] = qN[q][kb];
  }
}

// ---------------------------------------------------------------------------
// k_slice_combine: the causal walk's feature slices, combined per query in
// slice order: y = sum_s 2^(L_s - L) num_s / sum_s 2^(L_s - L) den_s, L = max_s
// L_s (each slice's numerator is its share of phi(q)^T S_i over its features,
// in value units, at the log2 scale L_s).  One thread per (query, 4 columns).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_slice_combine(const float* __restrict__ pnum,
                                                       const float* __restrict__ pdl, float* __restrict__ out,
                                                       long long rows, int d, int nslices) {
  const long long g = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const int cg = d >> 2;
  const long long row = g / cg;
  const int c4 = static_cast<int>(g - row * cg);
  if (row >= rows) return;
  float L = -kFInf;
  for (int s = 0; s < nslices; ++s) L = fmaxf(L, pdl[(s * rows + row) * 2 + 1]);
  float den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nslices; ++s) {
    const long long r = s * rows + row;
    const f32x2 dl = *reinterpret_cast<const f32x2*>(pdl + r * 2);
    const float wt = dl[1] == -kFInf ? 0.f : exp2f(dl[1] - L);
    den = fmaf(wt, dl[0], den);
    const f32x4 x = *reinterpret_cast<const f32x4*>(pnum + r * kD + 4 * c4);
#pragma unroll
    for (int j = 0; j < 4; ++j) num[j] = fmaf(wt, x[j], num[j]);
  }
  const float inv = 1.0f / den;
  *reinterpret_cast<f32x4*>(out + row * d + 4 * c4) = num * inv;
}

// Pieces per (b, h) when B H sequences of `items` work items each are cut
// into B H pieces workgroups, `slots` of which are resident at a time: the
// count with the fewest rounds times items per piece (ties: the fewest
// pieces).  For B H = 32 and 512 slots that is 16 pieces, one round; for
// B H = 384 it is 4, three full rounds, rather than one piece each, which
// leaves a quarter of the slots empty for the whole launch.
long long balanced_pieces(long long BH, long long items, long long slots) {
  long long best = 1, cost = -1;
  const long long top = std::min(items, std::max<long long>(1, 4 * slots / BH));
  for (long long q = 1; q <= top; ++q) {
    const long long c = ((BH * q + slots - 1) / slots) * ((items + q - 1) / q);
    if (cost < 0 || c < cost) {
      cost = c;
      best = q;
    }
  }
  return best;
}

template <int NW, int FT>
hipError_t launch_kv_piece(const Bf16Plan& p, int fo0, int pieces, const uint16_t* k, const uint16_t* v,
                           const uint16_t* W, float* pS, float* pzc, float* pvm, const KvFinal& fin,
                           hipStream_t s) {
  // the causal path runs the same kernel over its segments; it is timed under its own name
  const char* name = p.causal ? "k_causal_state" : "k_kv_state";
  const dim3 grid(p.B * p.H * p.splits, pieces), block(NW * 64);
  if (p.d == kD)
    FAVOR_LAUNCH(name, (k_kv_state<NW, FT, kD>), grid, block, 0, s, k, v, W, pS, pzc, pvm, fin, p.H, p.n, p.m,
                 p.ma, fo0, p.splits, p.span);
  else
    FAVOR_LAUNCH(name, (k_kv_state<NW, FT, 32>), grid, block, 0, s, k, v, W, pS, pzc, pvm, fin, p.H, p.n, p.m,
                 p.ma, fo0, p.splits, p.span);
  return hipGetLastError();
}

// Output kernel launch for MT feature tiles: workgroups of a contiguous run
// of query tiles each, two or one resident per CU (by LDS), as many per (b, h)
// as finish in the fewest rounds (one round at B H = 32, three full rounds
// at B H = 384: 12.6% faster than one round with a quarter of the slots empty).
template <int MT>
hipError_t launch_output(const Bf16Plan& p, const uint16_t* q, const uint16_t* W, const uint16_t* yh,
                         const float* beta, const float* sigma, float* out, hipStream_t s) {
  constexpr bool two = out_two_per_cu(MT);
  constexpr int step = 32 * (two ? 1 : 2) * kOutWaves;   // queries per workgroup iteration
  const long long BH = static_cast<long long>(p.B) * p.H;
  const long long per = balanced_pieces(BH, (p.n + step - 1) / step, two ? 512 : 256);
  long long span = (p.n + per - 1) / per;
  span = align_up(span < step ? step : span, step);
  const int nblk = static_cast<int>((p.n + span - 1) / span);
  if (p.d == 64)
    FAVOR_LAUNCH("k_output", (k_output<MT, 64>), dim3(p.B * p.H * nblk), dim3(kOutWaves * 64), 0, s, q, W, yh,
                 beta, sigma, out, p.H, p.n, p.m, static_cast<int>(span));
  else
    FAVOR_LAUNCH("k_output", (k_output<MT, 32>), dim3(p.B * p.H * nblk), dim3(kOutWaves * 64), 0, s, q, W, yh,
                 beta, sigma, out, p.H, p.n, p.m, static_cast<int>(span));
  return hipGetLastError();
}

}  // namespace

bool bf16_supported(int d, int m) {
  return (d == 32 || d == kD) && m >= 16 && m <= kMaxFeatures && m % 16 == 0;
}

bool chunk_supported(int chunk) { return chunk == 16 || chunk == 32 || chunk == 64 || chunk == 128; }

bool causal_chunks_shape(const Bf16Plan& p) {
  return p.causal && p.d == kD && p.chunk == 64 && (p.m == 64 || p.m == 128 || p.m == 256);
}

Bf16Plan bf16_plan(int B, int H, int n, int d, int m, int causal, int chunk) {
  Bf16Plan p{};
  p.B = B;
  p.H = H;
  p.n = n;
  p.d = d;
  p.m = m;
  p.ma = (m + 31) / 32 * 32;
  p.causal = causal;
  p.chunk = chunk;
  const long long BH = static_cast<long long>(B) * H;
  const int tiles = p.ma / 32;
  // causal: feature slices of at most 256 features (128 with chunks of 128),
  // in at most two groups of equal width
  p.nslices = 1;
  p.ngroups = 1;
  p.groups[0] = SliceGroup{0, 1, tiles, 0};
  if (causal) {
    const int maxw = (chunk == 128 ? 128 : 256) / 32;
    const int ns = (tiles + maxw - 1) / maxw;
    const int base = tiles / ns, extra = tiles % ns;
    p.nslices = ns;
    if (extra == 0) {
      p.groups[0] = SliceGroup{0, ns, base, 0};
    } else {
      p.ngroups = 2;
      p.groups[0] = SliceGroup{0, extra, base + 1, 0};
      p.groups[1] = SliceGroup{extra, ns - extra, base, extra * (base + 1) * 32};
    }
  }
  const long long max_splits = (n + kKT - 1) / kKT;
  long long splits;
  if (causal) {
    // one chunk-walking workgroup per CU (their LDS allows no second): as many
    // segments per (b, h) and slice as fill the 256 CUs in one round.  Rounded
    // down: one segment more would leave a second round of a few workgroups
    // that walks as long as the first.
    splits = 256 / (BH * p.nslices);
  } else {
    // about 2048 state waves (8 per CU) in one round; a range has ma/32 waves
    // over its pieces (rounded down, as above).  When B H leaves part of the
    // round empty (B H = 384 at m = 128: 384 ranges of 512), more splits in
    // fuller rounds measured no faster: each split adds a partial state that
    // the merge reads.
    const long long wgs = 2048 / tiles;
    splits = wgs / BH;
  }
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  const int al = causal && chunk > kKT ? chunk : kKT;
  const long long span = align_up((n + splits - 1) / splits, al);
  p.span = static_cast<int>(span);
  p.splits = static_cast<int>((n + span - 1) / span);
  const size_t ma = p.ma;
  size_t o = 0;
  p.off_part_S = o;
  o = align_up(o + sizeof(float) * BH * p.splits * ma * kD, 256);
  p.off_part_zc = o;
  o = align_up(o + sizeof(float) * BH * p.splits * 2 * ma, 256);
  p.off_vmax = o;
  o = align_up(o + sizeof(float) * BH * p.splits, 256);
  const size_t nc = causal ? 0 : 1;   // buffers of the non-causal merge and output
  p.off_yhat = o;
  o = align_up(o + nc * sizeof(uint16_t) * BH * kD * ma, 256);
  p.off_beta = o;
  o = align_up(o + nc * sizeof(float) * BH * ma, 256);
  p.off_sigma = o;
  o = align_up(o + nc * sizeof(float) * BH * kD, 256);
  const size_t ms = (causal && p.nslices > 1) ? p.nslices : 0;   // slice partials of the causal walk
  p.off_pnum = o;
  o = align_up(o + ms * sizeof(float) * BH * n * kD, 256);
  p.off_pdl = o;
  o = align_up(o + ms * sizeof(float) * BH * n * 2, 256);
  p.off_end = o;
  return p;
}

hipError_t launch_kv_all(const Bf16Plan& p, const uint16_t* k, const uint16_t* v, const uint16_t* W, float* pS,
                         float* pzc, float* pvm, hipStream_t s, uint16_t* yhat, float* beta, float* sigma) {
  const KvFinal fin{yhat, beta, sigma};
  // the ma / 32 feature tiles as pieces of 8, 4, 2 and 1 tiles (one wave per
  // tile: two tiles per wave, sharing the operand reads, measured slower and
  // needed twice the key ranges for the same occupancy)
  int rem = p.ma / 32, fo = 0;
  for (int nw = 8; nw >= 1; nw >>= 1) {
    const int cnt = rem / nw;
    if (cnt == 0) continue;
    hipError_t e = hipSuccess;
    switch (nw) {
      case 8: e = launch_kv_piece<8, 1>(p, fo, cnt, k, v, W, pS, pzc, pvm, fin, s); break;
      case 4: e = launch_kv_piece<4, 1>(p, fo, cnt, k, v, W, pS, pzc, pvm, fin, s); break;
      case 2: e = launch_kv_piece<2, 1>(p, fo, cnt, k, v, W, pS, pzc, pvm, fin, s); break;
      case 1: e = launch_kv_piece<1, 1>(p, fo, cnt, k, v, W, pS, pzc, pvm, fin, s); break;
    }
    if (e != hipSuccess) return e;
    fo += cnt * nw * 32;
    rem -= cnt * nw;
  }
  return hipSuccess;
}

hipError_t launch_state_bf16(const Bf16Plan& p, const uint16_t* k, const uint16_t* v,
                            const uint16_t* W, void* ws, float* state, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  float* pS = reinterpret_cast<float*>(base + p.off_part_S);
  float* pzc = reinterpret_cast<float*>(base + p.off_part_zc);
  float* pvm = reinterpret_cast<float*>(base + p.off_vmax);
  hipError_t e = launch_kv_all(p, k, v, W, pS, pzc, pvm, s);
  if (e != hipSuccess) return e;
  FAVOR_LAUNCH("k_state_merge", k_state_merge, dim3(p.B * p.H * (p.ma / 16)), dim3(256), 0, s, pS, pzc,
               state, p.B * p.H, p.ma, p.splits);
  return hipGetLastError();
}

namespace walk {

hipError_t launch_causal(const Bf16Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* W, const float* part_S, const float* part_zc, const float* vmax,
                         float* out, float* pnum, float* pdl, hipStream_t s) {
  Args a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.W = W;
  a.part_S = part_S;
  a.part_zc = part_zc;
  a.seg_vmax = vmax;
  a.out = out;
  a.pnum = pnum;
  a.pdl = pdl;
  a.BH = p.B * p.H;
  a.H = p.H;
  a.n = p.n;
  a.d = p.d;
  a.m = p.m;
  a.malloc_ = p.ma;
  a.nseg = p.splits;
  a.seglen = p.span;
  a.has_carry = p.splits > 1 ? 1 : 0;
  a.nslices = p.nslices;
  for (int g = 0; g < p.ngroups; ++g) {
    const SliceGroup& gr = p.groups[g];
    a.fbase = gr.fbase;
    a.slice0 = gr.first_slice;
    a.ms = 32 * gr.nw;
    hipError_t e = hipErrorInvalidValue;
    switch (p.chunk) {
      case 16: e = launch_walk_c16(a, gr.nw, gr.nslices, s); break;
      case 32: e = launch_walk_c32(a, gr.nw, gr.nslices, s); break;
      case 64: e = launch_walk_c64(a, gr.nw, gr.nslices, s); break;
      case 128: e = launch_walk_c128(a, gr.nw, gr.nslices, s); break;
    }
    if (e != hipSuccess) return e;
  }
  if (p.nslices > 1) {
    const long long rows = static_cast<long long>(p.B) * p.H * p.n;
    const long long threads = rows * (p.d / 4);
    FAVOR_LAUNCH("k_slice_combine", k_slice_combine, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256),
                 0, s, pnum, pdl, out, rows, p.d, p.nslices);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace walk

hipError_t launch_attention_bf16(const Bf16Plan& p, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const uint16_t* W, float* out, void* ws,
                                 hipStream_t s) {
  char* base = static_cast<char*>(ws);
  float* pS = reinterpret_cast<float*>(base + p.off_part_S);
  float* pzc = reinterpret_cast<float*>(base + p.off_part_zc);
  float* pvm = reinterpret_cast<float*>(base + p.off_vmax);
  uint16_t* yh = reinterpret_cast<uint16_t*>(base + p.off_yhat);
  float* beta = reinterpret_cast<float*>(base + p.off_beta);
  float* sigma = reinterpret_cast<float*>(base + p.off_sigma);
  hipError_t e = hipSuccess;
  // one key range per (b, h) (non-causal): the state pass writes the merge's
  // outputs itself
  const bool single = !p.causal && p.splits == 1;
  if (!p.causal || p.splits > 1) {
    if ((e = launch_kv_all(p, k, v, W, pS, pzc, pvm, s, single ? yh : nullptr, beta, sigma)) != hipSuccess)
      return e;
  }
  if (p.causal) {
    if (causal_chunks_shape(p))
      return launch_causal_chunks(p, q, k, v, W, pS, pzc, p.splits > 1 ? pvm : nullptr, out, s);
    return walk::launch_causal(p, q, k, v, W, pS, pzc, p.splits > 1 ? pvm : nullptr, out,
                               reinterpret_cast<float*>(base + p.off_pnum),
                               reinterpret_cast<float*>(base + p.off_pdl), s);
  }
  if (!single) {
    FAVOR_LAUNCH("k_merge", k_merge, dim3(p.B * p.H * (p.ma / 16)), dim3(256), 0, s, pS, pzc, pvm, yh,
                 beta, sigma, p.ma, p.splits);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
#define FAVOR_OUT_CASE(MTV) \
  case MTV: return launch_output<MTV>(p, q, W, yh, beta, sigma, out, s);
  switch (p.ma / 32) {
    FAVOR_OUT_CASE(1) FAVOR_OUT_CASE(2) FAVOR_OUT_CASE(3) FAVOR_OUT_CASE(4)
    FAVOR_OUT_CASE(5) FAVOR_OUT_CASE(6) FAVOR_OUT_CASE(7) FAVOR_OUT_CASE(8)
    FAVOR_OUT_CASE(9) FAVOR_OUT_CASE(10) FAVOR_OUT_CASE(11) FAVOR_OUT_CASE(12)
    FAVOR_OUT_CASE(13) FAVOR_OUT_CASE(14) FAVOR_OUT_CASE(15) FAVOR_OUT_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef FAVOR_OUT_CASE
  return hipGetLastError();
}

}  // namespace favor
