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
//     (exact for bf16 values); z sums the same rounded features, so each
//     yhat_f = S_f / z_f is an exact weighted average of the values.
//   * query softmax weights are in (0, 1] and go to fp16; yhat is scaled by
//     one power of two per (b, h) into (-1, 1) and goes to fp16; the denominator is
//     the same fp16 weights times 1.0, so rounding of a weight moves numerator
//     and denominator together.
//   * projections w.x (+ the -|k|^2/2 or beta term, carried as three bf16
//     parts in an extra k-block) accumulate in fp32.
#include <math.h>

#include "favor_bf16_common.h"
#include "favor_internal.h"
#include "favor_mfma.h"

namespace favor {
namespace {

using namespace bf16k;

// ---------------------------------------------------------------------------
// k_kv_state: one workgroup = NW waves of FT 32-feature tiles (all m features)
// of one (b, h) over one contiguous key range.
//
// Per 32-key tile and feature tile:
//   proj (32x32 MFMA, k = 64 d + 1 aug block) -> D[key, feature] =
//        w_f.k_j - |k_j|^2/2                    (lane = feature column)
//   phi  = exp2(D log2e - c_f) -> fp16           (c_f: per feature, the first
//                                                 tile's maximum + 8)
//   S_f += phi^T (V / sigma_v)                   (fp16 MFMA; output registers
//                                                 reused as the A operand)
//   z_f += phi                                   (same rounded values)
// sigma_v is a power of two above the first tile's largest |v|.  If anything
// overflowed (a later key or value far above the first tile's), the range is
// recomputed with c_f and sigma_v from an exact max-only pass.
// ---------------------------------------------------------------------------
constexpr int kKBuf = 2;   // staged key/value tiles (double buffering)

template <int NW>
struct KvSmem {
  uint16_t k[kKBuf][kKT * kD];     // keys, bf16
  uint16_t v[kKBuf][kKT * kD];     // values / sigma_v, fp16
  uint32_t aug[kKBuf][kKT * 2];   // per key: bf16 parts of -|k|^2/2, packed (p0 | p1 << 16, p2)
  float vred[NW];
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
template <int NW>
__device__ __forceinline__ void load_kv(KvRegs<NW>& r, const uint16_t* Kb, const uint16_t* Vb,
                                        int tile0, int ntok, int tid) {
#pragma unroll
  for (int i = 0; i < KvRegs<NW>::R; ++i) {
    const int c = tid + NW * 64 * i;
    const int tok = min(tile0 + (c >> 3), ntok - 1), ch = c & 7;
    r.k[i] = *reinterpret_cast<const u32x4*>(Kb + static_cast<size_t>(tok) * kD + ch * 8);
    r.v[i] = *reinterpret_cast<const u32x4*>(Vb + static_cast<size_t>(tok) * kD + ch * 8);
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
// threads holding a key's 8 chunks are adjacent lanes).  vmx tracks the
// largest |v| staged.
template <int NW>
__device__ __forceinline__ void stage_kv(KvSmem<NW>& sm, int buf, const KvRegs<NW>& r, int tid,
                                         float vinv, float& vmx) {
#pragma unroll
  for (int i = 0; i < KvRegs<NW>::R; ++i) {
    const int c = tid + NW * 64 * i;
    const int key = c >> 3, ch = c & 7;
    *reinterpret_cast<u32x4*>(&sm.k[buf][swz(key, ch)]) = r.k[i];
    u32x4 vh;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      vh[w] = pack_f16(bf16_lo_as_f32(r.v[i][w]) * vinv, bf16_hi_as_f32(r.v[i][w]) * vinv);
    *reinterpret_cast<u32x4*>(&sm.v[buf][swz(key, ch)]) = vh;
    vmx = fmaxf(vmx, chunk_absmax(r.v[i]));
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = bf16_lo_as_f32(r.k[i][w]), b = bf16_hi_as_f32(r.k[i][w]);
      s = fmaf(a, a, s);
      s = fmaf(b, b, s);
    }
    s = sum8(s);
    if (ch == 0) {
      uint32_t w01, w23;
      split3_bf16(-0.5f * s, w01, w23);
      *reinterpret_cast<u32x2*>(&sm.aug[buf][2 * key]) = u32x2{w01, w23};
    }
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
// shift c_f, the running z_f and S_f (D layout, rows = features).
struct KvFeat {
  u32x4 wB[4];
  float c;
  f32x16 sacc[2];
  f32x16 zacc;   // z_f in every column of D-layout row f
};

// Projection of 32 keys (rows row0 .. row0+31 of a staged tile) on one
// 32-feature tile: D[key, feature] = w_f.k_j - |k_j|^2/2 (lane = feature column).
template <int NW>
__device__ __forceinline__ f32x16 kv_proj(const KvSmem<NW>& sm, int buf, int row0, int col, int half,
                                          const u32x4 (&wB)[4], const u32x4 augB) {
  const int row = row0 + col;
  f32x16 acc = {};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    acc = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.k[buf][swz(row, 2 * kb + half)])),
                    as_bf16x8(wB[kb]), acc);
  const u32x2 a = *reinterpret_cast<const u32x2*>(&sm.aug[buf][2 * row]);
  const u32x4 ka4 = half == 0 ? u32x4{a[0], a[1], 0u, 0u} : u32x4{0u, 0u, 0u, 0u};
  return mfma_bf16(as_bf16x8(ka4), as_bf16x8(augB), acc);
}

// phi = 2^(D log2e - c) for 32 keys, rounded to fp16; S += phi^T (V / sigma_v)
// and z += phi^T 1 on fp16 MFMA from the same rounded values, so every
// S_f / z_f is an exact average of the staged values with the rounded weights.
template <int NW>
__device__ __forceinline__ void kv_accumulate(const KvSmem<NW>& sm, int buf, int row0,
                                              const f32x16& pacc, KvFeat& fs, int lane) {
  const float nc = -fs.c;
  const u32x4 ones = u32x4{kF16OnePair, kF16OnePair, kF16OnePair, kF16OnePair};
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
    u32x4 a;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float p0 = fast_exp2(fmaf(pacc[8 * kb2 + 2 * w], kLog2e, nc));
      const float p1 = fast_exp2(fmaf(pacc[8 * kb2 + 2 * w + 1], kLog2e, nc));
      a[w] = pack_f16(p0, p1);
    }
    fs.zacc = mfma_f16(as_f16x8(a), as_f16x8(ones), fs.zacc);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const u32x4 vb = v_operand(sm.v[buf], row0 + 16 * kb2, dt, lane);
      fs.sacc[dt] = mfma_f16(as_f16x8(a), as_f16x8(vb), fs.sacc[dt]);
    }
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

// One 64-key tile for the wave's FT feature tiles.  MAX: only raise c.  ACC:
// accumulate with c fixed.  PARTIAL: the tile runs past the end of the key
// range; tail keys are masked.
enum { kModeMax = 1, kModeAcc = 2 };
template <int NW, int FT, int MODE, bool PARTIAL>
__device__ __forceinline__ void kv_tile(KvSmem<NW>& sm, int buf, int tile0, int ntok,
                                        const u32x4 augB, KvFeat (&fs)[FT], int col, int half,
                                        int lane) {
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int tok_base = tile0 + 32 * st;
    if (PARTIAL && tok_base >= ntok) break;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      f32x16 pacc = kv_proj(sm, buf, 32 * st, col, half, fs[ft].wB, augB);
      if (MODE == kModeMax) {
        kv_max(pacc, tok_base, ntok, half, PARTIAL, fs[ft].c);
        continue;
      }
      if (PARTIAL) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + 4 * half + (i & 3);
          if (tok_base + r >= ntok) pacc[i] = -kFInf;
        }
      }
      kv_accumulate(sm, buf, 32 * st, pacc, fs[ft], lane);
    }
  }
}

// One pass over the key range.  Tiles are loaded into registers two tiles
// ahead of use (one tile of compute does not cover the load latency), staged
// into the LDS buffer the next tile reads, and computed from LDS.
template <int NW, int FT, int MODE>
__device__ __forceinline__ void kv_step(KvSmem<NW>& sm, int t, int ntiles, int ntok,
                                        KvRegs<NW>& r, const uint16_t* Kb, const uint16_t* Vb,
                                        const u32x4 augB, KvFeat (&fs)[FT], float vinv, float& vmx,
                                        int tid, int lane) {
  // Lane-dependent LDS addresses are recomputed per tile rather than held in
  // loop-invariant registers.
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int lcol = ln & 31, lhalf = ln >> 5;
  kv_tile<NW, FT, MODE, false>(sm, t & 1, t * kKT, ntok, augB, fs, lcol, lhalf, ln);
  // r holds tile t + 1: stage it, then reuse r for tile t + 3.  The load is
  // issued on every path (past the end it re-reads the clamped last key), so
  // the wait before the next stage can leave the other tile's load in flight.
  if (t + 1 < ntiles) stage_kv<NW>(sm, (t + 1) & 1, r, tid, vinv, vmx);
  load_kv<NW>(r, Kb, Vb, (t + 3) * kKT, ntok, tid);
  lds_barrier();
}

// FIRST: c is first set from tile 0 alone (a max over its keys) and the value
// scale from tile 0's largest |v|, then the range is accumulated with both
// fixed; otherwise MODE applies to every tile with the given vinv.  vmx
// returns the largest |v| of the range (MAX passes).
template <int NW, int FT, int MODE, bool FIRST>
__device__ __forceinline__ void kv_range(KvSmem<NW>& sm, const uint16_t* Kb, const uint16_t* Vb,
                                         int ntok, const u32x4 augB, KvFeat (&fs)[FT], float& vinv,
                                         float& vmx, int tid, int lane) {
  const int ntiles = (ntok + kKT - 1) / kKT;
  if (ntiles == 0) return;   // uniform over the workgroup
  KvRegs<NW> ra, rb;
  load_kv<NW>(ra, Kb, Vb, 0, ntok, tid);
  if (FIRST) {
    // values are staged as fp16 after scaling by 1 / sigma_v, a power of two
    // above tile 0's largest |v| (a later tile over 2^15 larger overflows
    // and sends the range to the exact pass)
    float m0 = 0.f;
#pragma unroll
    for (int i = 0; i < KvRegs<NW>::R; ++i) m0 = fmaxf(m0, chunk_absmax(ra.v[i]));
    vinv = inv_pow2_above(block_max<NW>(sm, m0, tid));
  }
  stage_kv<NW>(sm, 0, ra, tid, vinv, vmx);
  load_kv<NW>(ra, Kb, Vb, kKT, ntok, tid);
  load_kv<NW>(rb, Kb, Vb, 2 * kKT, ntok, tid);
  lds_barrier();
  if (FIRST) {
    const int col = lane & 31, half = lane >> 5;
    if (kKT <= ntok)
      kv_tile<NW, FT, kModeMax, false>(sm, 0, 0, ntok, augB, fs, col, half, lane);
    else
      kv_tile<NW, FT, kModeMax, true>(sm, 0, 0, ntok, augB, fs, col, half, lane);
    // 2^8 of headroom: fp16 features of later keys overflow only 2^24 above
    // tile 0's largest
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) fs[ft].c += 8.0f;
  }
  // full tiles in pairs (ra holds the odd tiles, rb the even ones), then at
  // most one more full tile and the partial last tile
  const int nfull = ntok / kKT;
  int t = 0;
  for (; t + 2 <= nfull; t += 2) {
    kv_step<NW, FT, MODE>(sm, t, ntiles, ntok, ra, Kb, Vb, augB, fs, vinv, vmx, tid, lane);
    kv_step<NW, FT, MODE>(sm, t + 1, ntiles, ntok, rb, Kb, Vb, augB, fs, vinv, vmx, tid, lane);
  }
  if (t < nfull) {
    kv_step<NW, FT, MODE>(sm, t, ntiles, ntok, ra, Kb, Vb, augB, fs, vinv, vmx, tid, lane);
    ++t;
  }
  if (t < ntiles)
    kv_tile<NW, FT, MODE, true>(sm, t & 1, t * kKT, ntok, augB, fs, lane & 31, lane >> 5, lane);
}

// NW waves of FT 32-feature tiles each cover all m = 32 NW FT features.  The
// library launches FT = 1: with FT = 2 (half the waves, so that two workgroups
// share a CU) the kernel does not fit its register budget without spills.
template <int NW, int FT>
__global__ __launch_bounds__(NW * 64, FT == 1 ? FAVOR_KV_WAVES_PER_EU : 2) void k_kv_state(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, const uint16_t* __restrict__ W,
    float* __restrict__ part_S, float* __restrict__ part_zc, float* __restrict__ part_vmax, int H,
    int n, int splits, int span) {
  constexpr int M = NW * 32 * FT;
  __shared__ __attribute__((aligned(16))) KvSmem<NW> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int bh = blockIdx.x / splits;
  const int split = blockIdx.x - bh * splits;
  const int hh = bh % H;
  const int j0 = split * span;
  const int ntok = max(0, min(n, j0 + span) - j0);
  const uint16_t* Kb = K + (static_cast<size_t>(bh) * n + j0) * kD;
  const uint16_t* Vb = V + (static_cast<size_t>(bh) * n + j0) * kD;

  KvFeat fs[FT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    const int f = 32 * (FT * wave + ft) + col;   // B operand column of the projection
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      fs[ft].wB[kb] = *reinterpret_cast<const u32x4*>(W + (static_cast<size_t>(hh) * M + f) * kD +
                                                      16 * kb + 8 * half);
      // Keep W resident: an opaque definition stops the compiler from re-loading
      // it inside the key loop (whose vmcnt waits would also stall on the prefetch).
      asm volatile("" : "+v"(fs[ft].wB[kb]));
    }
    fs[ft].c = -kFInf;
    fs[ft].zacc = f32x16{};
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
  kv_range<NW, FT, kModeAcc, true>(sm, Kb, Vb, ntok, augB, fs, vinv, vmx, tid, lane);
  bool bad = false;
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
#pragma unroll
    for (int i = 0; i < 16; ++i) bad |= !(fabsf(fs[ft].zacc[i]) <= 3.0e38f);
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
      fs[ft].zacc = f32x16{};
      fs[ft].sacc[0] = f32x16{};
      fs[ft].sacc[1] = f32x16{};
    }
    vmx = 0.f;
    kv_range<NW, FT, kModeMax, false>(sm, Kb, Vb, ntok, augB, fs, vinv, vmx, tid, lane);
    vinv = inv_pow2_above(block_max<NW>(sm, vmx, tid));
    kv_range<NW, FT, kModeAcc, false>(sm, Kb, Vb, ntok, augB, fs, vinv, vmx, tid, lane);
  }

  // write this range's partial state (S back in value units) and its largest |v|
  const float sig = 1.0f / vinv;
  const size_t base = static_cast<size_t>(bh) * splits + split;
  {
    const float vm = block_max<NW>(sm, vmx, tid);
    if (tid == 0) part_vmax[base] = vm;
  }
  float* zc = part_zc + base * 2 * M;
  float* Sb = part_S + base * M * kD;
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    const int f0 = 32 * (FT * wave + ft);
    if (half == 0) zc[M + f0 + col] = fs[ft].c;
    if (col == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) zc[f0 + 8 * (i >> 2) + 4 * half + (i & 3)] = fs[ft].zacc[i];
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int fr = f0 + 8 * (i >> 2) + 4 * half + (i & 3);
        Sb[static_cast<size_t>(fr) * kD + 32 * dt + col] = fs[ft].sacc[dt][i] * sig;
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
  const float inv = 1.0f / zt;
  const int pos = kblock_pos(f & 15);
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const _Float16 hv = static_cast<_Float16>((acc[cc] * inv) / sg);
    ys[4 * cq + cc][pos] = __builtin_bit_cast(uint16_t, hv);
  }
  if (cq == 0) beta[static_cast<size_t>(bh) * m + f] = (cm + log2f(zt)) * kLn2;
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
// k_output: 4 waves; each wave handles 32 queries at a time with all m
// features.  LDS holds W' = [W | beta parts] (A operand of the projection)
// and yhat^T (B operand of the output product) for the workgroup's (b, h).
//   proj: D[feature, query] = w_f.q + beta_f           (lane = query column)
//   M_i  = max_f D;  u = exp2((D - M_i) log2e) -> fp16 (A operand, k = feature)
//   [num | den] = u [yhat' | 1]                        (fp16 MFMA, fp32 acc)
//   y = sigma * num / den
// ---------------------------------------------------------------------------
template <int MT>
__global__ __launch_bounds__(256, 2) void k_output(const uint16_t* __restrict__ Q,
                                                   const uint16_t* __restrict__ W,
                                                   const uint16_t* __restrict__ yhat,
                                                   const float* __restrict__ beta,
                                                   const float* __restrict__ sigma,
                                                   float* __restrict__ out, int H, int n,
                                                   int span) {
  constexpr int M = 32 * MT;
  constexpr int YS = M + 8;  // fp16 per staged yhat^T row
  __shared__ __attribute__((aligned(16))) uint16_t wsh[M * kWStride];
  __shared__ __attribute__((aligned(16))) uint16_t ysh[kD * YS];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int nblk = (n + span - 1) / span;
  const int bh = blockIdx.x / nblk;
  const int blk = blockIdx.x - bh * nblk;
  const int hh = bh % H;
  const int t0 = blk * span;
  const int t1 = min(n, t0 + span);

  // stage W' and yhat^T
  for (int c = tid; c < M * 8; c += 256) {
    const int f = c >> 3, ch = c & 7;
    *reinterpret_cast<u32x4*>(&wsh[f * kWStride + ch * 8]) =
        *reinterpret_cast<const u32x4*>(W + (static_cast<size_t>(hh) * M + f) * kD + ch * 8);
  }
  for (int f = tid; f < M; f += 256) {
    uint32_t w01, w23;
    split3_bf16(beta[static_cast<size_t>(bh) * M + f], w01, w23);
    *reinterpret_cast<u32x4*>(&wsh[f * kWStride + 64]) = u32x4{w01, w23, 0u, 0u};
    *reinterpret_cast<u32x4*>(&wsh[f * kWStride + 72]) = u32x4{0u, 0u, 0u, 0u};
  }
  for (int c = tid; c < kD * (M / 8); c += 256) {
    const int dv = c / (M / 8), ch = c - dv * (M / 8);
    *reinterpret_cast<u32x4*>(&ysh[dv * YS + ch * 8]) =
        *reinterpret_cast<const u32x4*>(yhat + (static_cast<size_t>(bh) * kD + dv) * M + ch * 8);
  }
  const float sg0 = sigma[static_cast<size_t>(bh) * kD + col];
  const float sg1 = sigma[static_cast<size_t>(bh) * kD + 32 + col];
  __syncthreads();

  const u32x4 augB = half == 0 ? u32x4{kBf16One | (kBf16One << 16), kBf16One, 0u, 0u}
                               : u32x4{0u, 0u, 0u, 0u};
  const u32x4 onesB = u32x4{kF16OnePair, kF16OnePair, kF16OnePair, kF16OnePair};
  const uint16_t* Qb = Q + static_cast<size_t>(bh) * n * kD;
  float* Ob = out + static_cast<size_t>(bh) * n * kD;

  auto load_q = [&](int tb, u32x4 (&qB)[4]) {
    const int qt = tb + col;  // this lane's query (B operand column)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      qB[kb] = (qt < t1) ? *reinterpret_cast<const u32x4*>(Qb + static_cast<size_t>(qt) * kD +
                                                            16 * kb + 8 * half)
                         : u32x4{0u, 0u, 0u, 0u};
  };
  u32x4 qB[4], qN[4];
  int tb = t0 + 32 * wave;
  if (tb < t1) load_q(tb, qB);
  for (; tb < t1; tb += 128) {
    // Shift: the first feature tile's row maximum (log2 units), so the largest
    // weights sit near 1 with the whole fp16 normal range below them.  A later
    // feature more than 2^15 above it would overflow fp16; that case is
    // detected and the tile is redone with the exact row maximum.
    f32x16 pa = out_proj(wsh, 0, col, half, qB, augB);
    if (tb + 128 < t1) load_q(tb + 128, qN);  // next tile's queries, in flight during this one
    float mx = pa[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, pa[i]);
    mx = pair_max(mx);
    float off = -mx * kLog2e;
    f32x16 yacc0 = {}, yacc1 = {}, dacc = {};
    float tmax = -kFInf;
    out_accumulate(pa, off, 0, ysh, YS, col, half, onesB, yacc0, yacc1, dacc, tmax);
#pragma unroll 1
    for (int ft = 1; ft < MT; ++ft) {
      const f32x16 pn = out_proj(wsh, ft, col, half, qB, augB);
      out_accumulate(pn, off, ft, ysh, YS, col, half, onesB, yacc0, yacc1, dacc, tmax);
    }
    if (__ballot(tmax > 15.0f) != 0) {
      // exact row maximum, then redo the tile
      mx = -kFInf;
#pragma unroll 1
      for (int ft = 0; ft < MT; ++ft) {
        const f32x16 pa = out_proj(wsh, ft, col, half, qB, augB);
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, pa[i]);
      }
      mx = pair_max(mx);
      off = -mx * kLog2e;
      yacc0 = f32x16{};
      yacc1 = f32x16{};
      dacc = f32x16{};
#pragma unroll 1
      for (int ft = 0; ft < MT; ++ft) {
        const f32x16 pa = out_proj(wsh, ft, col, half, qB, augB);
        out_accumulate(pa, off, ft, ysh, YS, col, half, onesB, yacc0, yacc1, dacc, tmax);
      }
    }
    float* orow = Ob + static_cast<size_t>(tb) * kD;
    if (tb + 32 <= t1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + 4 * half + (i & 3);
        const float inv = fast_rcp(dacc[i]);
        __builtin_nontemporal_store(yacc0[i] * sg0 * inv, orow + row * kD + col);
        __builtin_nontemporal_store(yacc1[i] * sg1 * inv, orow + row * kD + 32 + col);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + 4 * half + (i & 3);
        if (tb + row < t1) {
          const float inv = fast_rcp(dacc[i]);
          orow[row * kD + col] = yacc0[i] * sg0 * inv;
          orow[row * kD + 32 + col] = yacc1[i] * sg1 * inv;
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) qB[kb] = qN[kb];
  }
}

template <int NW, int FT>
hipError_t launch_kv(const Bf16Plan& p, const uint16_t* k, const uint16_t* v, const uint16_t* W,
                     float* pS, float* pzc, float* pvm, hipStream_t s) {
  // the causal path runs the same kernel over its segments; it is timed under its own name
  FAVOR_LAUNCH(p.causal ? "k_causal_state" : "k_kv_state", (k_kv_state<NW, FT>),
               dim3(p.B * p.H * p.splits), dim3(NW * 64), 0, s, k, v, W, pS, pzc, pvm, p.H, p.n,
               p.splits, p.span);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_out(const Bf16Plan& p, const uint16_t* q, const uint16_t* W, const uint16_t* yh,
                      const float* beta, const float* sigma, float* out, int span,
                      hipStream_t s) {
  const int nblk = (p.n + span - 1) / span;
  FAVOR_LAUNCH("k_output", k_output<MT>, dim3(p.B * p.H * nblk), dim3(256), 0, s, q, W, yh, beta, sigma,
                     out, p.H, p.n, span);
  return hipGetLastError();
}

}  // namespace

bool bf16_supported(int d, int m) { return d == kD && (m == 64 || m == 128 || m == 256); }

Bf16Plan bf16_plan(int B, int H, int n, int d, int m, int causal) {
  Bf16Plan p{};
  p.B = B;
  p.H = H;
  p.n = n;
  p.d = d;
  p.m = m;
  p.causal = causal;
  const long long BH = static_cast<long long>(B) * H;
  const long long max_splits = (n + kKT - 1) / kKT;
  long long splits;
  if (causal) {
    // one chunk-walking workgroup per CU: segments per (b, h)
    splits = (256 + BH - 1) / BH;
  } else {
    // about 2048 state waves (8 per CU); a workgroup has m/32 waves
    const long long wgs = 2048 / (m / 32);
    splits = (wgs + BH - 1) / BH;
  }
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  const long long span = align_up((n + splits - 1) / splits, kKT);
  p.span = static_cast<int>(span);
  p.splits = static_cast<int>((n + span - 1) / span);
  size_t o = 0;
  p.off_part_S = o;
  o = align_up(o + sizeof(float) * BH * p.splits * m * kD, 256);
  p.off_part_zc = o;
  o = align_up(o + sizeof(float) * BH * p.splits * 2 * m, 256);
  p.off_vmax = o;
  o = align_up(o + sizeof(float) * BH * p.splits, 256);
  p.off_yhat = o;
  o = align_up(o + sizeof(uint16_t) * BH * kD * m, 256);
  p.off_beta = o;
  o = align_up(o + sizeof(float) * BH * m, 256);
  p.off_sigma = o;
  o = align_up(o + sizeof(float) * BH * kD, 256);
  p.off_end = o;
  return p;
}

hipError_t launch_state_bf16(const Bf16Plan& p, const uint16_t* k, const uint16_t* v,
                            const uint16_t* W, void* ws, float* state, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  float* pS = reinterpret_cast<float*>(base + p.off_part_S);
  float* pzc = reinterpret_cast<float*>(base + p.off_part_zc);
  float* pvm = reinterpret_cast<float*>(base + p.off_vmax);
  hipError_t e = hipSuccess;
  switch (p.m) {
    case 64: e = launch_kv<2, 1>(p, k, v, W, pS, pzc, pvm, s); break;
    case 128: e = launch_kv<4, 1>(p, k, v, W, pS, pzc, pvm, s); break;
    case 256: e = launch_kv<8, 1>(p, k, v, W, pS, pzc, pvm, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  FAVOR_LAUNCH("k_state_merge", k_state_merge, dim3(p.B * p.H * (p.m / 16)), dim3(256), 0, s, pS, pzc,
               state, p.B * p.H, p.m, p.splits);
  return hipGetLastError();
}

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
  if (!p.causal || p.splits > 1) {
    switch (p.m) {
      case 64: e = launch_kv<2, 1>(p, k, v, W, pS, pzc, pvm, s); break;
      case 128: e = launch_kv<4, 1>(p, k, v, W, pS, pzc, pvm, s); break;
      case 256: e = launch_kv<8, 1>(p, k, v, W, pS, pzc, pvm, s); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  if (p.causal) {
    return launch_causal_chunks(p, q, k, v, W, pS, pzc, p.splits > 1 ? pvm : nullptr, out, s);
  }
  FAVOR_LAUNCH("k_merge", k_merge, dim3(p.B * p.H * (p.m / 16)), dim3(256), 0, s, pS, pzc, pvm, yh,
               beta, sigma, p.m, p.splits);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // output: about 512 workgroups, each a contiguous run of query tiles
  const long long BH = static_cast<long long>(p.B) * p.H;
  long long per = (512 + BH - 1) / BH;
  long long span = (p.n + per - 1) / per;
  span = align_up(span < 128 ? 128 : span, 128);
  switch (p.m) {
    case 64: return launch_out<2>(p, q, W, yh, beta, sigma, out, static_cast<int>(span), s);
    case 128: return launch_out<4>(p, q, W, yh, beta, sigma, out, static_cast<int>(span), s);
    case 256: return launch_out<8>(p, q, W, yh, beta, sigma, out, static_cast<int>(span), s);
  }
  return hipErrorInvalidValue;
}

}  // namespace favor
