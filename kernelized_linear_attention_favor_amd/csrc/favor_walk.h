// Causal FAVOR+ attention on gfx950: the chunk walk (prefix-sum form).
//
// The method (Performer for vision, How It Works, Step 2; Performer notes,
// Normalization): query i aggregates keys j <= i,
//     y_i = phi(q_i)^T S_i / phi(q_i)^T z_i,  S_i = sum_{j<=i} phi(k_j) v_j^T,
//     z_i = sum_{j<=i} phi(k_j),   phi(x) = exp(W x - |x|^2/2) / sqrt(m).
// Each (b, h) sequence is cut into segments, one workgroup each; the segment
// states (S, z and a per-feature shift c of the segment's own keys) come from
// the state pass (k_kv_state).  A workgroup first merges the states of the
// segments before its own, in index order, into its carry, then walks its
// segment in chunks of C tokens.  For chunk t, query i sums
//   carry  the keys before the chunk: phi(q_i)^T S and phi(q_i)^T z as a
//          softmax over features with weights phi(q_i)_f z_f and values
//          yhat_f = S_f / z_f, and
//   chunk  sum_{j in t, j <= i} (phi(q_i)^T phi(k_j)) v_j and its weights,
// then the chunk's keys join the state: S += Phi(K_t)^T V_t, z += Phi(K_t)^T 1.
// Factors common to a row (exp(-|q_i|^2/2), 1/sqrt(m)) cancel and are left out.
//
// Work split: wave w owns 32 features f of the slice for both sides of the
// chunk.  Its key features (one projection, one exponential per key and
// feature) serve the state update and, read back transposed from the wave's
// own LDS area, the chunk's kernel matrix; its state S_f lives in its
// registers and is, divided by z_f, the carry's value operand directly.  Each
// wave thus forms a partial numerator, denominator and log2 scale per query
// over its own features; the partials meet in LDS and are combined in wave
// order.  With more than 256 features (128 for C = 128) the features are cut
// into slices, one workgroup each, whose partials a last kernel combines.
//
// Shifts (log2 units, e_jf = log2e (w_f.k_j - |k_j|^2/2), a_if = log2e w_f.q_i):
//   * keys: S_f and z_f are carried times 2^-c_f; c_f is raised to the chunk's
//     largest e_jf when that exceeds it by more than 2^8 (the state is
//     rescaled), so key features 2^(e_jf - c_f) are at most 2^8;
//   * queries: u_if = 2^(a_if + c_f - s_i), s_i = max_f (a_if + c_f) over the
//     wave's features, so the kernel matrix is P_ij = 2^s_i sum_f u_if
//     2^(e_jf - c_f); the carry weights 2^(a_if + gam_f - mc_i) (gam_f =
//     c_f + log2 z_f of the state before the chunk, mc_i their row maximum)
//     go with the normalised values yhat_f;
//   * both terms are brought to the row scale L_i = max(mc_i, s_i + log2
//     max_j P_ij) before they enter the fp16 products.
// When a chunk's keys in some feature spread more than 2^60 below that
// feature's shift while the state there is empty or far below it, early rows
// could see only keys that fall out of range; the wave then forms that
// chunk's kernel matrix from the projections in fp32, each row scaled by its
// own largest visible term (the slow path).  When a row's carry weights
// would all fall below 2^-60 of u, they are taken from the projections too.
//
// Precision: key features enter the state update as fp16 against values
// scaled by a power of two into fp16 (exact for bf16 values), and z sums the
// same rounded features, so yhat_f is an exact weighted average; query and key
// features of the kernel matrix are bf16 hi + lo pairs (about 16 bits, with
// fp32's exponent range); the carry weights, yhat and the row-normalised
// kernel matrix are fp16; all products accumulate in fp32.
#pragma once

#include <math.h>

#include "favor_bf16_common.h"
#include "favor_internal.h"
#include "favor_mfma.h"

namespace favor {
namespace walk {

using namespace bf16k;

constexpr float kSpreadLimit = 60.f;   // log2 units: see the fast-path condition above

template <int C>
struct Cfg {
  static constexpr int T = C >= 32 ? C / 32 : 1;   // 32-row tiles per chunk
  static constexpr int R = C >= 32 ? 32 : C;       // rows of a tile inside the chunk
  static constexpr int NWMAX = C >= 128 ? 4 : 8;   // waves (32-feature tiles) per slice
};

template <int C>
struct Smem {
  static constexpr int T = Cfg<C>::T, NWM = Cfg<C>::NWMAX;
  uint16_t k[T][32 * 64];              // key tiles, bf16, 64-column swizzled rows (d = 32: upper half 0)
  uint16_t v[T][32 * 64];              // values / sigma_v, fp16
  uint16_t q[T][32 * 64];              // query tiles, bf16
  uint32_t kaug[T * 32][2];            // per key: -|k|^2/2 as three bf16 parts
  uint32_t tr[NWM][32 * 32 * T];       // per wave: key features [feature][key] bf16 hi then lo
                                       // (32 x 32T each); slow path: fp32 e_jf [feature][key]
  float np[NWM][32 * 64];              // per wave: partial numerators of one query tile
  float dp[NWM][32];                   // ... denominators
  float lp[NWM][32];                   // ... log2 scales
  float xs[NWM][32];                   // per wave: per-feature scalars, lane -> register layout
  float xs2[NWM][32];
  float iz[NWM][32];                   // per wave: 1/z_f of the state (feature order)
  float cp[NWM][32];                   // per wave: the chunk's key shift c'_f (feature order)
};

// Row of D-layout register i of a 32 x 32 MFMA tile for lane half `half`.
__device__ __forceinline__ int drow(int i, int half) { return 8 * (i >> 2) + 4 * half + (i & 3); }

// The 8 registers of k-block kb (16 rows) of a D-layout f32x16, two per word.
__device__ __forceinline__ u32x4 pack_kblock_f16(const f32x16& x, int kb, float s) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) r[w] = pack_f16(x[8 * kb + 2 * w] * s, x[8 * kb + 2 * w + 1] * s);
  return r;
}

// Key feature area of one wave: row f (a feature) holds the chunk's 32T keys
// as bf16; its 8-byte units (4 keys) are XOR-swizzled by f & 7.
template <int T>
__device__ __forceinline__ int tr_unit(int f, int u) { return f * (8 * T) + (u ^ (f & 7)); }

// A operand (rows = 32 keys of tile kt, k = 16 features of k-block kb) from a
// wave's [feature][key] area, by the LDS transpose read: lane 4v+q of each
// 16-lane group points at feature row base + v, keys 4q .. 4q+3 of the group's
// 16 keys, and receives the 4 features of its own key.
template <int T>
__device__ __forceinline__ u32x4 tr_operand(const uint32_t* area, int kt, int kb, int lane) {
  const int g = lane >> 4, v = (lane >> 2) & 3, q = lane & 3, h = lane >> 5;
  const int u = 8 * kt + 4 * (g & 1) + q;
  const int fa = 16 * kb + 4 * h + v, fb = fa + 8;
  const uint16_t* base = reinterpret_cast<const uint16_t*>(area);
  const v4i16 ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)as_lds(base + 4 * tr_unit<T>(fa, u)));
  const v4i16 rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)as_lds(base + 4 * tr_unit<T>(fb, u)));
  const u32x2 x = __builtin_bit_cast(u32x2, ra), y = __builtin_bit_cast(u32x2, rb);
  return u32x4{x[0], x[1], y[0], y[1]};
}

struct Args {
  const uint16_t *q, *k, *v, *W;
  const float *part_S, *part_zc, *seg_vmax;
  float* out;      // y [BH][n][d] (one slice)
  float* pnum;     // several slices: partial numerators [nslices][BH][n][64], value units
  float* pdl;      // ... denominators and log2 scales [nslices][BH][n][2]
  int BH, H, n, d, m, malloc_;   // malloc_: features per state row (m rounded up to 32)
  int nseg, seglen, has_carry;
  int fbase, slice0, nslices, ms;   // launch's first feature and slice, slices over m, features per slice
};

// Global -> registers for the chunk at token t0 (rows past the segment end
// re-read its last token; their weights are masked).  Thread c of NT loads
// 16-byte pieces c, c + NT, ... of the chunk's K, V and Q rows.
template <int C, int NT>
struct Regs {
  static constexpr int TILE = Cfg<C>::T * 32;          // staged rows (whole tiles)
  static constexpr int P = (TILE * 8 + NT - 1) / NT;   // pieces per thread
  u32x4 k[P], v[P], q[P];
};

template <int C, int NT>
__device__ __forceinline__ void load_chunk(Regs<C, NT>& r, const uint16_t* Kb, const uint16_t* Vb, const uint16_t* Qb,
                                           int t0, int ntok, int d, int tid) {
  constexpr int TILE = Regs<C, NT>::TILE;
#pragma unroll
  for (int i = 0; i < Regs<C, NT>::P; ++i) {
    const int c = tid + NT * i;
    const int row = c >> 3, ch = c & 7;
    const bool live = c < TILE * 8 && 8 * ch < d;
    const size_t off = static_cast<size_t>(min(t0 + min(row, Cfg<C>::R - 1 + 32 * (row >> 5)), ntok - 1)) * d + 8 * ch;
    r.k[i] = live ? *reinterpret_cast<const u32x4*>(Kb + off) : u32x4{0u, 0u, 0u, 0u};
    r.v[i] = live ? *reinterpret_cast<const u32x4*>(Vb + off) : u32x4{0u, 0u, 0u, 0u};
    r.q[i] = live ? *reinterpret_cast<const u32x4*>(Qb + off) : u32x4{0u, 0u, 0u, 0u};
  }
}

// Registers -> LDS tiles (values times vinv as fp16) and -|k|^2/2 per key as
// three bf16 parts (the 8 threads holding a key's row are adjacent lanes).
template <int C, int NT>
__device__ __forceinline__ void stage_chunk(Smem<C>& sm, const Regs<C, NT>& r, float vinv, int tid) {
  constexpr int TILE = Regs<C, NT>::TILE;
#pragma unroll
  for (int i = 0; i < Regs<C, NT>::P; ++i) {
    const int c = tid + NT * i;
    if (c >= TILE * 8) break;
    const int row = c >> 3, ch = c & 7, kt = row >> 5, rr = row & 31;
    *reinterpret_cast<u32x4*>(&sm.k[kt][swz(rr, ch)]) = r.k[i];
    *reinterpret_cast<u32x4*>(&sm.q[kt][swz(rr, ch)]) = r.q[i];
    u32x4 vh;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      vh[w] = pack_f16(bf16_lo_as_f32(r.v[i][w]) * vinv, bf16_hi_as_f32(r.v[i][w]) * vinv);
    *reinterpret_cast<u32x4*>(&sm.v[kt][swz(rr, ch)]) = vh;
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
      *reinterpret_cast<u32x2*>(&sm.kaug[row][0]) = u32x2{w01, w23};
    }
  }
}

// D[key, feature] = w_f.k_j - |k_j|^2/2 for the 32 keys of tile kt (lane =
// feature column, registers = keys).
template <int C>
__device__ __forceinline__ f32x16 key_proj(const Smem<C>& sm, int kt, int col, int half, const u32x4 (&wB)[4],
                                           const u32x4 augB) {
  f32x16 acc = {};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    acc = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.k[kt][swz(col, 2 * kb + half)])),
                    as_bf16x8(wB[kb]), acc);
  const u32x2 a = *reinterpret_cast<const u32x2*>(&sm.kaug[32 * kt + col][0]);
  const u32x4 ka4 = half == 0 ? u32x4{a[0], a[1], 0u, 0u} : u32x4{0u, 0u, 0u, 0u};
  return mfma_bf16(as_bf16x8(ka4), as_bf16x8(augB), acc);
}

// D[feature, query] = w_f.q_i + c_f ln 2 for the 32 queries of tile qt (lane
// = query column, registers = features); qaug carries c_f ln 2 as three bf16
// parts in the feature rows' extra k-block.
template <int C>
__device__ __forceinline__ f32x16 query_proj(const Smem<C>& sm, int qt, int col, int half, const u32x4 (&wB)[4],
                                             const u32x4 qaug, const u32x4 augB) {
  f32x16 acc = {};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    acc = mfma_bf16(as_bf16x8(wB[kb]),
                    as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.q[qt][swz(col, 2 * kb + half)])), acc);
  return mfma_bf16(as_bf16x8(qaug), as_bf16x8(augB), acc);
}

// Sixteen per-register values (features of a D-layout tile), passed by value.
struct F16 {
  float v[16];
};

// Slow path of the kernel matrix for query tile qt of one wave: entries
// straight from the exponents over the wave's features, each row scaled by its
// own largest visible term 2^B_i,
//   P_ij 2^-B_i = sum_f 2^(a_if + e_jf - B_i),  B_i = max_{j <= i, f} (a_if + e_jf),
// from a_if (the query projections, lane = query, registers = features) and
// e_jf (fp32, the wave's [feature][key] area).  slow_rowmax gives B_i for the
// lane's query; slow_tile writes key tile kt's entries as pscr[query][key]
// (32 x 32 floats), from where the caller reads them in the P^T register
// layout (lane = query, registers = keys).  Taken only for chunks that need
// it (a wave-uniform branch); the loops stay rolled to keep registers few.
template <int C>
__device__ __forceinline__ float slow_rowmax(const float* e, const F16& a, int qt, int nvalid, int lane) {
  constexpr int KS = 32 * Cfg<C>::T;
  const int half = lane >> 5, qi = 32 * qt + (lane & 31);
  const int nk = min(32 * (qt + 1), nvalid);
  float B = -kFInf;
#pragma unroll 1
  for (int kj = 0; kj < nk; ++kj) {
    float mx = -kFInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, a.v[i] + e[drow(i, half) * KS + kj]);
    mx = pair_max(mx);
    if (kj <= qi) B = fmaxf(B, mx);
  }
  return B;
}

template <int C>
__device__ __forceinline__ void slow_tile(const float* e, const F16& a, int kt, int qt, int nvalid, float B, int lane,
                                          float* pscr) {
  constexpr int KS = 32 * Cfg<C>::T;
  const int half = lane >> 5, col = lane & 31, qi = 32 * qt + col;
#pragma unroll 1
  for (int j = 0; j < 32; ++j) {
    const int kj = 32 * kt + j;
    float sum = 0.f;
    if (B != -kFInf && kj < nvalid) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += fast_exp2(a.v[i] + e[drow(i, half) * KS + kj] - B);
    }
    sum = pair_sum(sum);
    if (!(kj <= qi && kj < nvalid)) sum = 0.f;
    if (half == 0) pscr[col * 32 + j] = sum;
  }
}

// Carry weights u_if = 2^(a_if + gam_f - mc_i) straight from the projections
// (when the row's weights relative to u would fall below 2^-60): a_if from
// the query projections (registers = features), gam_f from the wave's scalar
// slots (feature order).  Returns mc_i for the lane's query.
__device__ __forceinline__ float carry_exact(const F16& a, const float* gam_slots, int half, u32x4 (&uc)[2]) {
  float g[16];
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    const f32x4 y = *reinterpret_cast<const f32x4*>(&gam_slots[8 * g4 + 4 * half]);
#pragma unroll
    for (int j = 0; j < 4; ++j) g[4 * g4 + j] = y[j];
  }
  float mc = -kFInf;
#pragma unroll
  for (int i = 0; i < 16; ++i) mc = fmaxf(mc, a.v[i] + g[i]);
  mc = pair_max(mc);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int i = 8 * kb + 2 * w;
      uc[kb][w] = pack_f16(fast_exp2(a.v[i] + g[i] - mc), fast_exp2(a.v[i + 1] + g[i + 1] - mc));
    }
  return mc;
}

// Power of two >= x (x >= 0); 1 for x = 0.
__device__ __forceinline__ float pow2_above(float x) {
  int ex = 0;
  if (x > 0.f && x <= 3.0e38f) frexpf(x, &ex);
  return ldexpf(1.0f, ex);
}

template <int NW, int C>
__global__ __launch_bounds__(NW * 64, 1) void k_causal_walk(Args a) {
  constexpr int T = Cfg<C>::T, R = Cfg<C>::R, NT = NW * 64, M = NW * 32;
  static_assert(NW <= Cfg<C>::NWMAX, "too many waves for this chunk length");
  __shared__ __attribute__((aligned(16))) Smem<C> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int wg = xcd_contiguous(blockIdx.x, gridDim.x);   // segments of one (b, h) share an L2
  const int seg = wg % a.nseg;
  const int rest = wg / a.nseg;
  const int bh = rest % a.BH;
  const int sl = rest / a.BH;
  const int slice = a.slice0 + sl;
  const int fsl = a.fbase + sl * a.ms;       // the slice's first feature
  const int hh = bh % a.H;
  const int d = a.d;
  const int s0 = seg * a.seglen;
  const int ntok = min(a.n, s0 + a.seglen) - s0;
  if (ntok <= 0) return;   // whole workgroup
  const size_t tok0 = static_cast<size_t>(bh) * a.n + s0;
  const uint16_t* Kb = a.k + tok0 * d;
  const uint16_t* Vb = a.v + tok0 * d;
  const uint16_t* Qb = a.q + tok0 * d;
  // features of this wave: fsl + 32 wave + j, j < nvf valid
  const int fw = fsl + 32 * wave;
  const int nvf = max(0, min(32, a.m - fw));   // wave-uniform

  // W rows of the wave's features: B operand of the key projection and A
  // operand of the query projection (the same registers; 0 past m or d)
  u32x4 wB[4];
  {
    const int f = fw + col;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bool live = col < nvf && 16 * kb + 8 * half < d;
      wB[kb] = live ? *reinterpret_cast<const u32x4*>(a.W + (static_cast<size_t>(hh) * a.m + f) * d + 16 * kb + 8 * half)
                    : u32x4{0u, 0u, 0u, 0u};
      asm volatile("" : "+v"(wB[kb]));
    }
  }
  const u32x4 augB = half == 0 ? u32x4{kBf16One | (kBf16One << 16), kBf16One, 0u, 0u} : u32x4{0u, 0u, 0u, 0u};
  const u32x4 ones = {kF16OnePair, kF16OnePair, kF16OnePair, kF16OnePair};

  // Value scale: a power of two above the largest |v| of this and the earlier
  // segments (the state pass's per-range maxima, else a pass over the values).
  float vm = 0.f;
  if (a.has_carry) {
    for (int s2 = 0; s2 <= seg; ++s2) vm = fmaxf(vm, a.seg_vmax[static_cast<size_t>(bh) * a.nseg + s2]);
  } else {
    for (int cc = tid; cc < ntok * 8; cc += NT) {
      if (8 * (cc & 7) >= d) continue;
      const u32x4 x = *reinterpret_cast<const u32x4*>(Vb + static_cast<size_t>(cc >> 3) * d + (cc & 7) * 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) vm = fmaxf(vm, fmaxf(fabsf(bf16_lo_as_f32(x[w])), fabsf(bf16_hi_as_f32(x[w]))));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) vm = fmaxf(vm, __shfl_xor(vm, o));
    if (lane == 0) sm.xs[wave][0] = vm;
    __syncthreads();
    vm = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) vm = fmaxf(vm, sm.xs[w][0]);
    __syncthreads();
  }
  const float vsig = pow2_above(vm);
  const float vinv = 1.0f / vsig;

  // State of the keys before the current chunk, for the wave's 32 features:
  // S (D layout: rows = features, lanes = value columns, in sigma_v units),
  // z and the shift c (lane = feature).  sum_j exp(w_f.k_j - |k_j|^2/2) = z_f 2^c_f.
  float c = -kFInf, z = 0.f;
  f32x16 sacc[2] = {};
  if (a.has_carry && seg > 0) {
    // Carry = ordered merge of the states of segments 0 .. seg-1.  Each partial,
    // and the running state, is renormalised to z = 1 by folding log2 z into its
    // shift.  Two threads per feature, 32 value columns each; the result goes
    // through the (still unused) partial area into the register layout.
    const int f = tid >> 1, hq = tid & 1;   // slice feature f (NT threads cover M = NT / 2 features)
    const int fg = fsl + f;
    float cr = -kFInf, zr = 0.f;
    f32x4 Sr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) Sr[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int MA = a.malloc_;
#pragma unroll 1
    for (int s2 = 0; s2 < seg; ++s2) {
      const size_t base = static_cast<size_t>(bh) * a.nseg + s2;
      float cp = a.part_zc[base * 2 * MA + MA + fg];
      const float zp = a.part_zc[base * 2 * MA + fg];
      const f32x4* src = reinterpret_cast<const f32x4*>(a.part_S + (base * MA + fg) * kD + 32 * hq);
      f32x4 r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = src[j];
      float bscale = 0.f;
      if (cp != -kFInf && zp > 0.f) {
        bscale = 1.0f / zp;
        cp += log2f(zp);
      } else {
        cp = -kFInf;
      }
      const float cn = fmaxf(cr, cp);
      const float al = (cr == -kFInf) ? 0.f : exp2f(cr - cn);
      const float be = (cp == -kFInf) ? 0.f : exp2f(cp - cn) * bscale;
      zr = fmaf(al, zr, be * zp);
#pragma unroll
      for (int j = 0; j < 8; ++j) Sr[j] = al * Sr[j] + be * r[j];
      cr = cn;
      if (zr > 0.f) {
        const float iz = 1.0f / zr;
        cr += log2f(zr);
        zr = 1.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) Sr[j] *= iz;
      }
    }
    float* cbuf = &sm.np[0][0];   // M x 64 floats: fits the partial area (NWMAX waves x 32 x 64)
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<f32x4*>(&cbuf[f * kD + 32 * hq + 4 * j]) = Sr[j];
    if (hq == 0) {
      sm.xs[f >> 5][f & 31] = zr;
      sm.xs2[f >> 5][f & 31] = cr;
    }
    __syncthreads();
    if (col < nvf) {
      z = sm.xs[wave][col];
      c = sm.xs2[wave][col];
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[dt][i] = cbuf[(32 * wave + drow(i, half)) * kD + 32 * dt + col] * vinv;
    __syncthreads();
  }

  // Summary of the state for the carry term: 1/z_f in the wave's slots (the
  // query side forms yhat_f = S_f / z_f from the state registers with it) and
  // gam_f = c_f + log2 z_f (lane = feature).
  float gam = -kFInf;
  auto summarize = [&]() {
    const float iz = z > 0.f ? fast_rcp(z) : 0.f;   // z >= 1 when nonzero (the shift's key counts 1)
    gam = z > 0.f ? c + __log2f(z) : -kFInf;
    if (half == 0) sm.iz[wave][col] = iz;
  };
  summarize();

  const int nchunks = (ntok + C - 1) / C;
  Regs<C, NT> regs;
  load_chunk<C, NT>(regs, Kb, Vb, Qb, 0, ntok, d, tid);
  stage_chunk<C, NT>(sm, regs, vinv, tid);
  if (nchunks > 1) load_chunk<C, NT>(regs, Kb, Vb, Qb, C, ntok, d, tid);
  __syncthreads();

  uint32_t* area = sm.tr[wave];
  for (int t = 0; t < nchunks; ++t) {
    const int t0 = t * C;
    const int nvalid = min(C, ntok - t0);   // keys / queries of the chunk inside the segment
    // Lane-dependent LDS addresses are recomputed per chunk rather than held
    // in loop-invariant registers.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int col = ln & 31, half = ln >> 5;

    // ---- keys: projections (lane = feature, registers = keys) and the shift
    f32x16 pk[T];
    float mx = -kFInf, mn = kFInf;
#pragma unroll
    for (int kt = 0; kt < T; ++kt) {
      pk[kt] = key_proj<C>(sm, kt, col, half, wB, augB);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kj = 32 * kt + drow(i, half);
        const bool ok = kj < nvalid && (C >= 32 || kj < R);
        const float e = pk[kt][i] * kLog2e;
        pk[kt][i] = ok ? e : -kFInf;
        mx = fmaxf(mx, pk[kt][i]);
        mn = fminf(mn, ok ? e : kFInf);
      }
    }
    mx = pair_max(mx);
    mn = -pair_max(-mn);
    const bool fvalid = col < nvf;
    const float cold = c;
    const bool need = fvalid && mx > c + 8.0f;
    const float cnew = need ? mx : c;
    // fast path unless some feature's keys spread far below its new shift
    // while the state there is empty or far below it
    const bool wide = fvalid && cnew - mn > kSpreadLimit && !(cold >= cnew - kSpreadLimit);
    const bool slow = __ballot(wide) != 0;
    // key features 2^(e - c') of the chunk: fp16 for the state update (kept),
    // bf16 hi + lo (or fp32 exponents on the slow path) to the wave's area
    u32x4 k16[T][2];
    const float cs = cnew == -kFInf ? 0.f : cnew;
#pragma unroll
    for (int kt = 0; kt < T; ++kt) {
      float ph[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) ph[i] = fvalid ? fast_exp2(pk[kt][i] - cs) : 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int w = 0; w < 4; ++w) k16[kt][kb][w] = pack_f16(ph[8 * kb + 2 * w], ph[8 * kb + 2 * w + 1]);
      if (!slow) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint32_t h0, l0, h1, l1;
          split_bf16_trunc(ph[4 * g], ph[4 * g + 1], h0, l0);
          split_bf16_trunc(ph[4 * g + 2], ph[4 * g + 3], h1, l1);
          const int u = tr_unit<T>(col, 8 * kt + 2 * g + half);
          *reinterpret_cast<u32x2*>(&area[2 * u]) = u32x2{h0, h1};
          *reinterpret_cast<u32x2*>(&area[2 * u + 16 * 32 * T]) = u32x2{l0, l1};
        }
      } else {
        float* ea = reinterpret_cast<float*>(area);
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4*>(&ea[col * (32 * T) + 32 * kt + 8 * g + 4 * half]) =
              f32x4{pk[kt][4 * g], pk[kt][4 * g + 1], pk[kt][4 * g + 2], pk[kt][4 * g + 3]};
      }
    }
    // c' ln 2 as the query projection's extra k-block (feature rows)
    u32x4 qaug = {0u, 0u, 0u, 0u};
    if (half == 0 && cnew != -kFInf) {
      uint32_t w01, w23;
      split3_bf16(cnew * kLn2, w01, w23);
      qaug = u32x4{w01, w23, 0u, 0u};
    }
    // per-feature values in the wave's scalar slots, read per register
    // (registers = features) where used: G'_f = 2^(gam_f - c'_f) (the carry's
    // weights relative to u) and gam_f
    if (half == 0) {
      sm.xs[wave][col] = (gam == -kFInf || !fvalid) ? 0.f : fast_exp2(gam - cs);
      sm.xs2[wave][col] = fvalid ? gam : -kFInf;
      sm.cp[wave][col] = cs;
    }
    const bool has_state = __ballot(fvalid && gam != -kFInf) != 0;
    const float* gslot = sm.xs[wave];
    const float* gamslot = sm.xs2[wave];

    // ---- queries, one 32-row tile at a time
#pragma unroll
    for (int qt = 0; qt < T; ++qt) {
      f32x16 pq = query_proj<C>(sm, qt, col, half, wB, qaug, augB);
      float s2 = -kFInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pq[i] = drow(i, half) < nvf ? pq[i] * kLog2e : -kFInf;   // a_if + c'_f, masked past m
        s2 = fmaxf(s2, pq[i]);
      }
      s2 = pair_max(s2);

      // kernel matrix P^T[key, query] of the key tiles kt <= qt (lane = query)
      f32x16 pt[T];
      float sc = s2;   // log2 scale of the entries of pt for this lane's query
      if (slow) {
        // a_if = (a_if + c'_f) - c'_f, with c'_f of the register's feature
        F16 av;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 c4 = *reinterpret_cast<const f32x4*>(&sm.cp[wave][8 * g4 + 4 * half]);
#pragma unroll
          for (int j = 0; j < 4; ++j) av.v[4 * g4 + j] = pq[4 * g4 + j] - c4[j];
        }
        float* pscr = sm.np[wave];   // 32 queries x 32 keys (the partial area is free here)
        const float* ea = reinterpret_cast<const float*>(area);
        sc = slow_rowmax<C>(ea, av, qt, nvalid, ln);
#pragma unroll
        for (int kt = 0; kt <= qt; ++kt) {
          slow_tile<C>(ea, av, kt, qt, nvalid, sc, ln, pscr);
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(&pscr[col * 32 + 8 * g4 + 4 * half]);
#pragma unroll
            for (int j = 0; j < 4; ++j) pt[kt][4 * g4 + j] = x[j];
          }
        }
      }
      float u[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) u[i] = fast_exp2(pq[i] - s2);
      if (!slow) {
        u32x4 uhi[2], ulo[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t h_, l_;
            split_bf16_trunc(u[8 * kb + 2 * w], u[8 * kb + 2 * w + 1], h_, l_);
            uhi[kb][w] = h_;
            ulo[kb][w] = l_;
          }
#pragma unroll
        for (int kt = 0; kt <= qt; ++kt) {
          f32x16 acc = {};
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const u32x4 ah = tr_operand<T>(area, kt, kb, ln);
            const u32x4 al = tr_operand<T>(area + 16 * 32 * T, kt, kb, ln);
            acc = mfma_bf16(as_bf16x8(ah), as_bf16x8(uhi[kb]), acc);
            acc = mfma_bf16(as_bf16x8(al), as_bf16x8(uhi[kb]), acc);
            acc = mfma_bf16(as_bf16x8(ah), as_bf16x8(ulo[kb]), acc);
          }
          pt[kt] = acc;
        }
        // causal mask on the diagonal tile; keys past the chunk are 0 already
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (drow(i, half) > col) pt[qt][i] = 0.f;
      }

      // carry weights (state before the chunk): u_if G'_f normalised to a row
      // maximum of 1, or from the projections when that maximum is tiny
      u32x4 uc[2] = {};
      float mc = -kFInf;
      if (has_state) {
        float pmx = 0.f;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 G = *reinterpret_cast<const f32x4*>(&gslot[8 * g4 + 4 * half]);
#pragma unroll
          for (int j = 0; j < 4; ++j) pmx = fmaxf(pmx, u[4 * g4 + j] * G[j]);
        }
        pmx = pair_max(pmx);
        if (__ballot(!(pmx >= 0x1p-60f)) == 0) {
          const float kap = fast_rcp(pmx);
          mc = __log2f(pmx) + s2;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 G = *reinterpret_cast<const f32x4*>(&gslot[8 * g4 + 4 * half]);
            const int i = 4 * g4;
            uc[g4 >> 1][2 * (g4 & 1)] = pack_f16(u[i] * G[0] * kap, u[i + 1] * G[1] * kap);
            uc[g4 >> 1][2 * (g4 & 1) + 1] = pack_f16(u[i + 2] * G[2] * kap, u[i + 3] * G[3] * kap);
          }
        } else {
          // the projections again (this path is rare), so that a_if need not stay live
          const f32x16 pr = query_proj<C>(sm, qt, col, half, wB, qaug, augB);
          F16 av;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 c4 = *reinterpret_cast<const f32x4*>(&sm.cp[wave][8 * g4 + 4 * half]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int i = 4 * g4 + j;
              av.v[i] = drow(i, half) < nvf ? pr[i] * kLog2e - c4[j] : -kFInf;
            }
          }
          mc = carry_exact(av, gamslot, half, uc);
        }
      }
      float rmx = 0.f;
#pragma unroll
      for (int kt = 0; kt <= qt; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) rmx = fmaxf(rmx, pt[kt][i]);
      rmx = pair_max(rmx);
      const float chunk_l = rmx > 0.f ? sc + __log2f(rmx) : -kFInf;
      const float L = fmaxf(mc, chunk_l);
      const float Ls = L == -kFInf ? 0.f : L;
      const float fac = rmx > 0.f ? fast_exp2(sc - Ls) : 0.f;
      const float cfac = mc == -kFInf ? 0.f : fast_exp2(mc - Ls);

      // numerator and denominator: carry (weights x yhat, yhat = S / z formed
      // from the state registers and 1/z in the scalar slots) and chunk (P x V)
      f32x16 np0 = {}, np1 = {}, den = {};
      if (has_state) {
        const f16x2 cf2 = {static_cast<_Float16>(cfac), static_cast<_Float16>(cfac)};
        const float* izs = sm.iz[wave];   // 1/z, written by summarize
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          u32x4 w4, y0, y1;
#pragma unroll
          for (int w = 0; w < 4; ++w) w4[w] = mul_f16x2(uc[kb][w], cf2);
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const f32x4 iz = *reinterpret_cast<const f32x4*>(&izs[8 * (2 * kb + g) + 4 * half]);
            const int i = 8 * kb + 4 * g;
            y0[2 * g] = pack_f16(sacc[0][i] * iz[0], sacc[0][i + 1] * iz[1]);
            y0[2 * g + 1] = pack_f16(sacc[0][i + 2] * iz[2], sacc[0][i + 3] * iz[3]);
            y1[2 * g] = pack_f16(sacc[1][i] * iz[0], sacc[1][i + 1] * iz[1]);
            y1[2 * g + 1] = pack_f16(sacc[1][i + 2] * iz[2], sacc[1][i + 3] * iz[3]);
          }
          np0 = mfma_f16(as_f16x8(w4), as_f16x8(y0), np0);
          np1 = mfma_f16(as_f16x8(w4), as_f16x8(y1), np1);
          den = mfma_f16(as_f16x8(w4), as_f16x8(ones), den);
        }
      }
#pragma unroll
      for (int kt = 0; kt <= qt; ++kt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 w4 = pack_kblock_f16(pt[kt], kb, fac);
          np0 = mfma_f16(as_f16x8(w4), as_f16x8(v_operand(sm.v[kt], 16 * kb, 0, ln)), np0);
          np1 = mfma_f16(as_f16x8(w4), as_f16x8(v_operand(sm.v[kt], 16 * kb, 1, ln)), np1);
          den = mfma_f16(as_f16x8(w4), as_f16x8(ones), den);
        }

      // partials of this query tile to LDS (rows with their 8-float blocks
      // XOR-swizzled by row & 7, so the combine's reads spread over the banks)
      float* npw = sm.np[wave];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = drow(i, half);
        const int sw = (r & 7) << 3;
        npw[r * kD + (col ^ sw)] = np0[i];
        npw[r * kD + ((32 + col) ^ sw)] = np1[i];
      }
      if (col == 0) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<f32x4*>(&sm.dp[wave][8 * g4 + 4 * half]) =
              f32x4{den[4 * g4], den[4 * g4 + 1], den[4 * g4 + 2], den[4 * g4 + 3]};
      }
      if (half == 0) sm.lp[wave][col] = L;

      if (qt == T - 1) {
        // ---- the chunk's keys join the state (after every query tile used it)
        if (__ballot(need) != 0) {
          const float scl = need ? ((cold == -kFInf) ? 0.f : exp2f(cold - cnew)) : 1.0f;
          z *= scl;
          if (half == 0) sm.xs[wave][col] = scl;
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 s4 = *reinterpret_cast<const f32x4*>(&sm.xs[wave][8 * g4 + 4 * half]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              sacc[0][4 * g4 + j] *= s4[j];
              sacc[1][4 * g4 + j] *= s4[j];
            }
          }
          __builtin_amdgcn_wave_barrier();
        }
        c = cnew;
        f32x16 zacc = {};
#pragma unroll
        for (int kt = 0; kt < T; ++kt)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
              sacc[dt] = mfma_f16(as_f16x8(k16[kt][kb]), as_f16x8(v_operand(sm.v[kt], 16 * kb, dt, ln)), sacc[dt]);
            zacc = mfma_f16(as_f16x8(k16[kt][kb]), as_f16x8(ones), zacc);
          }
        // every column of zacc holds the chunk's z of the feature in that row:
        // rows to lanes through the wave's scalar slots
        if (col == 0) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            *reinterpret_cast<f32x4*>(&sm.xs2[wave][8 * g4 + 4 * half]) =
                f32x4{zacc[4 * g4], zacc[4 * g4 + 1], zacc[4 * g4 + 2], zacc[4 * g4 + 3]};
        }
        __builtin_amdgcn_wave_barrier();
        if (fvalid) z += sm.xs2[wave][col];
        __builtin_amdgcn_wave_barrier();
        if (t + 1 < nchunks) summarize();
      }

      // ---- combine the partials of this query tile's rows and store
      lds_barrier();
      const int rows = min(R, nvalid - 32 * qt);   // rows of this tile inside the segment
      for (int it = tid; it < 32 * 8; it += NT) {
        const int r = it >> 3, c8 = it & 7;
        if (r >= rows || 8 * c8 >= d && a.nslices == 1) continue;
        float lmax = -kFInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) lmax = fmaxf(lmax, sm.lp[w][r]);
        float dsum = 0.f;
        f32x4 n0 = {0.f, 0.f, 0.f, 0.f}, n1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float l = sm.lp[w][r];
          const float wt = l == -kFInf ? 0.f : fast_exp2(l - lmax);
          dsum = fmaf(wt, sm.dp[w][r], dsum);
          const int ds = (8 * c8) ^ ((r & 7) << 3);
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(&sm.np[w][r * kD + ds]);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(&sm.np[w][r * kD + ds + 4]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            n0[j] = fmaf(wt, x0[j], n0[j]);
            n1[j] = fmaf(wt, x1[j], n1[j]);
          }
        }
        const size_t tok = tok0 + t0 + 32 * qt + r;
        if (a.nslices == 1) {
          const float inv = vsig * fast_rcp(dsum);
          f32x4* dst = reinterpret_cast<f32x4*>(a.out + tok * d + 8 * c8);
          __builtin_nontemporal_store(n0 * inv, dst);
          __builtin_nontemporal_store(n1 * inv, dst + 1);
        } else {
          const size_t prow = static_cast<size_t>(slice) * a.BH * a.n + tok;
          f32x4* dst = reinterpret_cast<f32x4*>(a.pnum + prow * kD + 8 * c8);
          dst[0] = n0 * vsig;
          dst[1] = n1 * vsig;
          if (c8 == 0) *reinterpret_cast<f32x2*>(a.pdl + prow * 2) = f32x2{dsum, lmax};
        }
      }
      if (qt < T - 1) lds_barrier();   // partial area free for the next query tile
    }

    // ---- next chunk's tiles (every wave is past its reads of this chunk)
    if (t + 1 < nchunks) {
      stage_chunk<C, NT>(sm, regs, vinv, tid);
      if (t + 2 < nchunks) load_chunk<C, NT>(regs, Kb, Vb, Qb, t0 + 2 * C, ntok, d, tid);
    }
    lds_barrier();
  }
}

// Launch one group of nsl slices of equal width (nw waves each) for chunk length C.
#define FAVOR_WALK_CASE(NWV)                                                                               \
  case NWV:                                                                                              \
    FAVOR_LAUNCH("k_causal_walk", (k_causal_walk<NWV, C>), dim3(a.BH * a.nseg * nsl), dim3(NWV * 64), 0, s, a); \
    break;

template <int C>
hipError_t launch_group_impl(const Args& a, int nw, int nsl, hipStream_t s) {
  if constexpr (Cfg<C>::NWMAX >= 8) {
    switch (nw) {
      FAVOR_WALK_CASE(1)
      FAVOR_WALK_CASE(2)
      FAVOR_WALK_CASE(3)
      FAVOR_WALK_CASE(4)
      FAVOR_WALK_CASE(5)
      FAVOR_WALK_CASE(6)
      FAVOR_WALK_CASE(7)
      FAVOR_WALK_CASE(8)
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (nw) {
      FAVOR_WALK_CASE(1)
      FAVOR_WALK_CASE(2)
      FAVOR_WALK_CASE(3)
      FAVOR_WALK_CASE(4)
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}
#undef FAVOR_WALK_CASE

}  // namespace walk
}  // namespace favor
