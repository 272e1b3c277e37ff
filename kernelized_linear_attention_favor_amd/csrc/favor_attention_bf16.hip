// bf16-input FAVOR+ attention on gfx950 MFMA (non-causal), three kernels:
//
//   k_kv_state  : per (key-range split, b, h): Phi(K)^T [V | 1] partial sums.
//   k_merge     : per (b, h, 8 value columns): combine splits in fixed order,
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
//   * key features exp(e - c) are split into bf16 hi + lo (16 significant
//     bits) for the S = Phi(K)^T V MFMA; V is used exactly as given (bf16).
//   * query softmax weights are in (0, 1] and go to fp16; yhat columns are
//     scaled by a power of two into (-1, 1) and go to fp16; the denominator is
//     the same fp16 weights times 1.0, so rounding of a weight moves numerator
//     and denominator together.
//   * projections w.x (+ the -|k|^2/2 or beta term, carried as three bf16
//     parts in an extra k-block) accumulate in fp32.
#include <math.h>

#include "favor_internal.h"
#include "favor_mfma.h"

namespace favor {
namespace {

constexpr int kD = 64;          // head dimension supported by the MFMA path
constexpr int kKT = 64;         // key tokens staged per iteration (two 32-token MFMA tiles)
constexpr int kKStride = 88;    // bf16 per staged key row: 64 d + 8 aug + 8 zero + 8 pad
constexpr int kVStride = 72;    // bf16 per staged value column: 64 tokens + 8 pad
constexpr uint32_t kBf16One = 0x3f80u;
constexpr float kFInf = __builtin_huge_valf();

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

// ---------------------------------------------------------------------------
// k_kv_state: one workgroup = NW waves = 64*NW features (all m features) of
// one (b, h) over one contiguous key range.  Wave w owns features
// [64w, 64w+64) as two 32-feature MFMA tiles.
//
// Per 32-key tile and feature tile:
//   proj (32x32 MFMA, k = 64 d + 1 aug block) -> D[key, feature] =
//        w_f.k_j - |k_j|^2/2                    (lane = feature column)
//   phi  = exp2(D log2e - c_f)                   (c_f: per feature, set from the
//                                                 first tile of the range)
//   S_f += (phi_hi + phi_lo)^T V                 (output registers reused as the
//                                                 A operand; V staged transposed)
//   z_f += phi
// If any phi overflowed (a later key far above the first tile), the range is
// recomputed with c_f set by a max-only pass.
// ---------------------------------------------------------------------------
template <int NW>
struct KvSmem {
  uint16_t ks[2][kKT * kKStride];
  uint16_t vt[2][kD * kVStride];
  int flag;
};

template <int NW>
__device__ __forceinline__ void stage_kv(KvSmem<NW>& sm, int buf, const u32x4* kreg,
                                         const u32x4* vreg, int tid) {
  constexpr int NT = NW * 64;
  constexpr int R = (kKT * 8 + NT - 1) / NT;  // 16-byte chunks per thread per tensor
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = tid + NT * r;
    if (c >= kKT * 8) break;  // whole waves drop out together (NT is a multiple of 64)
    const int tok = c >> 3, ch = c & 7;
    *reinterpret_cast<u32x4*>(&sm.ks[buf][tok * kKStride + ch * 8]) = kreg[r];
    // -|k|^2/2 from the 8 threads holding this token's 64 values
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = bf16_lo_as_f32(kreg[r][w]), b = bf16_hi_as_f32(kreg[r][w]);
      s = fmaf(a, a, s);
      s = fmaf(b, b, s);
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    if (ch == 0) {
      uint32_t w01, w23;
      split3_bf16(-0.5f * s, w01, w23);
      *reinterpret_cast<u32x4*>(&sm.ks[buf][tok * kKStride + 64]) = u32x4{w01, w23, 0u, 0u};
      *reinterpret_cast<u32x4*>(&sm.ks[buf][tok * kKStride + 72]) = u32x4{0u, 0u, 0u, 0u};
    }
    // V transposed: vt[dv][pos(tok)], pos applies the k-block slot permutation
    const int pos = (tok & ~15) | kblock_pos(tok & 15);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sm.vt[buf][(ch * 8 + 2 * w) * kVStride + pos] = static_cast<uint16_t>(vreg[r][w] & 0xffffu);
      sm.vt[buf][(ch * 8 + 2 * w + 1) * kVStride + pos] = static_cast<uint16_t>(vreg[r][w] >> 16);
    }
  }
}

template <int NW>
__device__ __forceinline__ void load_kv(const uint16_t* Kb, const uint16_t* Vb, int tile0, int ntok,
                                        u32x4* kreg, u32x4* vreg, int tid) {
  constexpr int NT = NW * 64;
  constexpr int R = (kKT * 8 + NT - 1) / NT;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = tid + NT * r;
    if (c >= kKT * 8) break;
    const int tok = tile0 + (c >> 3), ch = c & 7;
    if (tok < ntok) {
      kreg[r] = *reinterpret_cast<const u32x4*>(Kb + static_cast<size_t>(tok) * kD + ch * 8);
      vreg[r] = *reinterpret_cast<const u32x4*>(Vb + static_cast<size_t>(tok) * kD + ch * 8);
    } else {
      kreg[r] = u32x4{0u, 0u, 0u, 0u};
      vreg[r] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// MODE 0: accumulate, first tile fixes c.  MODE 1: max only.  MODE 2: accumulate with fixed c.
template <int NW, int MODE>
__device__ __forceinline__ void kv_tile(KvSmem<NW>& sm, int buf, int tile0, int ntok,
                                        const u32x4 (&wB)[2][4], const u32x4 augB, float (&c)[2],
                                        float (&z)[2], f32x16 (&sacc)[2][2], bool& cinit, int col,
                                        int half) {
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int tok_base = tile0 + 32 * st;
    if (tok_base >= ntok) break;
    const bool partial = tok_base + 32 > ntok;
    bf16x8 ka[5];
#pragma unroll
    for (int kb = 0; kb < 5; ++kb)
      ka[kb] = as_bf16x8(*reinterpret_cast<const u32x4*>(
          &sm.ks[buf][(32 * st + col) * kKStride + 16 * kb + 8 * half]));
    f32x16 pacc[2];
#pragma unroll
    for (int ft = 0; ft < 2; ++ft) {
      f32x16 acc = {};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) acc = mfma_bf16(ka[kb], as_bf16x8(wB[ft][kb]), acc);
      acc = mfma_bf16(ka[4], as_bf16x8(augB), acc);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float e = acc[i] * kLog2e;
        if (partial) {
          const int row = 8 * (i >> 2) + 4 * half + (i & 3);
          if (tok_base + row >= ntok) e = -kFInf;
        }
        acc[i] = e;
      }
      pacc[ft] = acc;
    }
    if (MODE == 1 || (MODE == 0 && !cinit)) {
#pragma unroll
      for (int ft = 0; ft < 2; ++ft) {
        float mx = pacc[ft][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, pacc[ft][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        c[ft] = fmaxf(c[ft], mx);
      }
      cinit = true;
    }
    if (MODE == 1) continue;
    // value operand: B[k = token slot][n = dv], read from the transposed stage
    u32x4 vb[2][2];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
        vb[dt][kb2] = *reinterpret_cast<const u32x4*>(
            &sm.vt[buf][(32 * dt + col) * kVStride + 32 * st + 16 * kb2 + 8 * half]);
#pragma unroll
    for (int ft = 0; ft < 2; ++ft) {
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = fast_exp2(pacc[ft][i] - c[ft]);
        z[ft] += p[i];
      }
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        u32x4 hi, lo;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t h_, l_;
          split_bf16(p[8 * kb2 + 2 * w], p[8 * kb2 + 2 * w + 1], h_, l_);
          hi[w] = h_;
          lo[w] = l_;
        }
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          sacc[ft][dt] = mfma_bf16(as_bf16x8(hi), as_bf16x8(vb[dt][kb2]), sacc[ft][dt]);
          sacc[ft][dt] = mfma_bf16(as_bf16x8(lo), as_bf16x8(vb[dt][kb2]), sacc[ft][dt]);
        }
      }
    }
  }
}

template <int NW, int MODE>
__device__ void kv_range(KvSmem<NW>& sm, const uint16_t* Kb, const uint16_t* Vb, int ntok,
                         const u32x4 (&wB)[2][4], const u32x4 augB, float (&c)[2], float (&z)[2],
                         f32x16 (&sacc)[2][2], bool& cinit, int tid, int col, int half) {
  constexpr int R = (kKT * 8 + NW * 64 - 1) / (NW * 64);
  const int ntiles = (ntok + kKT - 1) / kKT;
  u32x4 kreg[R], vreg[R];
  if (ntiles > 0) {
    load_kv<NW>(Kb, Vb, 0, ntok, kreg, vreg, tid);
    stage_kv<NW>(sm, 0, kreg, vreg, tid);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) load_kv<NW>(Kb, Vb, (t + 1) * kKT, ntok, kreg, vreg, tid);
    kv_tile<NW, MODE>(sm, t & 1, t * kKT, ntok, wB, augB, c, z, sacc, cinit, col, half);
    if (more) stage_kv<NW>(sm, (t + 1) & 1, kreg, vreg, tid);
    __syncthreads();
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 2) void k_kv_state(const uint16_t* __restrict__ K,
                                                         const uint16_t* __restrict__ V,
                                                         const uint16_t* __restrict__ W,
                                                         float* __restrict__ part_S,
                                                         float* __restrict__ part_zc, int H,
                                                         int n, int splits, int span) {
  constexpr int M = NW * 64;
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

  u32x4 wB[2][4];
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int f = 64 * wave + 32 * ft + col;
      wB[ft][kb] = *reinterpret_cast<const u32x4*>(W + (static_cast<size_t>(hh) * M + f) * kD +
                                                   16 * kb + 8 * half);
    }
  const u32x4 augB = half == 0 ? u32x4{kBf16One | (kBf16One << 16), kBf16One, 0u, 0u}
                               : u32x4{0u, 0u, 0u, 0u};

  float c[2] = {-kFInf, -kFInf}, z[2] = {0.f, 0.f};
  f32x16 sacc[2][2] = {};
  bool cinit = false;
  kv_range<NW, 0>(sm, Kb, Vb, ntok, wB, augB, c, z, sacc, cinit, tid, col, half);

  // Overflow guard: a key far above the first tile's maximum makes phi, z or S
  // non-finite; recompute the range with c from a max-only pass.
  bool bad = !(fabsf(z[0]) <= 3.0e38f) || !(fabsf(z[1]) <= 3.0e38f);
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) bad |= !(fabsf(sacc[ft][dt][i]) <= 3.0e38f);
  if (tid == 0) sm.flag = 0;
  __syncthreads();
  if (bad) sm.flag = 1;
  __syncthreads();
  if (sm.flag) {
    c[0] = c[1] = -kFInf;
    z[0] = z[1] = 0.f;
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) sacc[ft][dt] = f32x16{};
    kv_range<NW, 1>(sm, Kb, Vb, ntok, wB, augB, c, z, sacc, cinit, tid, col, half);
    kv_range<NW, 2>(sm, Kb, Vb, ntok, wB, augB, c, z, sacc, cinit, tid, col, half);
  }

  // write this range's partial state
  const size_t base = static_cast<size_t>(bh) * splits + split;
  float* zc = part_zc + base * 2 * M;
#pragma unroll
  for (int ft = 0; ft < 2; ++ft) {
    const float zt = z[ft] + __shfl_xor(z[ft], 32);
    const int f = 64 * wave + 32 * ft + col;
    if (half == 0) {
      zc[f] = zt;
      zc[M + f] = c[ft];
    }
  }
  float* Sb = part_S + base * M * kD;
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int f = 64 * wave + 32 * ft + 8 * (i >> 2) + 4 * half + (i & 3);
        Sb[static_cast<size_t>(f) * kD + 32 * dt + col] = sacc[ft][dt][i];
      }
}

// ---------------------------------------------------------------------------
// k_merge: one workgroup per (b, h, group of 8 value columns); thread f owns
// feature f.  Splits are combined in index order (deterministic):
//   c_f = max_s c_fs;  z_f = sum_s 2^{c_fs - c_f} z_fs;  S_f likewise;
//   yhat_f = S_f / z_f;  beta_f = (c_f + log2 z_f) ln 2  (natural-log units).
// yhat is stored as fp16 after dividing each column by sigma_c, a power of two
// above the column's largest |yhat|, transposed to [dv][slot] in the slot
// order the output kernel's B operand reads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_merge(const float* __restrict__ part_S,
                                               const float* __restrict__ part_zc,
                                               uint16_t* __restrict__ yhat,
                                               float* __restrict__ beta,
                                               float* __restrict__ sigma, int m, int splits) {
  __shared__ float red[8][8];
  const int bh = blockIdx.x >> 3;
  const int g = blockIdx.x & 7;
  const int f = threadIdx.x;
  float y[8];
  float amax[8];
  if (f < m) {
    float cm = -kFInf;
    for (int s = 0; s < splits; ++s)
      cm = fmaxf(cm, part_zc[(static_cast<size_t>(bh) * splits + s) * 2 * m + m + f]);
    float zt = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; ++s) {
      const size_t base = static_cast<size_t>(bh) * splits + s;
      const float cs = part_zc[base * 2 * m + m + f];
      if (cs == -kFInf) continue;
      const float a = exp2f(cs - cm);
      zt = fmaf(a, part_zc[base * 2 * m + f], zt);
      const f32x4* row = reinterpret_cast<const f32x4*>(part_S + (base * m + f) * kD + 8 * g);
      const f32x4 r0 = row[0], r1 = row[1];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        acc[cc] = fmaf(a, r0[cc], acc[cc]);
        acc[4 + cc] = fmaf(a, r1[cc], acc[4 + cc]);
      }
    }
    const float inv = 1.0f / zt;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      y[cc] = acc[cc] * inv;
      amax[cc] = fabsf(y[cc]);
    }
    if (g == 0) beta[static_cast<size_t>(bh) * m + f] = (cm + log2f(zt)) * kLn2;
  } else {
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      y[cc] = 0.f;
      amax[cc] = 0.f;
    }
  }
  // column maxima over the m features
#pragma unroll
  for (int cc = 0; cc < 8; ++cc)
    for (int o = 32; o > 0; o >>= 1) amax[cc] = fmaxf(amax[cc], __shfl_xor(amax[cc], o));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) red[wave][cc] = amax[cc];
  __syncthreads();
  float sc[8];
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
    float mx = fmaxf(fmaxf(red[0][cc], red[1][cc]), fmaxf(red[2][cc], red[3][cc]));
    // smallest power of two strictly above mx (1 for an all-zero column)
    int ex = 0;
    if (mx > 0.f && mx <= 3.0e38f) {
      frexpf(mx, &ex);  // mx = frac * 2^ex, frac in [0.5, 1)
    }
    sc[cc] = ldexpf(1.0f, ex);
  }
  if (f < m) {
    const int pos = (f & ~15) | kblock_pos(f & 15);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const _Float16 hv = static_cast<_Float16>(y[cc] / sc[cc]);
      yhat[(static_cast<size_t>(bh) * kD + 8 * g + cc) * m + pos] = __builtin_bit_cast(uint16_t, hv);
    }
  }
  if (threadIdx.x < 8) sigma[static_cast<size_t>(bh) * kD + 8 * g + threadIdx.x] = sc[threadIdx.x];
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
  const uint32_t h1 = 0x3c003c00u;  // fp16 (1.0, 1.0)
  const u32x4 onesB = u32x4{h1, h1, h1, h1};
  const uint16_t* Qb = Q + static_cast<size_t>(bh) * n * kD;
  float* Ob = out + static_cast<size_t>(bh) * n * kD;

  for (int tb = t0 + 32 * wave; tb < t1; tb += 128) {
    const int qt = tb + col;  // this lane's query (B operand column)
    u32x4 qB[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      qB[kb] = (qt < t1) ? *reinterpret_cast<const u32x4*>(Qb + static_cast<size_t>(qt) * kD +
                                                            16 * kb + 8 * half)
                         : u32x4{0u, 0u, 0u, 0u};
    // Shift: the first feature tile's row maximum plus 8 (log2 units).  Any
    // later feature more than 23 above it would overflow fp16; that case is
    // detected and the tile is redone with the exact row maximum.
    f32x16 p0 = out_proj(wsh, 0, col, half, qB, augB);
    float mx = p0[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, p0[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float off = -fmaf(mx, kLog2e, 8.0f);
    f32x16 yacc0 = {}, yacc1 = {}, dacc = {};
    float tmax = -kFInf;
    out_accumulate(p0, off, 0, ysh, YS, col, half, onesB, yacc0, yacc1, dacc, tmax);
#pragma unroll 1
    for (int ft = 1; ft < MT; ++ft) {
      const f32x16 pa = out_proj(wsh, ft, col, half, qB, augB);
      out_accumulate(pa, off, ft, ysh, YS, col, half, onesB, yacc0, yacc1, dacc, tmax);
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
      mx = fmaxf(mx, __shfl_xor(mx, 32));
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
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 8 * (i >> 2) + 4 * half + (i & 3);
      const int t = tb + row;
      if (t < t1) {
        const float inv = 1.0f / dacc[i];
        Ob[static_cast<size_t>(t) * kD + col] = yacc0[i] * sg0 * inv;
        Ob[static_cast<size_t>(t) * kD + 32 + col] = yacc1[i] * sg1 * inv;
      }
    }
  }
}

template <int NW>
hipError_t launch_kv(const Bf16Plan& p, const uint16_t* k, const uint16_t* v, const uint16_t* W,
                     float* pS, float* pzc, hipStream_t s) {
  hipLaunchKernelGGL(k_kv_state<NW>, dim3(p.B * p.H * p.splits), dim3(NW * 64), 0, s, k, v, W, pS,
                     pzc, p.H, p.n, p.splits, p.span);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_out(const Bf16Plan& p, const uint16_t* q, const uint16_t* W, const uint16_t* yh,
                      const float* beta, const float* sigma, float* out, int span,
                      hipStream_t s) {
  const int nblk = (p.n + span - 1) / span;
  hipLaunchKernelGGL(k_output<MT>, dim3(p.B * p.H * nblk), dim3(256), 0, s, q, W, yh, beta, sigma,
                     out, p.H, p.n, span);
  return hipGetLastError();
}

}  // namespace

bool bf16_supported(int d, int m) {
  return d == kD && (m == 64 || m == 128 || m == 192 || m == 256);
}

Bf16Plan bf16_plan(int B, int H, int n, int d, int m, int causal) {
  Bf16Plan p{};
  p.B = B;
  p.H = H;
  p.n = n;
  p.d = d;
  p.m = m;
  p.causal = causal;
  const long long BH = static_cast<long long>(B) * H;
  // aim for >= 512 state workgroups (two per CU), each with >= 64 keys
  long long splits = (512 + BH - 1) / BH;
  const long long max_splits = (n + kKT - 1) / kKT;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  p.splits = static_cast<int>(splits);
  p.span = static_cast<int>(align_up((n + splits - 1) / splits, kKT));
  size_t o = 0;
  p.off_part_S = o;
  o = align_up(o + sizeof(float) * BH * p.splits * m * kD, 256);
  p.off_part_zc = o;
  o = align_up(o + sizeof(float) * BH * p.splits * 2 * m, 256);
  p.off_yhat = o;
  o = align_up(o + sizeof(uint16_t) * BH * kD * m, 256);
  p.off_beta = o;
  o = align_up(o + sizeof(float) * BH * m, 256);
  p.off_sigma = o;
  o = align_up(o + sizeof(float) * BH * kD, 256);
  p.off_carry = o;
  p.off_end = o;
  return p;
}

hipError_t launch_attention_bf16(const Bf16Plan& p, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const uint16_t* W, float* out, void* ws,
                                 hipStream_t s) {
  if (p.causal) return hipErrorNotSupported;
  char* base = static_cast<char*>(ws);
  float* pS = reinterpret_cast<float*>(base + p.off_part_S);
  float* pzc = reinterpret_cast<float*>(base + p.off_part_zc);
  uint16_t* yh = reinterpret_cast<uint16_t*>(base + p.off_yhat);
  float* beta = reinterpret_cast<float*>(base + p.off_beta);
  float* sigma = reinterpret_cast<float*>(base + p.off_sigma);
  hipError_t e;
  switch (p.m) {
    case 64: e = launch_kv<1>(p, k, v, W, pS, pzc, s); break;
    case 128: e = launch_kv<2>(p, k, v, W, pS, pzc, s); break;
    case 192: e = launch_kv<3>(p, k, v, W, pS, pzc, s); break;
    case 256: e = launch_kv<4>(p, k, v, W, pS, pzc, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_merge, dim3(p.B * p.H * 8), dim3(256), 0, s, pS, pzc, yh, beta, sigma, p.m,
                     p.splits);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // output: about 512+ workgroups, each a contiguous run of query tiles
  const long long BH = static_cast<long long>(p.B) * p.H;
  long long per = (1024 + BH - 1) / BH;
  long long span = (p.n + per - 1) / per;
  span = align_up(span < 128 ? 128 : span, 128);
  switch (p.m) {
    case 64: return launch_out<2>(p, q, W, yh, beta, sigma, out, static_cast<int>(span), s);
    case 128: return launch_out<4>(p, q, W, yh, beta, sigma, out, static_cast<int>(span), s);
    case 192: return launch_out<6>(p, q, W, yh, beta, sigma, out, static_cast<int>(span), s);
    case 256: return launch_out<8>(p, q, W, yh, beta, sigma, out, static_cast<int>(span), s);
  }
  return hipErrorInvalidValue;
}

}  // namespace favor
