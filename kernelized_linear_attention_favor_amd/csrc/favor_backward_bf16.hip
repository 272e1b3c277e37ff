// Backward pass of FAVOR+ attention (dQ, dK, dV for an upstream gradient dY),
// derived from the forward (Performer notes, Kernel Attention View,
// Normalization and FAVOR+) by the chain rule: the pages mention training and
// gradients but print no formulas.
//
// Exact rewrite used throughout (log2 units): with e_jf = log2e (w_f.k_j -
// |k_j|^2/2), C_f = max_j e_jf over the head's keys, g_if = log2e w_f.q_i + C_f
// and a per-query shift M_i (the row maximum max_f g_if; the non-causal query
// pass takes the first feature tile's, with a_if checked to stay below 2^64),
//   b_jf = 2^(e_jf - C_f) in (0, 1],   a_if = 2^(g_if - M_i),
// phi(q_i).phi(k_j) = lambda_i a_i.b_j for a per-query constant lambda_i, which
// cancels in y and in every gradient below.  With S = sum_j b_j v_j^T, z =
// sum_j b_j, D_i = a_i.z, delta_i = dy_i.y_i (y the forward output):
//   G_if = a_if (S_f.dy_i - z_f delta_i) / D_i,  dq_i = W^T G_i - q_i sum_f G_if
//   R = sum_i (a_i / D_i) dy_i^T,  rho = sum_i (a_i / D_i) delta_i,
//   dv_j = R^T b_j,  H_jf = b_jf (R_f.v_j - rho_f),  dk_j = W^T H_j - k_j sum_f H_jf
// (d phi_f(x) / dx = phi_f(x) (w_f - x)).  The key shift C_f is one constant per
// feature for the whole head, so these are plain bounded sums in fp32; a
// feature's key exponents may spread up to ~2^126 below its largest.  A query
// whose D_i underflows to 0 (all its visible keys beyond that spread in every
// feature) gets dq_i = 0 and adds nothing to R, rho: a defined, finite result
// at the range limit instead of inf/NaN.
//
// Kernels (non-causal): k_bw_keys (S, z partials with a running shift per
// range), k_bw_merge (C_f; the sum, written as bf16 hi + lo row-major tiles),
// k_bw_query (dq; M_i, D_i, delta_i per query), k_bw_rstate (R, rho partials),
// k_bw_merge, k_bw_key (dk, dv).  Causal: k_bw_keys (segment states), k_bw_cmax
// (C_f), k_bw_query_causal (a forward chunk walk per segment), k_bw_rstate
// (segment partials of R, rho), k_bw_key_causal (a backward chunk walk).  bf16
// MFMA with fp32 accumulation; fp32 operands enter as bf16 hi + lo pairs, the
// bf16 inputs exactly.
#include <math.h>

#include "favor_bf16_common.h"
#include "favor_internal.h"
#include "favor_mfma.h"

namespace favor {
namespace bw {
namespace {

using bf16k::kD;
using bf16k::swz;
using bf16k::v_operand;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ int drow(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// 1 / D_i, and 0 where D_i = 0: a query whose visible keys all lie more than
// ~2^126 below the head's per-feature key maximum C_f in every feature (the
// range limit of the shift) then contributes nothing: dq_i = 0 and no share of
// R, rho.  NaN stays NaN.
__device__ __forceinline__ float recip_or_zero(float D) { return D == 0.f ? 0.f : 1.f / D; }

template <typename X>
__device__ __forceinline__ void split8(const X& x, int kb, u32x4& hi, u32x4& lo) {
  uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
  split_bf16(x[8 * kb + 0], x[8 * kb + 1], h0, l0);
  split_bf16(x[8 * kb + 2], x[8 * kb + 3], h1, l1);
  split_bf16(x[8 * kb + 4], x[8 * kb + 5], h2, l2);
  split_bf16(x[8 * kb + 6], x[8 * kb + 7], h3, l3);
  hi = u32x4{h0, h1, h2, h3};
  lo = u32x4{l0, l1, l2, l3};
}

// Row-major [rows][64] bf16 arrays are kept as swizzled 64-row tiles: element
// (r, c) lives in 16-byte chunk c / 8 of row r % 64 of tile r / 64.
__device__ __forceinline__ int tile_at(int r, int chunk) { return (r >> 6) * 4096 + swz(r & 63, chunk); }

// A operand of rows r0 .. r0+31 of a tiled array, k-step ks: lane l holds row
// r0 + l % 32, columns 16ks + 8(l/32) .. +7.
__device__ __forceinline__ u32x4 rows_operand(const uint16_t* tiles, int r0, int lane, int ks) {
  return *reinterpret_cast<const u32x4*>(tiles + tile_at(r0 + (lane & 31), 2 * ks + (lane >> 5)));
}
// B operand (k = rows r0 + 16kb .. in MFMA register order, n = columns 32dt ..)
// of a tiled array, by the LDS transpose read.
__device__ __forceinline__ u32x4 cols_operand(const uint16_t* tiles, int r0, int kb, int dt, int lane) {
  return v_operand(tiles + (r0 >> 6) * 4096, (r0 & 63) + 16 * kb, dt, lane);
}

// 8 consecutive fp32 values as bf16 hi and lo words.
__device__ __forceinline__ void split_row8(const float* p, u32x4& hi, u32x4& lo) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  split8(x, 0, hi, lo);
}

// ---------------------------------------------------------------------------
// k_bw_keys<M>: the key state of one key range of one (b, h); M/32 waves, wave w
// owns features [32w, 32w+32).  Per 64 keys: K and V tiles and |k|^2 in LDS;
// each wave projects the two 32-key halves to TF tiles (lane = feature,
// register = key), e_jf = log2e (w_f.k_j - |k_j|^2/2).  The range keeps a
// running maximum m_f of e_jf: when a half raises it, z and S so far are scaled
// by 2^(m_old - m_new) (a factor per feature; S's registers, a feature each,
// take theirs through the wave's LDS row).  Then b_jf = 2^(e_jf - m_f), z += b,
// S += b^T V with b as bf16 hi + lo.  Out: part_S, part_z and m_f -> cpart, so
// that a range's sums times 2^(m_f - C_f) are its share at any shift C_f >= m_f.
// ---------------------------------------------------------------------------
template <int M>
__global__ __launch_bounds__(2 * M) __attribute__((amdgpu_waves_per_eu(M == 256 ? 4 : 1))) void k_bw_keys(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                   const uint16_t* __restrict__ W, float* __restrict__ cpart,
                                                   float* __restrict__ part_S, float* __restrict__ part_z, int H,
                                                   int n, int splits, int span) {
  constexpr int NT = 2 * M, NW = M / 32;
  constexpr int CPT = 1024 / NT;
  __shared__ __attribute__((aligned(16))) uint16_t kt[64 * 64];
  __shared__ __attribute__((aligned(16))) uint16_t vt[64 * 64];
  __shared__ float kk[64];
  __shared__ __attribute__((aligned(16))) float fac[NW][32];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, h = lane >> 5;
  const int bh = blockIdx.x / splits, sp = blockIdx.x % splits, hh = bh % H;
  const int j0 = sp * span, j1 = min(n, j0 + span);
  const int fb = 32 * wave, f = fb + (lane & 31);
  u32x4 wop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    wop[ks] = *reinterpret_cast<const u32x4*>(W + (static_cast<size_t>(hh) * M + f) * kD + 16 * ks + 8 * h);

  const size_t rowbase = static_cast<size_t>(bh) * n;
  u32x4 pre[CPT];
  auto fetch = [&](int tok0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = t + NT * i, mat = c >> 9, r = (c >> 3) & 63, ch = c & 7;
      pre[i] = tok0 + r < j1 ? *reinterpret_cast<const u32x4*>((mat ? V : K) + (rowbase + tok0 + r) * kD + 8 * ch)
                             : u32x4{0u, 0u, 0u, 0u};
    }
  };

  f32x16 acc[2] = {};
  float zp = 0.f, mrun = kNegInf;
  if (j0 < j1) fetch(j0);
  for (int tok0 = j0; tok0 < j1; tok0 += 64) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = t + NT * i, mat = c >> 9, r = (c >> 3) & 63, ch = c & 7;
      *reinterpret_cast<u32x4*>((mat ? vt : kt) + swz(r, ch)) = pre[i];
    }
    __syncthreads();
    if (t < 64) {
      float sq = 0.f;
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(kt + swz(t, ch));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = bf16_lo_as_f32(x[e]), hi = bf16_hi_as_f32(x[e]);
          sq = fmaf(lo, lo, sq);
          sq = fmaf(hi, hi, sq);
        }
      }
      kk[t] = sq;
    }
    __syncthreads();
    if (tok0 + 64 < j1) fetch(tok0 + 64);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      // exponents of this 32-key half and their maximum per feature
      f32x16 pr = {};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 xk = *reinterpret_cast<const u32x4*>(kt + swz(32 * st + (lane & 31), 2 * ks + h));
        pr = mfma_bf16(as_bf16x8(xk), as_bf16x8(wop[ks]), pr);
      }
      float e[16], tm = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 32 * st + drow(i, lane);
        e[i] = tok0 + r < j1 ? kLog2e * fmaf(-0.5f, kk[r], pr[i]) : kNegInf;
        tm = fmaxf(tm, e[i]);
      }
      tm = pair_max(tm);
      // the running maximum and the rescale of the sums so far (a factor of one
      // when the maximum stays; the first half scales the zero sums by zero)
      const float mnew = fmaxf(mrun, tm);
      const float sc = fast_exp2(mrun - mnew);
      mrun = mnew;
      zp *= sc;
      if (lane < 32) fac[wave][lane] = sc;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(&fac[wave][8 * j + 4 * h]);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[dt][4 * j + q] *= v4[q];
      }
      __builtin_amdgcn_wave_barrier();
      float bv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        bv[i] = fast_exp2(e[i] - mrun);   // 0 for keys past the end
        zp += bv[i];
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        u32x4 ahi, alo;
        split8(bv, kb, ahi, alo);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const u32x4 vb = v_operand(vt, 32 * st + 16 * kb, dt, lane);
          acc[dt] = mfma_bf16(as_bf16x8(ahi), as_bf16x8(vb), acc[dt]);
          acc[dt] = mfma_bf16(as_bf16x8(alo), as_bf16x8(vb), acc[dt]);
        }
      }
    }
  }
  const size_t slot = static_cast<size_t>(bh) * splits + sp;
  float* PS = part_S + slot * M * kD;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) PS[(fb + drow(i, lane)) * kD + 32 * dt + (lane & 31)] = acc[dt][i];
  zp = pair_sum(zp);
  if (lane < 32) {
    part_z[slot * M + f] = zp;
    cpart[slot * M + f] = mrun;
  }
}

// ---------------------------------------------------------------------------
// k_bw_merge: the ranges of one (b, h) summed in index order; the m x 64 sum as
// bf16 hi + lo tiled arrays and the m-vector in fp32.  With cpart (the ranges'
// key shifts m_r): C_f = max_r m_r -> cfin, and range r enters at 2^(m_r - C_f).
// One workgroup per (b, h, 4 rows).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bw_merge(const float* __restrict__ part, const float* __restrict__ pvec,
                                                  uint16_t* __restrict__ tiles, float* __restrict__ vec,
                                                  const float* __restrict__ cpart, float* __restrict__ cfin, int BH,
                                                  int M, int splits) {
  const int q4 = M / 4;
  const int bh = blockIdx.x / q4, r = (blockIdx.x % q4) * 4 + (threadIdx.x >> 6), c = threadIdx.x & 63;
  // with cpart: each range's sums carry the shift m_r, and enter at 2^(m_r - C)
  float C = 0.f, a = 0.f, s = 0.f;
  const float* P = part + (static_cast<size_t>(bh) * splits * M + r) * kD + c;
  const float* Z = pvec + static_cast<size_t>(bh) * splits * M + r;
  const float* CP = cpart ? cpart + static_cast<size_t>(bh) * splits * M + r : nullptr;
  if (splits <= 16) {
    // every range's values read at once, then combined in index order (slots past
    // the ranges add exact zeros)
    float pv[16], zv[16], mv[16];
#pragma unroll
    for (int sp = 0; sp < 16; ++sp) {
      const bool in = sp < splits;
      pv[sp] = in ? P[static_cast<size_t>(sp) * M * kD] : 0.f;
      zv[sp] = in ? Z[static_cast<size_t>(sp) * M] : 0.f;
      mv[sp] = in && CP ? CP[static_cast<size_t>(sp) * M] : kNegInf;
    }
    if (CP) {
      C = kNegInf;
#pragma unroll
      for (int sp = 0; sp < 16; ++sp) C = fmaxf(C, mv[sp]);
    }
#pragma unroll
    for (int sp = 0; sp < 16; ++sp) {
      const float w = CP ? fast_exp2(mv[sp] - C) : 1.f;
      a = fmaf(pv[sp], w, a);
      s = fmaf(zv[sp], w, s);
    }
  } else {
    if (CP) {
      C = kNegInf;
      for (int sp = 0; sp < splits; ++sp) C = fmaxf(C, CP[static_cast<size_t>(sp) * M]);
    }
#pragma unroll 8
    for (int sp = 0; sp < splits; ++sp) {
      const float w = CP ? fast_exp2(CP[static_cast<size_t>(sp) * M] - C) : 1.f;
      a = fmaf(P[static_cast<size_t>(sp) * M * kD], w, a);
      s = fmaf(Z[static_cast<size_t>(sp) * M], w, s);
    }
  }
  const uint32_t pk = pack_bf16(a, 0.f);
  const uint16_t hi = static_cast<uint16_t>(pk & 0xffffu);
  const uint16_t lo = static_cast<uint16_t>(pack_bf16(a - bf16_lo_as_f32(pk), 0.f) & 0xffffu);
  const size_t base = static_cast<size_t>(bh) * M * kD + tile_at(r, c >> 3) + (c & 7);
  tiles[base] = hi;
  tiles[static_cast<size_t>(BH) * M * kD + base] = lo;
  if (c == 0) {
    vec[static_cast<size_t>(bh) * M + r] = s;
    if (cpart) cfin[static_cast<size_t>(bh) * M + r] = C;
  }
}

// k_bw_cmax: the largest key exponent per (b, h, feature) over the ranges.
__global__ __launch_bounds__(256) void k_bw_cmax(const float* __restrict__ cpart, float* __restrict__ cfin, int total,
                                                 int M, int splits) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int bh = i / M, f = i % M;
  float m = kNegInf;
  for (int sp = 0; sp < splits; ++sp) m = fmaxf(m, cpart[(static_cast<size_t>(bh) * splits + sp) * M + f]);
  cfin[i] = m;
}

// Stage a (b, h)'s tiled bf16 hi / lo array, W (tiled) and two m-vectors in LDS.
template <int M>
__device__ __forceinline__ void stage_common(uint16_t (&th)[2][M * kD], uint16_t (&wl)[M * kD], float (&v0)[M],
                                             float (&v1)[M], const uint16_t* tiles, const uint16_t* W,
                                             const float* g0, const float* g1, int BH, int bh, int hh, int t,
                                             int NT) {
  const u32x4* sh = reinterpret_cast<const u32x4*>(tiles + static_cast<size_t>(bh) * M * kD);
  const u32x4* sl = reinterpret_cast<const u32x4*>(tiles + (static_cast<size_t>(BH) + bh) * M * kD);
  for (int i = t; i < M * 8; i += NT) {
    reinterpret_cast<u32x4*>(th[0])[i] = sh[i];
    reinterpret_cast<u32x4*>(th[1])[i] = sl[i];
  }
  const uint16_t* Wh = W + static_cast<size_t>(hh) * M * kD;
  for (int c = t; c < M * 8; c += NT)
    *reinterpret_cast<u32x4*>(wl + tile_at(c >> 3, c & 7)) = *reinterpret_cast<const u32x4*>(Wh + 8 * c);
  for (int i = t; i < M; i += NT) {
    v0[i] = g0[static_cast<size_t>(bh) * M + i];
    v1[i] = g1[static_cast<size_t>(bh) * M + i];
  }
}

// ---------------------------------------------------------------------------
// k_bw_query: dq, and M_i, D_i, delta_i per query (aux [BH][n][4]).  8 waves;
// each wave takes 32-query tiles of its (b, h) and walks the feature tiles once
// for a (FT: lane = query), D_i, T = S dy (three MFMAs per k-step against S hi /
// lo), G and the product G W, with the first feature tile's row maximum as the
// shift M_i (a second walk with the exact maximum when some a_if exceeds 2^64).
// ---------------------------------------------------------------------------
template <int M>
__global__ __launch_bounds__(512) void k_bw_query(const uint16_t* __restrict__ Q, const float* __restrict__ Y,
                                                  const float* __restrict__ dY, const uint16_t* __restrict__ W,
                                                  const uint16_t* __restrict__ stiles, const float* __restrict__ zg,
                                                  const float* __restrict__ cfin, float* __restrict__ dQ,
                                                  float* __restrict__ aux, int BH, int H, int n, int qblocks) {
  constexpr int NWV = 8;
  __shared__ __attribute__((aligned(16))) uint16_t sl[2][M * kD];
  __shared__ __attribute__((aligned(16))) uint16_t wl[M * kD];
  __shared__ __attribute__((aligned(16))) float zl[M];
  __shared__ __attribute__((aligned(16))) float cl[M];
  __shared__ float rdl[NWV][32], gsl[NWV][32];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, h = lane >> 5;
  const int bh = blockIdx.x / qblocks, qb = blockIdx.x % qblocks, hh = bh % H;
  stage_common<M>(sl, wl, zl, cl, stiles, W, zg, cfin, BH, bh, hh, t, 512);
  __syncthreads();

  const int ntiles = (n + 31) / 32;
  const size_t rowbase = static_cast<size_t>(bh) * n;
  for (int tile = qb * NWV + wave; tile < ntiles; tile += qblocks * NWV) {
    const int row = 32 * tile + (lane & 31);
    const bool ok = row < n;
    u32x4 xq[4], dyh[4], dyl[4];
    float dl = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c0 = 16 * ks + 8 * h;
      if (ok) {
        xq[ks] = *reinterpret_cast<const u32x4*>(Q + (rowbase + row) * kD + c0);
        const float* dp = dY + (rowbase + row) * kD + c0;
        const float* yp = Y + (rowbase + row) * kD + c0;
        split_row8(dp, dyh[ks], dyl[ks]);
#pragma unroll
        for (int e = 0; e < 8; ++e) dl = fmaf(dp[e], yp[e], dl);
      } else {
        xq[ks] = dyh[ks] = dyl[ks] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    const float delta = pair_sum(dl);
    // the row maximum of g over all features, from the projections
    auto row_max = [&](int nft) {
      float mx = kNegInf;
#pragma unroll 1
      for (int ft = 0; ft < nft; ++ft) {
        f32x16 pr = {};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          pr = mfma_bf16(as_bf16x8(rows_operand(wl, 32 * ft, lane, ks)), as_bf16x8(xq[ks]), pr);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 cc = *reinterpret_cast<const f32x4*>(&cl[32 * ft + 8 * j + 4 * h]);
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaf(kLog2e, pr[4 * j + e], cc[e]));
        }
      }
      return pair_max(mx);
    };
    f32x16 acc[2];
    float Dp, Gs, tmax;
    auto accumulate = [&](float Ms) {
      acc[0] = acc[1] = f32x16{};
      Dp = Gs = 0.f;
      tmax = kNegInf;
#pragma unroll 1
      for (int ft = 0; ft < M / 32; ++ft) {
        f32x16 pr = {}, tacc = {};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          pr = mfma_bf16(as_bf16x8(rows_operand(wl, 32 * ft, lane, ks)), as_bf16x8(xq[ks]), pr);
          const u32x4 ah = rows_operand(sl[0], 32 * ft, lane, ks), al = rows_operand(sl[1], 32 * ft, lane, ks);
          tacc = mfma_bf16(as_bf16x8(ah), as_bf16x8(dyh[ks]), tacc);
          tacc = mfma_bf16(as_bf16x8(ah), as_bf16x8(dyl[ks]), tacc);
          tacc = mfma_bf16(as_bf16x8(al), as_bf16x8(dyh[ks]), tacc);
        }
        float G[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 cc = *reinterpret_cast<const f32x4*>(&cl[32 * ft + 8 * j + 4 * h]);
          const f32x4 zz = *reinterpret_cast<const f32x4*>(&zl[32 * ft + 8 * j + 4 * h]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ge = fmaf(kLog2e, pr[4 * j + e], cc[e]) - Ms;
            tmax = fmaxf(tmax, ge);
            const float a = fast_exp2(ge);
            Dp = fmaf(a, zz[e], Dp);
            G[4 * j + e] = a * fmaf(-zz[e], delta, tacc[4 * j + e]);
            Gs += G[4 * j + e];
          }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          u32x4 gh, gl;
          split8(G, kb, gh, gl);
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) {
            const u32x4 wb = cols_operand(wl, 32 * ft, kb, dt, lane);
            acc[dt] = mfma_bf16(as_bf16x8(gh), as_bf16x8(wb), acc[dt]);
            acc[dt] = mfma_bf16(as_bf16x8(gl), as_bf16x8(wb), acc[dt]);
          }
        }
      }
    };
    // The shift M_i is the first feature tile's row maximum: any per-row constant
    // cancels, and the a_if above 1 that it leaves are bounded by 2^64 (checked);
    // beyond that the exact maximum is taken and the tile redone.
    float Mi = row_max(1);
    accumulate(Mi);
    if (__ballot(tmax > 64.f) != 0) {
      Mi = row_max(M / 32);
      accumulate(Mi);
    }
    const float Di = pair_sum(Dp), Gsum = pair_sum(Gs);
    if (lane < 32) {
      rdl[wave][lane] = recip_or_zero(Di);
      gsl[wave][lane] = Gsum;
      if (ok) *reinterpret_cast<f32x4*>(aux + (rowbase + row) * 4) = f32x4{Mi, Di, delta, 0.f};
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = drow(i, lane), r = 32 * tile + q;
      if (r < n) {
        const float rq = rdl[wave][q], gq = gsl[wave][q];
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const int c = 32 * dt + (lane & 31);
          const float qv = __uint_as_float(static_cast<uint32_t>(Q[(rowbase + r) * kD + c]) << 16);
          dQ[(rowbase + r) * kD + c] = (acc[dt][i] - qv * gq) * rq;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------------------
// k_bw_rstate: R = sum_i (a_i / D_i) dy_i^T and rho = sum_i (a_i / D_i) delta_i
// over one query range; M/32 waves, wave w owns features [32w, 32w+32).  Per 64
// queries (read one tile ahead into registers): Q, dY (as bf16 hi and lo tiles)
// and (M_i, 1 / D_i, delta_i) in LDS; per 32 queries a TF projection gives
// a_if / D_i, which enters as bf16 hi + lo.
// ---------------------------------------------------------------------------
template <int M>
__global__ __launch_bounds__(2 * M) void k_bw_rstate(const uint16_t* __restrict__ Q, const float* __restrict__ dY,
                                                     const uint16_t* __restrict__ W, const float* __restrict__ cfin,
                                                     const float* __restrict__ aux, float* __restrict__ part_R,
                                                     float* __restrict__ part_rho, int H, int n, int splits,
                                                     int span) {
  constexpr int NT = 2 * M;
  __shared__ __attribute__((aligned(16))) uint16_t qt[64 * 64];
  __shared__ __attribute__((aligned(16))) uint16_t dh[64 * 64];
  __shared__ __attribute__((aligned(16))) uint16_t dlo[64 * 64];
  __shared__ __attribute__((aligned(16))) f32x4 ax[64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, h = lane >> 5;
  const int bh = blockIdx.x / splits, sp = blockIdx.x % splits, hh = bh % H;
  const int j0 = sp * span, j1 = min(n, j0 + span);
  const int fb = 32 * wave, f = fb + (lane & 31);
  u32x4 wop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    wop[ks] = *reinterpret_cast<const u32x4*>(W + (static_cast<size_t>(hh) * M + f) * kD + 16 * ks + 8 * h);
  const float C = cfin[static_cast<size_t>(bh) * M + f];
  const size_t rowbase = static_cast<size_t>(bh) * n;

  // a 64-query tile's reads, held in registers while the previous tile computes:
  // Q (64 rows x 8 chunks), dY (64 rows x 8 groups of 8 floats), (M, D, delta)
  constexpr int QN = 512 / NT;
  u32x4 pq[QN];
  f32x4 pdy[2 * QN], pa = {0.f, 1.f, 0.f, 0.f};
  auto fetch = [&](int tok0) {
#pragma unroll
    for (int i = 0; i < QN; ++i) {
      const int c = t + NT * i, r = c >> 3, ch = c & 7;
      const bool ok = tok0 + r < j1;
      const size_t row = rowbase + tok0 + r;
      pq[i] = ok ? *reinterpret_cast<const u32x4*>(Q + row * kD + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
      pdy[2 * i] = ok ? *reinterpret_cast<const f32x4*>(dY + row * kD + 8 * ch) : f32x4{0.f, 0.f, 0.f, 0.f};
      pdy[2 * i + 1] = ok ? *reinterpret_cast<const f32x4*>(dY + row * kD + 8 * ch + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (t < 64)
      pa = tok0 + t < j1 ? *reinterpret_cast<const f32x4*>(aux + (rowbase + tok0 + t) * 4) : f32x4{0.f, 1.f, 0.f, 0.f};
  };

  f32x16 acc[2] = {};
  float rp = 0.f;
  if (j0 < j1) fetch(j0);
  for (int tok0 = j0; tok0 < j1; tok0 += 64) {
    __syncthreads();   // the previous tile's reads of LDS are done
#pragma unroll
    for (int i = 0; i < QN; ++i) {   // Q; dY as bf16 hi and lo
      const int c = t + NT * i, r = c >> 3, ch = c & 7;
      *reinterpret_cast<u32x4*>(qt + swz(r, ch)) = pq[i];
      const float x[8] = {pdy[2 * i][0], pdy[2 * i][1], pdy[2 * i][2], pdy[2 * i][3],
                          pdy[2 * i + 1][0], pdy[2 * i + 1][1], pdy[2 * i + 1][2], pdy[2 * i + 1][3]};
      u32x4 hi, lo;
      split8(x, 0, hi, lo);
      *reinterpret_cast<u32x4*>(dh + swz(r, ch)) = hi;
      *reinterpret_cast<u32x4*>(dlo + swz(r, ch)) = lo;
    }
    if (t < 64) ax[t] = f32x4{pa[0], recip_or_zero(pa[1]), pa[2], 0.f};   // (M_i, 1 / D_i, delta_i)
    __syncthreads();
    if (tok0 + 64 < j1) fetch(tok0 + 64);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x16 pr = {};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 xq = *reinterpret_cast<const u32x4*>(qt + swz(32 * st + (lane & 31), 2 * ks + h));
        pr = mfma_bf16(as_bf16x8(xq), as_bf16x8(wop[ks]), pr);
      }
      float cf[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 32 * st + drow(i, lane);
        const f32x4 a = ax[r];   // M_i, 1 / D_i, delta_i
        const float x = fast_exp2(fmaf(kLog2e, pr[i], C) - a[0]) * a[1];
        cf[i] = tok0 + r < j1 ? x : 0.f;
        rp = fmaf(cf[i], a[2], rp);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        u32x4 chi, clo;
        split8(cf, kb, chi, clo);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const u32x4 bh_ = v_operand(dh, 32 * st + 16 * kb, dt, lane);
          const u32x4 bl_ = v_operand(dlo, 32 * st + 16 * kb, dt, lane);
          acc[dt] = mfma_bf16(as_bf16x8(chi), as_bf16x8(bh_), acc[dt]);
          acc[dt] = mfma_bf16(as_bf16x8(chi), as_bf16x8(bl_), acc[dt]);
          acc[dt] = mfma_bf16(as_bf16x8(clo), as_bf16x8(bh_), acc[dt]);
        }
      }
    }
  }
  const size_t slot = static_cast<size_t>(bh) * splits + sp;
  float* PR = part_R + slot * M * kD;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) PR[(fb + drow(i, lane)) * kD + 32 * dt + (lane & 31)] = acc[dt][i];
  rp = pair_sum(rp);
  if (lane < 32) part_rho[slot * M + f] = rp;
}

// ---------------------------------------------------------------------------
// k_bw_key: dk and dv.  8 waves; each wave takes 32-key tiles and walks the
// feature tiles: b (FT: lane = key), dv += b R (three MFMAs against R hi / lo),
// R v (FT, two MFMAs), H = b (R v - rho), dk += H W.
// ---------------------------------------------------------------------------
template <int M>
__global__ __launch_bounds__(512) void k_bw_key(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                const uint16_t* __restrict__ W, const uint16_t* __restrict__ rtiles,
                                                const float* __restrict__ rho, const float* __restrict__ cfin,
                                                float* __restrict__ dK, float* __restrict__ dV, int BH, int H, int n,
                                                int qblocks) {
  constexpr int NWV = 8;
  __shared__ __attribute__((aligned(16))) uint16_t rl[2][M * kD];
  __shared__ __attribute__((aligned(16))) uint16_t wl[M * kD];
  __shared__ __attribute__((aligned(16))) float pl[M];
  __shared__ __attribute__((aligned(16))) float cl[M];
  __shared__ float hsl[NWV][32];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, h = lane >> 5;
  const int bh = blockIdx.x / qblocks, qb = blockIdx.x % qblocks, hh = bh % H;
  stage_common<M>(rl, wl, pl, cl, rtiles, W, rho, cfin, BH, bh, hh, t, 512);
  __syncthreads();

  const int ntiles = (n + 31) / 32;
  const size_t rowbase = static_cast<size_t>(bh) * n;
  for (int tile = qb * NWV + wave; tile < ntiles; tile += qblocks * NWV) {
    const int row = 32 * tile + (lane & 31);
    const bool ok = row < n;
    u32x4 xk[4], xv[4];
    float kp = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c0 = 16 * ks + 8 * h;
      xk[ks] = ok ? *reinterpret_cast<const u32x4*>(K + (rowbase + row) * kD + c0) : u32x4{0u, 0u, 0u, 0u};
      xv[ks] = ok ? *reinterpret_cast<const u32x4*>(V + (rowbase + row) * kD + c0) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_lo_as_f32(xk[ks][e]), hi = bf16_hi_as_f32(xk[ks][e]);
        kp = fmaf(lo, lo, kp);
        kp = fmaf(hi, hi, kp);
      }
    }
    const float kk = pair_sum(kp);
    f32x16 adv[2] = {}, adk[2] = {};
    float Hs = 0.f;
    for (int ft = 0; ft < M / 32; ++ft) {
      f32x16 pr = {}, rv = {};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        pr = mfma_bf16(as_bf16x8(rows_operand(wl, 32 * ft, lane, ks)), as_bf16x8(xk[ks]), pr);
        rv = mfma_bf16(as_bf16x8(rows_operand(rl[0], 32 * ft, lane, ks)), as_bf16x8(xv[ks]), rv);
        rv = mfma_bf16(as_bf16x8(rows_operand(rl[1], 32 * ft, lane, ks)), as_bf16x8(xv[ks]), rv);
      }
      float b[16], Hh[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 cc = *reinterpret_cast<const f32x4*>(&cl[32 * ft + 8 * j + 4 * h]);
        const f32x4 pp = *reinterpret_cast<const f32x4*>(&pl[32 * ft + 8 * j + 4 * h]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          b[4 * j + e] = ok ? fast_exp2(kLog2e * fmaf(-0.5f, kk, pr[4 * j + e]) - cc[e]) : 0.f;
          Hh[4 * j + e] = b[4 * j + e] * (rv[4 * j + e] - pp[e]);
          Hs += Hh[4 * j + e];
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        u32x4 bhi, blo, hhi, hlo;
        split8(b, kb, bhi, blo);
        split8(Hh, kb, hhi, hlo);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const u32x4 rh = cols_operand(rl[0], 32 * ft, kb, dt, lane);
          const u32x4 rlo = cols_operand(rl[1], 32 * ft, kb, dt, lane);
          adv[dt] = mfma_bf16(as_bf16x8(bhi), as_bf16x8(rh), adv[dt]);
          adv[dt] = mfma_bf16(as_bf16x8(bhi), as_bf16x8(rlo), adv[dt]);
          adv[dt] = mfma_bf16(as_bf16x8(blo), as_bf16x8(rh), adv[dt]);
          const u32x4 wb = cols_operand(wl, 32 * ft, kb, dt, lane);
          adk[dt] = mfma_bf16(as_bf16x8(hhi), as_bf16x8(wb), adk[dt]);
          adk[dt] = mfma_bf16(as_bf16x8(hlo), as_bf16x8(wb), adk[dt]);
        }
      }
    }
    const float Hsum = pair_sum(Hs);
    if (lane < 32) hsl[wave][lane] = Hsum;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = drow(i, lane), r = 32 * tile + q;
      if (r < n) {
        const float hq = hsl[wave][q];
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const int c = 32 * dt + (lane & 31);
          const float kv = __uint_as_float(static_cast<uint32_t>(K[(rowbase + r) * kD + c]) << 16);
          dK[(rowbase + r) * kD + c] = adk[dt][i] - kv * hq;
          dV[(rowbase + r) * kD + c] = adv[dt][i];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ===========================================================================
// Causal backward: the sums run over j <= i (S, z: prefix sums of the keys)
// and i >= j (R, rho: suffix sums of the queries).  Both kernels walk one
// segment of one (b, h) in chunks of 32 tokens; M/32 waves, wave w owns
// features [32w, 32w+32).  Each wave forms its features' share of every
// per-token quantity; the shares are summed in wave order in LDS.  The query
// side keeps S transposed (S^T[c][f]: lane = feature, register = value column),
// the A operand of S.dy, so the value columns of dy are read in the MFMA
// register order: k-block kb of 16 columns, lane half h: columns 16kb + 4h .. +3
// and 16kb + 8 + 4h .. +3.
// ===========================================================================
// bf16 (1, 0) per register pair of a k-block: 1 where key drow <= query, for the
// B operand of the running sum over the keys of the chunk.
__device__ __forceinline__ u32x4 tril_ones(int kb, int q, int lane) {
  uint32_t w[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r0 = drow(8 * kb + 2 * p, lane), r1 = drow(8 * kb + 2 * p + 1, lane);
    w[p] = (r0 <= q ? bf16k::kBf16One : 0u) | ((r1 <= q ? bf16k::kBf16One : 0u) << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// One 32-token chunk of a (b, h) in LDS, staged once per workgroup: q, k, v and
// dy (as three bf16 words hi, mid, lo) in swizzled row-major [32][64] bf16 tiles,
// |k|^2 per key, and per token delta_i (dy.y, formed here on the query side) and,
// on the key side, M_i and 1 / D_i; each a separate array, so that the 4
// consecutive tokens of an MFMA register group come in one vector read.  Rows
// past the end are zero (1 / D_i: one).
struct ChunkBuf {
  uint16_t q[32 * 64], k[32 * 64], v[32 * 64], dh[32 * 64], dm[32 * 64], dl[32 * 64];
  float am[32], ar[32], ad[32], kk[32];
};
// Values of a per-token array for the 16 rows drow(i, lane) of a D tile.
__device__ __forceinline__ void rows16(const float* a, int h, float (&x)[16]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(a + 8 * j + 4 * h);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * j + e] = v[e];
  }
}

// The chunk's global reads, held in registers between chunks so that they are in
// flight while the previous chunk computes.  16-byte pieces: 768 of q, k, v
// (32 rows x 8 per matrix), 512 of dy (32 rows x 16), as many of y (query side).
template <int NT, bool QSIDE>
struct ChunkRegs {
  static constexpr int NB = (768 + NT - 1) / NT, ND = (512 + NT - 1) / NT;
  u32x4 b[NB];
  f32x4 dy[ND];
  f32x4 y[QSIDE ? ND : 1];
  f32x4 ax;
};

template <int NT, bool QSIDE>
__device__ __forceinline__ void chunk_load(ChunkRegs<NT, QSIDE>& R, const uint16_t* Q, const uint16_t* K,
                                           const uint16_t* V, const float* dY, const float* Y, const float* aux,
                                           size_t rowbase, int c0, int t1, int t) {
#pragma unroll
  for (int i = 0; i < R.NB; ++i) {
    const int c = t + NT * i;
    if (c < 768) {   // uniform per wave (NT and 256 are multiples of 64)
      const int mat = c >> 8, r = (c >> 3) & 31, ch = c & 7;
      const uint16_t* src = mat == 0 ? Q : (mat == 1 ? K : V);
      R.b[i] = c0 + r < t1 ? *reinterpret_cast<const u32x4*>(src + (rowbase + c0 + r) * kD + 8 * ch)
                           : u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int i = 0; i < R.ND; ++i) {
    const int c = t + NT * i;
    if (c < 512) {
      const int r = c >> 4, c4 = (c & 15) * 4;
      const bool ok = c0 + r < t1;
      R.dy[i] = ok ? *reinterpret_cast<const f32x4*>(dY + (rowbase + c0 + r) * kD + c4) : f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (QSIDE)
        R.y[i] = ok ? *reinterpret_cast<const f32x4*>(Y + (rowbase + c0 + r) * kD + c4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  if constexpr (!QSIDE) {
    if (t < 32) R.ax = c0 + t < t1 ? *reinterpret_cast<const f32x4*>(aux + (rowbase + c0 + t) * 4) : f32x4{0.f, 1.f, 0.f, 0.f};
  }
}

template <int NT, bool QSIDE>
__device__ __forceinline__ void chunk_store(const ChunkRegs<NT, QSIDE>& R, ChunkBuf& B, int t) {
#pragma unroll
  for (int i = 0; i < R.NB; ++i) {
    const int c = t + NT * i;
    if (c < 768) {
      const int mat = c >> 8, r = (c >> 3) & 31, ch = c & 7;
      uint16_t* dst = mat == 0 ? B.q : (mat == 1 ? B.k : B.v);
      *reinterpret_cast<u32x4*>(dst + swz(r, ch)) = R.b[i];
      if (mat == 1) {   // |k|^2: the 8 lanes of one row
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = bf16_lo_as_f32(R.b[i][e]), hi = bf16_hi_as_f32(R.b[i][e]);
          s = fmaf(lo, lo, s);
          s = fmaf(hi, hi, s);
        }
        s = sum8(s);
        if ((t & 7) == 0) B.kk[r] = s;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < R.ND; ++i) {
    const int c = t + NT * i;
    if (c < 512) {
      const int r = c >> 4, c4 = (c & 15) * 4;
      const f32x4 x = R.dy[i];
      uint32_t h0, m0, h1, m1;
      split_bf16(x[0], x[1], h0, m0);
      split_bf16(x[2], x[3], h1, m1);
      const uint32_t l0 = pack_bf16(x[0] - bf16_lo_as_f32(h0) - bf16_lo_as_f32(m0),
                                    x[1] - bf16_hi_as_f32(h0) - bf16_hi_as_f32(m0));
      const uint32_t l1 = pack_bf16(x[2] - bf16_lo_as_f32(h1) - bf16_lo_as_f32(m1),
                                    x[3] - bf16_hi_as_f32(h1) - bf16_hi_as_f32(m1));
      const int off = swz(r, c4 >> 3) + (c4 & 7);
      *reinterpret_cast<u32x2*>(B.dh + off) = u32x2{h0, h1};
      *reinterpret_cast<u32x2*>(B.dm + off) = u32x2{m0, m1};
      *reinterpret_cast<u32x2*>(B.dl + off) = u32x2{l0, l1};
      if constexpr (QSIDE) {   // delta: the 16 lanes of one row
        const f32x4 y = R.y[i];
        float d = x[0] * y[0];
        d = fmaf(x[1], y[1], d);
        d = fmaf(x[2], y[2], d);
        d = fmaf(x[3], y[3], d);
        d = sum8(d);
        d += __shfl_xor(d, 8);
        if ((t & 15) == 0) B.ad[r] = d;
      }
    }
  }
  if constexpr (!QSIDE) {   // (M_i, 1 / D_i, delta_i)
    if (t < 32) {
      B.am[t] = R.ax[0];
      B.ar[t] = recip_or_zero(R.ax[1]);
      B.ad[t] = R.ax[2];
    }
  }
}

// Operands of token row `row` of a chunk tile: 8 columns 16ks + 8h .. (natural
// order) or the register order of a k-block (columns 16kb + 4h .. +3 and
// 16kb + 8 + 4h .. +3).
__device__ __forceinline__ u32x4 tile_row8(const uint16_t* tile, int row, int ks, int h) {
  return *reinterpret_cast<const u32x4*>(tile + swz(row, 2 * ks + h));
}
__device__ __forceinline__ u32x4 tile_perm8(const uint16_t* tile, int row, int kb, int h) {
  const u32x2 a = *reinterpret_cast<const u32x2*>(tile + swz(row, 2 * kb) + 4 * h);
  const u32x2 b = *reinterpret_cast<const u32x2*>(tile + swz(row, 2 * kb + 1) + 4 * h);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// ---------------------------------------------------------------------------
// k_bw_query_causal: dq and (M_i, D_i, delta_i) per query.  Wave w owns TPW
// feature tiles of 32 (features [32 TPW w, 32 TPW (w+1))).  Per chunk, wave w:
//   a_if = 2^(g_if - M_wi) (FT, M_wi the wave's row maximum over its features);
//   T_if - z_if delta_i = (S_f.dy_i - z_f delta_i over keys before the chunk,
//   S^T in registers) + sum over keys j <= i of the chunk b_jf (v_j.dy_i - delta_i);
//   D_w = sum_f a z,  Ghat = a (T - z delta),  u_w = sum_f Ghat,  U_w = Ghat W;
// then S^T, z take the chunk's keys.  Combine: scale_w = 2^(M_wi - M_i),
// dq_i = (sum_w scale_w U_w - q_i sum_w scale_w u_w) / sum_w scale_w D_w.
// The masked chunk matrix V dY^T - delta does not depend on the feature and is
// formed once per wave.  Chunks are staged in LDS (two buffers) with the next
// chunk's reads in flight.
// ---------------------------------------------------------------------------
template <int M, int TPW>
__global__ __launch_bounds__(M * 2 / TPW) void k_bw_query_causal(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ W, const float* __restrict__ Y, const float* __restrict__ dY,
    const float* __restrict__ cfin, const float* __restrict__ cpart, const float* __restrict__ part_S,
    const float* __restrict__ part_z, float* __restrict__ dQ, float* __restrict__ aux, int H, int n, int segs,
    int span) {
  constexpr int NW = M / (32 * TPW), NT = 64 * NW;
  __shared__ __attribute__((aligned(16))) uint16_t wl[M * kD];
  __shared__ __attribute__((aligned(16))) ChunkBuf buf[2];
  __shared__ __attribute__((aligned(16))) float ul[NW][32][kD];
  __shared__ float sl_u[NW][32], sl_d[NW][32], sl_m[NW][32];
  __shared__ __attribute__((aligned(16))) float zl[NW][TPW * 32];
  __shared__ __attribute__((aligned(16))) float cl[M];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, h = lane >> 5, ql = lane & 31;
  const int bh = blockIdx.x / segs, sg = blockIdx.x % segs, hh = bh % H;
  const int t0 = sg * span, t1 = min(n, t0 + span);
  const int fw = 32 * TPW * wave;   // the wave's first feature; tile p starts at fw + 32 p
  const size_t rowbase = static_cast<size_t>(bh) * n;
  ChunkRegs<NT, true> pre;
  chunk_load<NT, true>(pre, Q, K, V, dY, Y, nullptr, rowbase, t0, t1, t);
  const uint16_t* Wh = W + static_cast<size_t>(hh) * M * kD;
  for (int c = t; c < M * 8; c += NT)
    *reinterpret_cast<u32x4*>(wl + tile_at(c >> 3, c & 7)) = *reinterpret_cast<const u32x4*>(Wh + 8 * c);
  for (int i = t; i < M; i += NT) cl[i] = cfin[static_cast<size_t>(bh) * M + i];
  float C[TPW];
  // S^T (rows = value columns, lane = feature) and z per tile, of the keys before the range
  f32x16 St[TPW][2];
#pragma unroll
  for (int p = 0; p < TPW; ++p) {
    const int f = fw + 32 * p + ql;
    C[p] = cfin[static_cast<size_t>(bh) * M + f];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 16; ++i) St[p][ct][i] = 0.f;
    float z = 0.f;
    for (int s = 0; s < sg; ++s) {   // each range's sums at its own shift m_s: times 2^(m_s - C)
      const size_t slot = static_cast<size_t>(bh) * segs + s;
      const float w = fast_exp2(cpart[slot * M + f] - C[p]);
      const float* PS = part_S + slot * M * kD + static_cast<size_t>(f) * kD;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 16; ++i) St[p][ct][i] = fmaf(PS[32 * ct + drow(i, lane)], w, St[p][ct][i]);
      z = fmaf(part_z[slot * M + f], w, z);
    }
    if (lane < 32) zl[wave][32 * p + lane] = z;
  }
  chunk_store<NT, true>(pre, buf[0], t);
  if (t0 + 32 < t1) chunk_load<NT, true>(pre, Q, K, V, dY, Y, nullptr, rowbase, t0 + 32, t1, t);
  __syncthreads();

  int it = 0;
  for (int c0 = t0; c0 < t1; c0 += 32, ++it) {
    const ChunkBuf& B = buf[it & 1];
    if (c0 + 32 < t1) {
      chunk_store<NT, true>(pre, buf[(it + 1) & 1], t);
      if (c0 + 64 < t1) chunk_load<NT, true>(pre, Q, K, V, dY, Y, nullptr, rowbase, c0 + 64, t1, t);
    }
    // the phases below are kept apart (sched_barrier) so that each one's operands
    // are read from LDS when used and die after it
    // 1. per tile: key features b (TF: lane = feature, register = key), as bf16 hi / lo
    u32x4 bth[TPW][2], btl[TPW][2];
    float zs[TPW];
    {
      float kr[16];
      rows16(B.kk, h, kr);
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        f32x16 pkt = {};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          pkt = mfma_bf16(as_bf16x8(tile_row8(B.k, ql, ks, h)), as_bf16x8(rows_operand(wl, fw + 32 * p, lane, ks)),
                          pkt);
        float b[16];
        zs[p] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = drow(i, lane);
          const float x = fast_exp2(kLog2e * fmaf(-0.5f, kr[i], pkt[i]) - C[p]);
          b[i] = c0 + r < t1 ? x : 0.f;
          zs[p] += b[i];
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) split8(b, kb, bth[p][kb], btl[p][kb]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // 2. the chunk's part of T - z delta and of z (FT: lane = query): b^T N with
    // N = V dY^T - delta masked to keys j <= i (v_j.dy_i - delta_i = dy_i.(v_j - y_i),
    // formed once, before the product with b; dy to all its 24 bits)
    const float delta = B.ad[ql];
    f32x16 tacc[TPW], zacc[TPW];
    {
      f32x16 mvd = {};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 xv = tile_row8(B.v, ql, ks, h);
        mvd = mfma_bf16(as_bf16x8(xv), as_bf16x8(tile_row8(B.dh, ql, ks, h)), mvd);
        mvd = mfma_bf16(as_bf16x8(xv), as_bf16x8(tile_row8(B.dm, ql, ks, h)), mvd);
        mvd = mfma_bf16(as_bf16x8(xv), as_bf16x8(tile_row8(B.dl, ql, ks, h)), mvd);
      }
      float mm[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) mm[i] = drow(i, lane) <= ql ? mvd[i] - delta : 0.f;
      u32x4 mh[2], ml[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) split8(mm, kb, mh[kb], ml[kb]);
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        tacc[p] = f32x16{};
        zacc[p] = f32x16{};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          tacc[p] = mfma_bf16(as_bf16x8(bth[p][kb]), as_bf16x8(mh[kb]), tacc[p]);
          tacc[p] = mfma_bf16(as_bf16x8(bth[p][kb]), as_bf16x8(ml[kb]), tacc[p]);
          tacc[p] = mfma_bf16(as_bf16x8(btl[p][kb]), as_bf16x8(mh[kb]), tacc[p]);
          const u32x4 ones = tril_ones(kb, ql, lane);
          zacc[p] = mfma_bf16(as_bf16x8(bth[p][kb]), as_bf16x8(ones), zacc[p]);
          zacc[p] = mfma_bf16(as_bf16x8(btl[p][kb]), as_bf16x8(ones), zacc[p]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // 3. the carry: S^T x dy (dy hi / mid in register order)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const u32x4 dph = tile_perm8(B.dh, ql, kb, h), dpl = tile_perm8(B.dm, ql, kb, h);
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        u32x4 sh, slo;
        split8(St[p][kb >> 1], kb & 1, sh, slo);
        tacc[p] = mfma_bf16(as_bf16x8(sh), as_bf16x8(dph), tacc[p]);
        tacc[p] = mfma_bf16(as_bf16x8(sh), as_bf16x8(dpl), tacc[p]);
        tacc[p] = mfma_bf16(as_bf16x8(slo), as_bf16x8(dph), tacc[p]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // 4. a (FT), the wave's row maximum over its tiles, and the wave's shares
    f32x16 pq[TPW];
    float mx = kNegInf;
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
      const int fb = fw + 32 * p;
      pq[p] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        pq[p] = mfma_bf16(as_bf16x8(rows_operand(wl, fb, lane, ks)), as_bf16x8(tile_row8(B.q, ql, ks, h)), pq[p]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 cc = *reinterpret_cast<const f32x4*>(&cl[fb + 8 * j + 4 * h]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pq[p][4 * j + e] = fmaf(kLog2e, pq[p][4 * j + e], cc[e]);
          mx = fmaxf(mx, pq[p][4 * j + e]);
        }
      }
    }
    const float Mw = pair_max(mx);
    float Dp = 0.f, Gs = 0.f;
    f32x16 acc[2] = {};
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
      const int fb = fw + 32 * p;
      float G[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 zc = *reinterpret_cast<const f32x4*>(&zl[wave][32 * p + 8 * j + 4 * h]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * j + e;
          const float a = fast_exp2(pq[p][i] - Mw);
          Dp = fmaf(a, zc[e] + zacc[p][i], Dp);
          G[i] = a * fmaf(-zc[e], delta, tacc[p][i]);
          Gs += G[i];
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        u32x4 gh, gl;
        split8(G, kb, gh, gl);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const u32x4 wb = cols_operand(wl, fb, kb, dt, lane);
          acc[dt] = mfma_bf16(as_bf16x8(gh), as_bf16x8(wb), acc[dt]);
          acc[dt] = mfma_bf16(as_bf16x8(gl), as_bf16x8(wb), acc[dt]);
        }
      }
    }
    const float Dw = pair_sum(Dp), Gw = pair_sum(Gs);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) ul[wave][drow(i, lane)][32 * dt + ql] = acc[dt][i];
    if (lane < 32) {
      sl_u[wave][lane] = Gw;
      sl_d[wave][lane] = Dw;
      sl_m[wave][lane] = Mw;
    }
    __builtin_amdgcn_sched_barrier(0);
    // 5. the chunk's keys join S^T and z
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const u32x4 va = v_operand(B.v, 16 * kb, ct, lane);
#pragma unroll
        for (int p = 0; p < TPW; ++p) {
          St[p][ct] = mfma_bf16(as_bf16x8(va), as_bf16x8(bth[p][kb]), St[p][ct]);
          St[p][ct] = mfma_bf16(as_bf16x8(va), as_bf16x8(btl[p][kb]), St[p][ct]);
        }
      }
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
      const float zsum = pair_sum(zs[p]);
      if (lane < 32) zl[wave][32 * p + lane] += zsum;
    }
    __syncthreads();   // shares visible
    // combine: thread -> one query and CPQ columns
    {
      constexpr int CPQ = 32 * kD / NT;
      const int q = t / (kD / CPQ), cb = (t % (kD / CPQ)) * CPQ, r = c0 + q;
      float Mq = sl_m[0][q];
#pragma unroll
      for (int w = 1; w < NW; ++w) Mq = fmaxf(Mq, sl_m[w][q]);
      float sc[NW], D = 0.f, u = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        sc[w] = fast_exp2(sl_m[w][q] - Mq);
        D = fmaf(sc[w], sl_d[w][q], D);
        u = fmaf(sc[w], sl_u[w][q], u);
      }
      if (r < t1) {
        const float rD = recip_or_zero(D);
#pragma unroll
        for (int e4 = 0; e4 < CPQ; e4 += 4) {
          f32x4 U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(&ul[w][q][cb + e4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) U[e] = fmaf(sc[w], x[e], U[e]);
          }
          const u32x2 qw = *reinterpret_cast<const u32x2*>(B.q + swz(q, (cb + e4) >> 3) + ((cb + e4) & 7));
          const float qv[4] = {bf16_lo_as_f32(qw[0]), bf16_hi_as_f32(qw[0]), bf16_lo_as_f32(qw[1]),
                               bf16_hi_as_f32(qw[1])};
          f32x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (U[e] - qv[e] * u) * rD;
          *reinterpret_cast<f32x4*>(dQ + (rowbase + r) * kD + cb + e4) = o;
        }
        if (cb == 0) *reinterpret_cast<f32x4*>(aux + (rowbase + r) * 4) = f32x4{Mq, D, B.ad[q], 0.f};
      }
    }
    __syncthreads();   // shares and this chunk's buffer free
  }
}

// ---------------------------------------------------------------------------
// k_bw_key_causal: dk and dv, walking the range's chunks from the last.  Wave w
// owns TPW feature tiles of 32 (features [32 TPW w, 32 TPW (w+1))); per tile, R
// (lane = value column) and rho hold the sums over queries after the chunk (the
// ranges after this one, then the later chunks); R.v reads R a feature per lane
// after a pass through LDS.  Per chunk, coef_if = 2^(g_if - M_i) / D_i:
//   dv_j = b_j.R + sum_{i >= j in chunk} (coef_i.b_j) dy_i
//   db_jf = R_f.v_j - rho_f + sum_{i >= j in chunk} coef_if (dy_i.v_j - delta_i)
//   H = b db,  dk_j = W^T H_j - k_j sum_f H_jf
// then R and rho take the chunk's queries.  A wave's share of dv and dk sums
// over its tiles, so the terms that do not depend on the feature (dY V^T and the
// product of the masked chunk matrix with dY) are formed once per wave; the dv
// and dk shares meet in two LDS areas after one barrier.  Staging as for the
// query side.
// ---------------------------------------------------------------------------
template <int M, int TPW>
__global__ __launch_bounds__(M * 2 / TPW) void k_bw_key_causal(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ W, const float* __restrict__ dY, const float* __restrict__ cfin,
    const float* __restrict__ aux, const float* __restrict__ part_R, const float* __restrict__ part_rho,
    float* __restrict__ dK, float* __restrict__ dV, int H, int n, int segs, int span) {
  constexpr int NW = M / (32 * TPW), NT = 64 * NW;
  __shared__ __attribute__((aligned(16))) uint16_t wl[M * kD];
  __shared__ __attribute__((aligned(16))) ChunkBuf buf[2];
  __shared__ __attribute__((aligned(16))) float ulv[NW][32][kD];
  __shared__ __attribute__((aligned(16))) float ulk[NW][32][kD];
  __shared__ float sl_h[NW][32];
  __shared__ __attribute__((aligned(16))) float rl[NW][TPW * 32];
  __shared__ __attribute__((aligned(16))) float cl[M];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, h = lane >> 5, ql = lane & 31;
  const int bh = blockIdx.x / segs, sg = blockIdx.x % segs, hh = bh % H;
  const int t0 = sg * span, t1 = min(n, t0 + span);
  const int fw = 32 * TPW * wave;   // the wave's first feature; tile p starts at fw + 32 p
  const size_t rowbase = static_cast<size_t>(bh) * n;
  const int nch = (t1 - t0 + 31) / 32;
  ChunkRegs<NT, false> pre;
  chunk_load<NT, false>(pre, Q, K, V, dY, nullptr, aux, rowbase, t0 + 32 * (nch - 1), t1, t);
  const uint16_t* Wh = W + static_cast<size_t>(hh) * M * kD;
  for (int c = t; c < M * 8; c += NT)
    *reinterpret_cast<u32x4*>(wl + tile_at(c >> 3, c & 7)) = *reinterpret_cast<const u32x4*>(Wh + 8 * c);
  for (int i = t; i < M; i += NT) cl[i] = cfin[static_cast<size_t>(bh) * M + i];
  float C[TPW];
  // R (D[f][c]: lane = column) and rho per tile: ranges after this one
  f32x16 R[TPW][2];
#pragma unroll
  for (int p = 0; p < TPW; ++p) {
    const int fb = fw + 32 * p, f = fb + ql;
    C[p] = cfin[static_cast<size_t>(bh) * M + f];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int i = 0; i < 16; ++i) R[p][x][i] = 0.f;
    float rho = 0.f;
    for (int s = segs - 1; s > sg; --s) {
      const float* PR = part_R + (static_cast<size_t>(bh) * segs + s) * M * kD;
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i) R[p][x][i] += PR[static_cast<size_t>(fb + drow(i, lane)) * kD + 32 * x + ql];
      rho += part_rho[(static_cast<size_t>(bh) * segs + s) * M + f];
    }
    if (lane < 32) rl[wave][32 * p + lane] = rho;
  }
  chunk_store<NT, false>(pre, buf[0], t);
  if (nch > 1) chunk_load<NT, false>(pre, Q, K, V, dY, nullptr, aux, rowbase, t0 + 32 * (nch - 2), t1, t);
  __syncthreads();

  int it = 0;
  for (int ci = nch - 1; ci >= 0; --ci, ++it) {
    const int c0 = t0 + 32 * ci;
    const ChunkBuf& B = buf[it & 1];
    if (ci > 0) chunk_store<NT, false>(pre, buf[(it + 1) & 1], t);
    const bool ok = c0 + ql < t1;
    // the phases below are kept apart (sched_barrier) so that each one's operands
    // are read from LDS when used and die after it
    // 0. R.v_j (FT: lane = key) per tile: R passes through the wave's dv share rows
    // (free until the dv share below) to be read back a feature per lane
    f32x16 rvd[TPW];
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) ulv[wave][drow(i, lane)][32 * dt + ql] = R[p][dt][i];
      __builtin_amdgcn_wave_barrier();
      rvd[p] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f32x4 ra = *reinterpret_cast<const f32x4*>(&ulv[wave][ql][16 * ks + 8 * h]);
        const f32x4 rb = *reinterpret_cast<const f32x4*>(&ulv[wave][ql][16 * ks + 8 * h + 4]);
        const float x[8] = {ra[0], ra[1], ra[2], ra[3], rb[0], rb[1], rb[2], rb[3]};
        u32x4 rh, rlo;
        split8(x, 0, rh, rlo);
        const u32x4 xv = tile_row8(B.v, ql, ks, h);
        rvd[p] = mfma_bf16(as_bf16x8(rh), as_bf16x8(xv), rvd[p]);
        rvd[p] = mfma_bf16(as_bf16x8(rlo), as_bf16x8(xv), rvd[p]);
      }
      __builtin_amdgcn_wave_barrier();
    }
    __builtin_amdgcn_sched_barrier(0);
    // 1. per tile: coef (FT: lane = query, and TF: lane = feature) and b (FT: lane =
    // key) as bf16 hi / lo; P'^T[i][j] = coef_i . b_j summed over the wave's tiles;
    // rho's new part
    u32x4 bh_[TPW][2], bl_[TPW][2], cth[TPW][2], ctl[TPW][2];
    float rs[TPW];
    f32x16 pp = {};
    {
      const float aqm = B.am[ql], aqr = B.ar[ql];   // the lane's query
      const float kk = B.kk[ql];                     // the lane's key
      float rm[16], rr[16], rd[16];
      rows16(B.am, h, rm);
      rows16(B.ar, h, rr);
      rows16(B.ad, h, rd);
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        const int fb = fw + 32 * p;
        f32x16 pqf = {}, pqt = {}, pkf = {};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4 xq = tile_row8(B.q, ql, ks, h);
          const u32x4 wa = rows_operand(wl, fb, lane, ks);
          pqf = mfma_bf16(as_bf16x8(wa), as_bf16x8(xq), pqf);
          pqt = mfma_bf16(as_bf16x8(xq), as_bf16x8(wa), pqt);
          pkf = mfma_bf16(as_bf16x8(wa), as_bf16x8(tile_row8(B.k, ql, ks, h)), pkf);
        }
        float cff[16], bk[16], cft[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 cc = *reinterpret_cast<const f32x4*>(&cl[fb + 8 * j + 4 * h]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * j + e;
            cff[i] = ok ? fast_exp2(fmaf(kLog2e, pqf[i], cc[e]) - aqm) * aqr : 0.f;
            bk[i] = ok ? fast_exp2(kLog2e * fmaf(-0.5f, kk, pkf[i]) - cc[e]) : 0.f;
          }
        }
        rs[p] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = drow(i, lane);
          const float x = fast_exp2(fmaf(kLog2e, pqt[i], C[p]) - rm[i]) * rr[i];
          cft[i] = c0 + r < t1 ? x : 0.f;   // register = query
          rs[p] = fmaf(cft[i], rd[i], rs[p]);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          split8(cft, kb, cth[p][kb], ctl[p][kb]);
          split8(bk, kb, bh_[p][kb], bl_[p][kb]);
          u32x4 cfh, cfl;
          split8(cff, kb, cfh, cfl);
          pp = mfma_bf16(as_bf16x8(cfh), as_bf16x8(bh_[p][kb]), pp);
          pp = mfma_bf16(as_bf16x8(cfh), as_bf16x8(bl_[p][kb]), pp);
          pp = mfma_bf16(as_bf16x8(cfl), as_bf16x8(bh_[p][kb]), pp);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // 2. dv: carry sum_p b R + chunk P' dY (kept for i >= j), written as the wave's
    // share; b stays on as its bf16 hi + lo
    {
      float pm[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) pm[i] = drow(i, lane) >= ql ? pp[i] : 0.f;
      u32x4 ph[2], pl[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) split8(pm, kb, ph[kb], pl[kb]);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        f32x16 adv = {};
#pragma unroll
        for (int p = 0; p < TPW; ++p)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            u32x4 rh, rlo;
            split8(R[p][dt], kb, rh, rlo);
            adv = mfma_bf16(as_bf16x8(bh_[p][kb]), as_bf16x8(rh), adv);
            adv = mfma_bf16(as_bf16x8(bh_[p][kb]), as_bf16x8(rlo), adv);
            adv = mfma_bf16(as_bf16x8(bl_[p][kb]), as_bf16x8(rh), adv);
          }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 yh = v_operand(B.dh, 16 * kb, dt, lane), ym = v_operand(B.dm, 16 * kb, dt, lane);
          adv = mfma_bf16(as_bf16x8(ph[kb]), as_bf16x8(yh), adv);
          adv = mfma_bf16(as_bf16x8(ph[kb]), as_bf16x8(ym), adv);
          adv = mfma_bf16(as_bf16x8(pl[kb]), as_bf16x8(yh), adv);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) ulv[wave][drow(i, lane)][32 * dt + ql] = adv[i];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // 3. db (FT: lane = key) per tile: R.v - rho + coef^T N with N = dY V^T - delta
    // masked to i >= j (formed once; dy to all its 24 bits); H = b db; the wave's
    // dk share sum_p H W
    f32x16 adk[2] = {};
    float Hs = 0.f;
    {
      f32x16 ndv = {};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 xv = tile_row8(B.v, ql, ks, h);
        ndv = mfma_bf16(as_bf16x8(tile_row8(B.dh, ql, ks, h)), as_bf16x8(xv), ndv);
        ndv = mfma_bf16(as_bf16x8(tile_row8(B.dm, ql, ks, h)), as_bf16x8(xv), ndv);
        ndv = mfma_bf16(as_bf16x8(tile_row8(B.dl, ql, ks, h)), as_bf16x8(xv), ndv);
      }
      float nm[16], rd[16];
      rows16(B.ad, h, rd);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = ndv[i] - rd[i];
        nm[i] = drow(i, lane) >= ql ? x : 0.f;
      }
      u32x4 nh[2], nl[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) split8(nm, kb, nh[kb], nl[kb]);
#pragma unroll
      for (int p = 0; p < TPW; ++p) {
        const int fb = fw + 32 * p;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          rvd[p] = mfma_bf16(as_bf16x8(cth[p][kb]), as_bf16x8(nh[kb]), rvd[p]);
          rvd[p] = mfma_bf16(as_bf16x8(cth[p][kb]), as_bf16x8(nl[kb]), rvd[p]);
          rvd[p] = mfma_bf16(as_bf16x8(ctl[p][kb]), as_bf16x8(nh[kb]), rvd[p]);
        }
        float Hh[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 rr = *reinterpret_cast<const f32x4*>(&rl[wave][32 * p + 8 * j + 4 * h]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * j + e;
            const uint32_t wh = bh_[p][i >> 3][(i & 7) >> 1], wlo = bl_[p][i >> 3][(i & 7) >> 1];
            const float bv = (i & 1) ? bf16_hi_as_f32(wh) + bf16_hi_as_f32(wlo) : bf16_lo_as_f32(wh) + bf16_lo_as_f32(wlo);
            Hh[i] = bv * (rvd[p][i] - rr[e]);
            Hs += Hh[i];
          }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          u32x4 hh_, hl_;
          split8(Hh, kb, hh_, hl_);
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) {
            const u32x4 wb = cols_operand(wl, fb, kb, dt, lane);
            adk[dt] = mfma_bf16(as_bf16x8(hh_), as_bf16x8(wb), adk[dt]);
            adk[dt] = mfma_bf16(as_bf16x8(hl_), as_bf16x8(wb), adk[dt]);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) ulk[wave][drow(i, lane)][32 * dt + ql] = adk[dt][i];
    const float Hw = pair_sum(Hs);
    if (lane < 32) sl_h[wave][lane] = Hw;
    // the reads of the chunk after next, in flight through the combine below
    if (ci > 1) chunk_load<NT, false>(pre, Q, K, V, dY, nullptr, aux, rowbase, c0 - 64, t1, t);
    // 4. the chunk's queries join R and rho (after their use above)
#pragma unroll
    for (int p = 0; p < TPW; ++p) {
      const float rsum = pair_sum(rs[p]);
      if (lane < 32) rl[wave][32 * p + lane] += rsum;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const u32x4 yh = v_operand(B.dh, 16 * kb, dt, lane), ym = v_operand(B.dm, 16 * kb, dt, lane);
          R[p][dt] = mfma_bf16(as_bf16x8(cth[p][kb]), as_bf16x8(yh), R[p][dt]);
          R[p][dt] = mfma_bf16(as_bf16x8(cth[p][kb]), as_bf16x8(ym), R[p][dt]);
          R[p][dt] = mfma_bf16(as_bf16x8(ctl[p][kb]), as_bf16x8(yh), R[p][dt]);
        }
    }
    __syncthreads();   // dv and dk shares visible
    constexpr int CPQ = 32 * kD / NT;
    const int q = t / (kD / CPQ), cb = (t % (kD / CPQ)) * CPQ, r = c0 + q;
    if (r < t1) {
      float hs = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) hs += sl_h[w][q];
#pragma unroll
      for (int e4 = 0; e4 < CPQ; e4 += 4) {
        f32x4 U = {0.f, 0.f, 0.f, 0.f}, Uk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          U += *reinterpret_cast<const f32x4*>(&ulv[w][q][cb + e4]);
          Uk += *reinterpret_cast<const f32x4*>(&ulk[w][q][cb + e4]);
        }
        *reinterpret_cast<f32x4*>(dV + (rowbase + r) * kD + cb + e4) = U;
        const u32x2 kw = *reinterpret_cast<const u32x2*>(B.k + swz(q, (cb + e4) >> 3) + ((cb + e4) & 7));
        const float kv[4] = {bf16_lo_as_f32(kw[0]), bf16_hi_as_f32(kw[0]), bf16_lo_as_f32(kw[1]),
                             bf16_hi_as_f32(kw[1])};
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = Uk[e] - kv[e] * hs;
        *reinterpret_cast<f32x4*>(dK + (rowbase + r) * kD + cb + e4) = o;
      }
    }
    __syncthreads();   // shares and this chunk's buffer free
  }
}

template <int M>
hipError_t launch_causal_m(const BwPlan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const uint16_t* W, const float* y, const float* dy, float* dq, float* dk, float* dv,
                           void* ws, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  float* cpart = reinterpret_cast<float*>(base + p.off_cpart);
  float* pS = reinterpret_cast<float*>(base + p.off_part);
  float* pz = reinterpret_cast<float*>(base + p.off_pvec);
  float* pR = reinterpret_cast<float*>(base + p.off_part2);
  float* prho = reinterpret_cast<float*>(base + p.off_pvec2);
  float* cfin = reinterpret_cast<float*>(base + p.off_cfin);
  float* aux = reinterpret_cast<float*>(base + p.off_aux);
  const int BH = p.B * p.H;
  const dim3 gs(BH * p.splits), bs(2 * M);
  auto kst = k_bw_keys<M>;
  FAVOR_LAUNCH("k_bw_kstate", kst, gs, bs, 0, s, k, v, W, cpart, pS, pz, p.H, p.n, p.splits, p.span);
  FAVOR_LAUNCH("k_bw_cmax", k_bw_cmax, dim3((BH * p.m + 255) / 256), dim3(256), 0, s, cpart, cfin, BH * p.m, p.m,
               p.splits);
  // a tile per wave: two tiles per wave (4 waves at m = 256) walked slower (453 against 400 us)
  auto kq = k_bw_query_causal<M, 1>;
  FAVOR_LAUNCH("k_bw_query_causal", kq, gs, bs, 0, s, q, k, v, W, y, dy, cfin, cpart, pS, pz, dq, aux, p.H, p.n,
               p.splits, p.span);
  auto kr = k_bw_rstate<M>;
  FAVOR_LAUNCH("k_bw_rstate", kr, gs, bs, 0, s, q, dy, W, cfin, aux, pR, prho, p.H, p.n, p.splits, p.span);
  // m = 256: 4 waves of two feature tiles (the dv and dk share areas fit in LDS
  // beside the staged chunks); else a tile per wave
  constexpr int TPW = M == 256 ? 2 : 1;
  auto kc = k_bw_key_causal<M, TPW>;
  FAVOR_LAUNCH("k_bw_key_causal", kc, gs, dim3(2 * M / TPW), 0, s, q, k, v, W, dy, cfin, aux, pR, prho, dk, dv, p.H, p.n,
               p.splits, p.span);
  return hipGetLastError();
}

template <int M>
hipError_t launch_m(const BwPlan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* W,
                    const float* y, const float* dy, float* dq, float* dk, float* dv, void* ws, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  float* cpart = reinterpret_cast<float*>(base + p.off_cpart);
  float* pS = reinterpret_cast<float*>(base + p.off_part);
  float* pz = reinterpret_cast<float*>(base + p.off_pvec);
  uint16_t* stl = reinterpret_cast<uint16_t*>(base + p.off_stiles);
  uint16_t* rtl = reinterpret_cast<uint16_t*>(base + p.off_rtiles);
  float* zg = reinterpret_cast<float*>(base + p.off_z);
  float* rho = reinterpret_cast<float*>(base + p.off_rho);
  float* cfin = reinterpret_cast<float*>(base + p.off_cfin);
  float* aux = reinterpret_cast<float*>(base + p.off_aux);
  const int BH = p.B * p.H;
  const dim3 gs(BH * p.splits), bs(2 * M);
  auto kst = k_bw_keys<M>;
  FAVOR_LAUNCH("k_bw_kstate", kst, gs, bs, 0, s, k, v, W, cpart, pS, pz, p.H, p.n, p.splits, p.span);
  FAVOR_LAUNCH("k_bw_merge", k_bw_merge, dim3(BH * (M / 4)), dim3(256), 0, s, pS, pz, stl, zg, cpart, cfin, BH, M,
               p.splits);
  const int ntiles = (p.n + 31) / 32;
  int qblocks = (256 + BH - 1) / BH;
  const int per = (ntiles + 7) / 8;
  if (qblocks > per) qblocks = per;
  if (qblocks < 1) qblocks = 1;
  auto kq = k_bw_query<M>;
  FAVOR_LAUNCH("k_bw_query", kq, dim3(BH * qblocks), dim3(512), 0, s, q, y, dy, W, stl, zg, cfin, dq, aux, BH, p.H,
               p.n, qblocks);
  auto kr = k_bw_rstate<M>;
  FAVOR_LAUNCH("k_bw_rstate", kr, gs, bs, 0, s, q, dy, W, cfin, aux, pS, pz, p.H, p.n, p.splits, p.span);
  FAVOR_LAUNCH("k_bw_merge", k_bw_merge, dim3(BH * (M / 4)), dim3(256), 0, s, pS, pz, rtl, rho,
               static_cast<const float*>(nullptr), static_cast<float*>(nullptr), BH, M, p.splits);
  auto kk_ = k_bw_key<M>;
  FAVOR_LAUNCH("k_bw_key", kk_, dim3(BH * qblocks), dim3(512), 0, s, k, v, W, rtl, rho, cfin, dk, dv, BH, p.H, p.n,
               qblocks);
  return hipGetLastError();
}

}  // namespace

BwPlan bw_plan(int B, int H, int n, int m, int causal) {
  BwPlan p{};
  p.B = B;
  p.H = H;
  p.n = n;
  p.m = m;
  p.causal = causal;
  const int BH = B * H;
  // about two workgroups per CU for the key-range kernels of the non-causal pass
  // (they fit twice); one segment walk per CU for the causal pass
  int s = ((causal ? 256 : 512) + BH - 1) / BH;
  const int tiles = (n + 63) / 64;
  if (s > tiles) s = tiles;
  if (s < 1) s = 1;
  p.span = ((n + s - 1) / s + 63) / 64 * 64;
  p.splits = (n + p.span - 1) / p.span;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = bf16k::align_up(off + bytes, 256);
    return o;
  };
  p.off_cpart = take(static_cast<size_t>(BH) * p.splits * m * 4);
  p.off_part = take(static_cast<size_t>(BH) * p.splits * m * kD * 4);
  p.off_pvec = take(static_cast<size_t>(BH) * p.splits * m * 4);
  p.off_part2 = causal ? take(static_cast<size_t>(BH) * p.splits * m * kD * 4) : 0;
  p.off_pvec2 = causal ? take(static_cast<size_t>(BH) * p.splits * m * 4) : 0;
  // the merged states (non-causal only: the causal kernels read the partials)
  p.off_stiles = causal ? 0 : take(static_cast<size_t>(BH) * m * kD * 2 * 2);
  p.off_rtiles = causal ? 0 : take(static_cast<size_t>(BH) * m * kD * 2 * 2);
  p.off_z = causal ? 0 : take(static_cast<size_t>(BH) * m * 4);
  p.off_rho = causal ? 0 : take(static_cast<size_t>(BH) * m * 4);
  p.off_cfin = take(static_cast<size_t>(BH) * m * 4);
  p.off_aux = take(static_cast<size_t>(BH) * n * 16);
  p.off_end = off;
  return p;
}

hipError_t launch_backward_bf16(const BwPlan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const uint16_t* W, const float* y, const float* dy, float* dq, float* dk, float* dv,
                                void* ws, hipStream_t s) {
  if (p.causal) {
    switch (p.m) {
      case 64: return launch_causal_m<64>(p, q, k, v, W, y, dy, dq, dk, dv, ws, s);
      case 128: return launch_causal_m<128>(p, q, k, v, W, y, dy, dq, dk, dv, ws, s);
      case 256: return launch_causal_m<256>(p, q, k, v, W, y, dy, dq, dk, dv, ws, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (p.m) {
    case 64: return launch_m<64>(p, q, k, v, W, y, dy, dq, dk, dv, ws, s);
    case 128: return launch_m<128>(p, q, k, v, W, y, dy, dq, dk, dv, ws, s);
    case 256: return launch_m<256>(p, q, k, v, W, y, dy, dq, dk, dv, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bw
}  // namespace favor
