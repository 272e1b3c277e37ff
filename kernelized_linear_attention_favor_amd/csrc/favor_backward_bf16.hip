// Backward pass of FAVOR+ attention (dQ, dK, dV for an upstream gradient dY),
// derived from the forward (Performer notes, Kernel Attention View,
// Normalization and FAVOR+) by the chain rule: the pages mention training and
// gradients but print no formulas.
//
// Exact rewrite used throughout (log2 units): with e_jf = log2e (w_f.k_j -
// |k_j|^2/2), C_f = max_j e_jf over the head's keys and g_if = log2e w_f.q_i +
// C_f, M_i = max_f g_if,
//   b_jf = 2^(e_jf - C_f) in (0, 1],   a_if = 2^(g_if - M_i) in (0, 1],
// phi(q_i).phi(k_j) = lambda_i a_i.b_j for a per-query constant lambda_i, which
// cancels in y and in every gradient below.  With S = sum_j b_j v_j^T, z =
// sum_j b_j, D_i = a_i.z, delta_i = dy_i.y_i (y the forward output):
//   G_if = a_if (S_f.dy_i - z_f delta_i) / D_i,  dq_i = W^T G_i - q_i sum_f G_if
//   R = sum_i (a_i / D_i) dy_i^T,  rho = sum_i (a_i / D_i) delta_i,
//   dv_j = R^T b_j,  H_jf = b_jf (R_f.v_j - rho_f),  dk_j = W^T H_j - k_j sum_f H_jf
// (d phi_f(x) / dx = phi_f(x) (w_f - x)).  The key shift C_f is one constant per
// feature for the whole head, so these are plain bounded sums in fp32; a
// feature's key exponents may spread up to ~2^126 below its largest.
//
// Kernels (non-causal): k_bw_keys<MAX> (C_f partials), k_bw_keys<STATE> (S, z
// partials), k_bw_merge (sum, written as bf16 hi + lo row-major tiles),
// k_bw_query (dq; M_i, D_i, delta_i per query), k_bw_rstate (R, rho partials),
// k_bw_merge, k_bw_key (dk, dv).  bf16 MFMA with fp32 accumulation; fp32
// operands enter as bf16 hi + lo pairs, the bf16 inputs exactly.
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
// k_bw_keys<M, PASS>: one key range of one (b, h); M/32 waves, wave w owns
// features [32w, 32w+32).  Per 64 keys: K (and V) tiles and |k|^2 in LDS; per
// 32 keys each wave projects to a TF tile (lane = feature, register = key).
//   PASS 0: the largest e_jf of the range per feature -> cpart.
//   PASS 1: b_jf = 2^(e_jf - C_f) (C_f = max over ranges of cpart); z += b,
//           S += b^T V with b as bf16 hi + lo -> part_S, part_z.
// ---------------------------------------------------------------------------
template <int M, int PASS>
__global__ __launch_bounds__(2 * M) void k_bw_keys(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                   const uint16_t* __restrict__ W, float* __restrict__ cpart,
                                                   float* __restrict__ part_S, float* __restrict__ part_z, int H,
                                                   int n, int splits, int span) {
  constexpr int NT = 2 * M;
  constexpr int NMAT = PASS == 0 ? 1 : 2;          // K only, or K and V
  constexpr int CPT = 512 * NMAT / NT;
  __shared__ __attribute__((aligned(16))) uint16_t kt[64 * 64];
  __shared__ __attribute__((aligned(16))) uint16_t vt[PASS == 0 ? 8 : 64 * 64];
  __shared__ float kk[64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, h = lane >> 5;
  const int bh = blockIdx.x / splits, sp = blockIdx.x % splits, hh = bh % H;
  const int j0 = sp * span, j1 = min(n, j0 + span);
  const int fb = 32 * wave, f = fb + (lane & 31);
  u32x4 wop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    wop[ks] = *reinterpret_cast<const u32x4*>(W + (static_cast<size_t>(hh) * M + f) * kD + 16 * ks + 8 * h);
  float C = 0.f;
  if constexpr (PASS == 1) {
    C = kNegInf;
    for (int s = 0; s < splits; ++s) C = fmaxf(C, cpart[(static_cast<size_t>(bh) * splits + s) * M + f]);
  }

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
  float zp = 0.f, mx = kNegInf;
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
      float s = 0.f;
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(kt + swz(t, ch));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = bf16_lo_as_f32(x[e]), hi = bf16_hi_as_f32(x[e]);
          s = fmaf(lo, lo, s);
          s = fmaf(hi, hi, s);
        }
      }
      kk[t] = s;
    }
    __syncthreads();
    if (tok0 + 64 < j1) fetch(tok0 + 64);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x16 pr = {};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 xk = *reinterpret_cast<const u32x4*>(kt + swz(32 * st + (lane & 31), 2 * ks + h));
        pr = mfma_bf16(as_bf16x8(xk), as_bf16x8(wop[ks]), pr);
      }
      float b[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 32 * st + drow(i, lane);
        const float e = kLog2e * fmaf(-0.5f, kk[r], pr[i]);
        const bool ok = tok0 + r < j1;
        if constexpr (PASS == 0) {
          mx = ok ? fmaxf(mx, e) : mx;
        } else {
          b[i] = ok ? fast_exp2(e - C) : 0.f;
          zp += b[i];
        }
      }
      if constexpr (PASS == 1) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          u32x4 ahi, alo;
          split8(b, kb, ahi, alo);
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) {
            const u32x4 vb = v_operand(vt, 32 * st + 16 * kb, dt, lane);
            acc[dt] = mfma_bf16(as_bf16x8(ahi), as_bf16x8(vb), acc[dt]);
            acc[dt] = mfma_bf16(as_bf16x8(alo), as_bf16x8(vb), acc[dt]);
          }
        }
      }
    }
  }
  const size_t slot = static_cast<size_t>(bh) * splits + sp;
  if constexpr (PASS == 0) {
    mx = pair_max(mx);
    if (lane < 32) cpart[slot * M + f] = mx;
  } else {
    float* PS = part_S + slot * M * kD;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) PS[(fb + drow(i, lane)) * kD + 32 * dt + (lane & 31)] = acc[dt][i];
    zp = pair_sum(zp);
    if (lane < 32) part_z[slot * M + f] = zp;
  }
}

// ---------------------------------------------------------------------------
// k_bw_merge: the ranges of one (b, h) summed in index order; the m x 64 sum as
// bf16 hi + lo tiled arrays, the m-vector in fp32, and (if cpart) the largest
// key exponent per feature over the ranges.  One workgroup per (b, h, 4 rows).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bw_merge(const float* __restrict__ part, const float* __restrict__ pvec,
                                                  uint16_t* __restrict__ tiles, float* __restrict__ vec,
                                                  const float* __restrict__ cpart, float* __restrict__ cfin, int BH,
                                                  int M, int splits) {
  const int q4 = M / 4;
  const int bh = blockIdx.x / q4, r = (blockIdx.x % q4) * 4 + (threadIdx.x >> 6), c = threadIdx.x & 63;
  float a = 0.f;
  const float* P = part + (static_cast<size_t>(bh) * splits * M + r) * kD + c;
#pragma unroll 8
  for (int sp = 0; sp < splits; ++sp) a += P[static_cast<size_t>(sp) * M * kD];
  const uint32_t pk = pack_bf16(a, 0.f);
  const uint16_t hi = static_cast<uint16_t>(pk & 0xffffu);
  const uint16_t lo = static_cast<uint16_t>(pack_bf16(a - bf16_lo_as_f32(pk), 0.f) & 0xffffu);
  const size_t base = static_cast<size_t>(bh) * M * kD + tile_at(r, c >> 3) + (c & 7);
  tiles[base] = hi;
  tiles[static_cast<size_t>(BH) * M * kD + base] = lo;
  if (c == 0) {
    float s = 0.f;
    for (int sp = 0; sp < splits; ++sp) s += pvec[(static_cast<size_t>(bh) * splits + sp) * M + r];
    vec[static_cast<size_t>(bh) * M + r] = s;
    if (cpart) {
      float m = kNegInf;
      for (int sp = 0; sp < splits; ++sp) m = fmaxf(m, cpart[(static_cast<size_t>(bh) * splits + sp) * M + r]);
      cfin[static_cast<size_t>(bh) * M + r] = m;
    }
  }
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
// each wave takes 32-query tiles of its (b, h) and walks the feature tiles
// twice: once for the row maximum M_i, once for a (FT: lane = query), D_i,
// T = S dy (three MFMAs per k-step against S hi / lo), G and the product G W.
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
    // pass 1: the row maximum of g
    float mx = kNegInf;
    for (int ft = 0; ft < M / 32; ++ft) {
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
    const float Mi = pair_max(mx);
    // pass 2
    f32x16 acc[2] = {};
    float Dp = 0.f, Gs = 0.f;
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
          const float a = fast_exp2(fmaf(kLog2e, pr[4 * j + e], cc[e]) - Mi);
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
    const float Di = pair_sum(Dp), Gsum = pair_sum(Gs);
    if (lane < 32) {
      rdl[wave][lane] = 1.f / Di;
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
// queries: Q, dY (as bf16 hi and lo tiles) and (M_i, D_i, delta_i) in LDS; per 32
// queries a TF projection gives a_if / D_i, which enters as bf16 hi + lo.
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

  f32x16 acc[2] = {};
  float rp = 0.f;
  for (int tok0 = j0; tok0 < j1; tok0 += 64) {
    __syncthreads();
    for (int c = t; c < 512; c += NT) {   // Q: 64 rows x 8 chunks
      const int r = c >> 3, ch = c & 7;
      *reinterpret_cast<u32x4*>(qt + swz(r, ch)) =
          tok0 + r < j1 ? *reinterpret_cast<const u32x4*>(Q + (rowbase + tok0 + r) * kD + 8 * ch)
                        : u32x4{0u, 0u, 0u, 0u};
    }
    for (int c = t; c < 512; c += NT) {   // dY: 64 rows x 8 groups of 8 floats -> hi, lo chunks
      const int r = c >> 3, ch = c & 7;
      u32x4 hi = {0u, 0u, 0u, 0u}, lo = {0u, 0u, 0u, 0u};
      if (tok0 + r < j1) split_row8(dY + (rowbase + tok0 + r) * kD + 8 * ch, hi, lo);
      *reinterpret_cast<u32x4*>(dh + swz(r, ch)) = hi;
      *reinterpret_cast<u32x4*>(dlo + swz(r, ch)) = lo;
    }
    for (int r = t; r < 64; r += NT)
      ax[r] = tok0 + r < j1 ? *reinterpret_cast<const f32x4*>(aux + (rowbase + tok0 + r) * 4) : f32x4{0.f, 1.f, 0.f, 0.f};
    __syncthreads();
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
        const f32x4 a = ax[r];   // M_i, D_i, delta_i
        cf[i] = tok0 + r < j1 ? fast_exp2(fmaf(kLog2e, pr[i], C) - a[0]) / a[1] : 0.f;
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
  auto kmax = k_bw_keys<M, 0>;
  FAVOR_LAUNCH("k_bw_kmax", kmax, gs, bs, 0, s, k, v, W, cpart, pS, pz, p.H, p.n, p.splits, p.span);
  auto kst = k_bw_keys<M, 1>;
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
  int s = (256 + BH - 1) / BH;
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
  p.off_stiles = take(static_cast<size_t>(BH) * m * kD * 2 * 2);
  p.off_rtiles = take(static_cast<size_t>(BH) * m * kD * 2 * 2);
  p.off_z = take(static_cast<size_t>(BH) * m * 4);
  p.off_rho = take(static_cast<size_t>(BH) * m * 4);
  p.off_cfin = take(static_cast<size_t>(BH) * m * 4);
  p.off_aux = take(static_cast<size_t>(BH) * n * 16);
  p.off_end = off;
  return p;
}

hipError_t launch_backward_bf16(const BwPlan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const uint16_t* W, const float* y, const float* dy, float* dq, float* dk, float* dv,
                                void* ws, hipStream_t s) {
  if (p.causal) return hipErrorInvalidValue;
  switch (p.m) {
    case 64: return launch_m<64>(p, q, k, v, W, y, dy, dq, dk, dv, ws, s);
    case 128: return launch_m<128>(p, q, k, v, W, y, dy, dq, dk, dv, ws, s);
    case 256: return launch_m<256>(p, q, k, v, W, y, dy, dq, dk, dv, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bw
}  // namespace favor
