// Linear attention with deterministic feature maps on gfx950: the same state,
// output and causal structure as FAVOR+ (Performer notes, Kernel Attention View
// and Normalization; Performer for vision, How It Works, Step 2) with a cheaper
// phi (Performer for vision, What Is Performer? and Kernel Choices: ReLU
// features of the random projections; the linear-attention quiz page's
// comparison table: the Linear Transformer's elu(x)+1):
//   relu:  phi_f(x) = max(w_f.x, 0)             (the 1/sqrt(m) cancels in y)
//   elu1:  phi_f(x) = elu(x_f) + 1, f < d = m   (the projection is the identity)
// Bounded features need no stabilising shift: the state is a plain fp32 sum and
// every term is linear in phi, so partial sums over keys, features or workgroups
// simply add.  Inputs bf16, output fp32.
//
// Operand precision: phi is split into bf16 hi + lo (about 16 bits) wherever it
// enters an MFMA, and so are S and the causal chunk matrix P; V is bf16 exactly.
// The denominators use the unrounded fp32 features.
//
// Layouts of a 32 x 32 MFMA tile used below (d = 64, 32 features, 32 tokens):
//   TF  D[token][feature] = X W^T: lane = feature, register i = token drow(i)
//   FT  D[feature][token] = W X^T: lane = token,   register i = feature drow(i)
// with drow(i) = 8 (i / 4) + 4 (lane / 32) + i % 4.  Registers 8kb .. 8kb+7 of
// either layout form one 16-wide k-block of an MFMA operand in that order, so a
// TF tile is the A operand of S += Phi^T V (rows = features, k = tokens), an FT
// tile is the A operand of num = phi(Q) S (rows = queries) or the B operand of
// P^T = phi(K) phi(Q)^T (columns = queries), and the matching B operands (V rows
// by the LDS transpose read, S from its own accumulator registers) follow the
// same order.
#include <math.h>

#include "favor_bf16_common.h"
#include "favor_internal.h"
#include "favor_mfma.h"

namespace favor {
namespace lin {
namespace {

using bf16k::kD;
using bf16k::swz;
using bf16k::v_operand;

constexpr int kRelu = 1, kElu1 = 2;

__device__ __forceinline__ int drow(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

template <int KIND>
__device__ __forceinline__ float phi_of(float p) {
  if constexpr (KIND == kRelu) {
    return fmaxf(p, 0.f);
  } else {
    return p > 0.f ? p + 1.f : fast_exp2(kLog2e * p);   // elu(p) + 1
  }
}

// Projection operand of a 32-feature tile starting at feature fb, k-step ks
// (dims 16ks .. 16ks+15): lane l holds row fb + l % 32, dims 16ks + 8(l/32) ..
// +7.  ReLU: the head's W row (bf16).  elu1: the identity (exact products).
template <int KIND>
__device__ __forceinline__ u32x4 w_operand(const uint16_t* Wh, int fb, int lane, int ks) {
  if constexpr (KIND == kRelu) {
    return *reinterpret_cast<const u32x4*>(Wh + static_cast<size_t>(fb + (lane & 31)) * kD + 16 * ks +
                                           8 * (lane >> 5));
  } else {
    const int s = fb + (lane & 31) - (16 * ks + 8 * (lane >> 5));   // slot of the 1, if 0 <= s < 8
    const uint32_t one = bf16k::kBf16One << (16 * (s & 1));
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = (s >= 0 && s < 8 && (s >> 1) == j) ? one : 0u;
    return r;
  }
}

// 8 fp32 values (one k-block) -> bf16 hi and lo operands.
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

// ---------------------------------------------------------------------------
// k_lin_state: partial key/value state of one key range (split or segment) of
// one (b, h).  M/32 waves; wave w owns features [32w, 32w+32).  Per 64 keys the
// K and V tiles are staged in LDS (the next tile's loads in flight meanwhile);
// per 32 keys each wave projects to a TF tile, applies phi, adds it to z and
// accumulates S_w += Phi^T V with phi as bf16 hi + lo.
// part_S: [BH][splits][M][64] fp32, part_z: [BH][splits][M].
// ---------------------------------------------------------------------------
template <int KIND, int M>
__global__ __launch_bounds__(2 * M) void k_lin_state(const uint16_t* __restrict__ K,
                                                     const uint16_t* __restrict__ V,
                                                     const uint16_t* __restrict__ W,
                                                     float* __restrict__ part_S, float* __restrict__ part_z,
                                                     int H, int n, int splits, int span) {
  constexpr int NT = 2 * M;          // M/32 waves
  constexpr int CPT = 1024 / NT;     // 16-byte chunks of the K and V tiles per thread
  __shared__ __attribute__((aligned(16))) uint16_t kt[64 * 64];
  __shared__ __attribute__((aligned(16))) uint16_t vt[64 * 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, h = lane >> 5;
  const int bh = blockIdx.x / splits, sp = blockIdx.x % splits, hh = bh % H;
  const int j0 = sp * span, j1 = min(n, j0 + span);
  const int fb = 32 * wave;
  const uint16_t* Wh = KIND == kRelu ? W + static_cast<size_t>(hh) * M * kD : nullptr;
  u32x4 wop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) wop[ks] = w_operand<KIND>(Wh, fb, lane, ks);

  const size_t rowbase = static_cast<size_t>(bh) * n;
  u32x4 pre[CPT];
  auto fetch = [&](int tok0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = t + NT * i, mat = c >> 9, r = (c >> 3) & 63, ch = c & 7;
      const int tok = tok0 + r;
      pre[i] = tok < j1 ? *reinterpret_cast<const u32x4*>((mat ? V : K) + (rowbase + tok) * kD + 8 * ch)
                        : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = t + NT * i, mat = c >> 9, r = (c >> 3) & 63, ch = c & 7;
      *reinterpret_cast<u32x4*>((mat ? vt : kt) + swz(r, ch)) = pre[i];
    }
  };

  f32x16 acc[2] = {};
  float zp = 0.f;
  if (j0 < j1) fetch(j0);
  for (int tok0 = j0; tok0 < j1; tok0 += 64) {
    __syncthreads();   // the previous tile's reads are done
    stage();
    __syncthreads();
    if (tok0 + 64 < j1) fetch(tok0 + 64);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int row = 32 * st + (lane & 31);
      f32x16 pr = {};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 xk = *reinterpret_cast<const u32x4*>(kt + swz(row, 2 * ks + h));
        pr = mfma_bf16(as_bf16x8(xk), as_bf16x8(wop[ks]), pr);
      }
      float ph[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        ph[i] = tok0 + 32 * st + drow(i, lane) < j1 ? phi_of<KIND>(pr[i]) : 0.f;
        zp += ph[i];
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        u32x4 ahi, alo;
        split8(ph, kb, ahi, alo);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const u32x4 vb = v_operand(vt, 32 * st + 16 * kb, dt, lane);
          acc[dt] = mfma_bf16(as_bf16x8(ahi), as_bf16x8(vb), acc[dt]);
          acc[dt] = mfma_bf16(as_bf16x8(alo), as_bf16x8(vb), acc[dt]);
        }
      }
    }
  }
  float* PS = part_S + (static_cast<size_t>(bh) * splits + sp) * M * kD;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) PS[(fb + drow(i, lane)) * kD + 32 * dt + (lane & 31)] = acc[dt][i];
  zp = pair_sum(zp);   // lanes l and l ^ 32 hold the same feature's two token halves
  if (lane < 32) part_z[(static_cast<size_t>(bh) * splits + sp) * M + fb + lane] = zp;
}

// ---------------------------------------------------------------------------
// k_lin_merge: the splits of one (b, h) summed in index order, written as the
// B operand of num = phi(Q) S: for feature k-block kb, value-column tile dt and
// lane l, 8 bf16 = S[f(kb, l, s)][32dt + l % 32], s = 0..7, in the FT register
// order f = 16kb + 8(s/4) + 4(l/32) + s%4; once as hi and once as lo.  z in
// fp32.  sop: [2 (hi, lo)][BH][M/16][2][64] u32x4.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void k_lin_merge(const float* __restrict__ part_S,
                                                   const float* __restrict__ part_z, u32x4* __restrict__ sop,
                                                   float* __restrict__ zout, int BH, int M, int splits) {
  const int kbs = M / 16;
  const int bh = blockIdx.x / kbs, kb = blockIdx.x % kbs;
  const int t = threadIdx.x, dt = t >> 6, lane = t & 63, h = lane >> 5;
  const int c = 32 * dt + (lane & 31);
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float* P0 = part_S + static_cast<size_t>(bh) * splits * M * kD + c;
  // splits in index order; the loads of 8 splits are issued before their adds
#pragma unroll 8
  for (int sp = 0; sp < splits; ++sp) {
    const float* P = P0 + static_cast<size_t>(sp) * M * kD;
#pragma unroll
    for (int s = 0; s < 8; ++s) v[s] += P[(16 * kb + 8 * (s >> 2) + 4 * h + (s & 3)) * kD];
  }
  u32x4 hi, lo;
  split8(v, 0, hi, lo);
  const size_t o = ((static_cast<size_t>(bh) * kbs + kb) * 2 + dt) * 64 + lane;
  sop[o] = hi;
  sop[static_cast<size_t>(BH) * kbs * 2 * 64 + o] = lo;
  if (t < 16) {
    float z = 0.f;
    for (int sp = 0; sp < splits; ++sp) z += part_z[(static_cast<size_t>(bh) * splits + sp) * M + 16 * kb + t];
    zout[static_cast<size_t>(bh) * M + 16 * kb + t] = z;
  }
}

// ---------------------------------------------------------------------------
// k_lin_output: y = phi(Q) S / phi(Q) z.  8 waves; each wave takes 32-query
// tiles of its (b, h); per 32-feature tile it projects W Q^T (FT: lane =
// query), applies phi, accumulates the denominator against z on the VALU and
// the numerator with three MFMAs (hi.hi, hi.lo, lo.hi) against S from LDS.
// ---------------------------------------------------------------------------
template <int KIND, int M>
__global__ __launch_bounds__(512) void k_lin_output(const uint16_t* __restrict__ Q,
                                                    const uint16_t* __restrict__ W,
                                                    const u32x4* __restrict__ sop, const float* __restrict__ zg,
                                                    float* __restrict__ out, int BH, int H, int n, int qblocks) {
  constexpr int NWV = 8, KBS = M / 16;
  __shared__ __attribute__((aligned(16))) u32x4 shi[KBS][2][64];
  __shared__ __attribute__((aligned(16))) u32x4 slo[KBS][2][64];
  __shared__ __attribute__((aligned(16))) uint16_t wl[KIND == kRelu ? M * kD : 8];
  __shared__ __attribute__((aligned(16))) float zl[M];
  __shared__ float dl[NWV][32];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, h = lane >> 5;
  const int bh = blockIdx.x / qblocks, qb = blockIdx.x % qblocks, hh = bh % H;

  {
    const u32x4* sh = sop + static_cast<size_t>(bh) * KBS * 2 * 64;
    const u32x4* sl = sh + static_cast<size_t>(BH) * KBS * 2 * 64;
    for (int i = t; i < KBS * 2 * 64; i += 512) {
      (&shi[0][0][0])[i] = sh[i];
      (&slo[0][0][0])[i] = sl[i];
    }
    for (int i = t; i < M; i += 512) zl[i] = zg[static_cast<size_t>(bh) * M + i];
    if constexpr (KIND == kRelu) {
      const uint16_t* Wh = W + static_cast<size_t>(hh) * M * kD;
      for (int c = t; c < M * 8; c += 512)
        *reinterpret_cast<u32x4*>(wl + swz(c >> 3, c & 7)) = *reinterpret_cast<const u32x4*>(Wh + 8 * c);
    }
  }
  __syncthreads();

  const int ntiles = (n + 31) / 32;
  const size_t rowbase = static_cast<size_t>(bh) * n;
  for (int tile = qb * NWV + wave; tile < ntiles; tile += qblocks * NWV) {
    const int row = 32 * tile + (lane & 31);
    u32x4 xq[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      xq[ks] = row < n ? *reinterpret_cast<const u32x4*>(Q + (rowbase + row) * kD + 16 * ks + 8 * h)
                       : u32x4{0u, 0u, 0u, 0u};
    f32x16 num[2] = {};
    float den = 0.f;
    for (int ft = 0; ft < M / 32; ++ft) {
      f32x16 pr = {};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        u32x4 wo;
        if constexpr (KIND == kRelu)
          wo = *reinterpret_cast<const u32x4*>(wl + swz(32 * ft + (lane & 31), 2 * ks + h));
        else
          wo = w_operand<KIND>(nullptr, 32 * ft, lane, ks);
        pr = mfma_bf16(as_bf16x8(wo), as_bf16x8(xq[ks]), pr);
      }
      float ph[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // registers 4j .. 4j+3 hold features 8j + 4h .. +3: one 16-byte read of z
        const f32x4 zz = *reinterpret_cast<const f32x4*>(&zl[32 * ft + 8 * j + 4 * h]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ph[4 * j + e] = phi_of<KIND>(pr[4 * j + e]);
          den = fmaf(ph[4 * j + e], zz[e], den);
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        u32x4 ahi, alo;
        split8(ph, kb, ahi, alo);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const u32x4 bhi = shi[2 * ft + kb][dt][lane], blo = slo[2 * ft + kb][dt][lane];
          num[dt] = mfma_bf16(as_bf16x8(ahi), as_bf16x8(bhi), num[dt]);
          num[dt] = mfma_bf16(as_bf16x8(ahi), as_bf16x8(blo), num[dt]);
          num[dt] = mfma_bf16(as_bf16x8(alo), as_bf16x8(bhi), num[dt]);
        }
      }
    }
    den = pair_sum(den);   // the two lane halves hold complementary features of one query
    if (lane < 32) dl[wave][lane] = den > 0.f ? 1.f / den : 0.f;   // y = 0 for a query without weight
    __builtin_amdgcn_wave_barrier();
    float* orow = out + (rowbase + 32 * tile + 4 * h) * kD + (lane & 31);
    const bool full = 32 * tile + 32 <= n;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = drow(i, lane);
      const float rq = dl[wave][q];
      if (full || 32 * tile + q < n) {
        const int o = (8 * (i >> 2) + (i & 3)) * kD;
        orow[o] = num[0][i] * rq;
        orow[o + 32] = num[1][i] * rq;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------------------
// k_lin_causal: one segment of one (b, h), in chunks of 32 tokens.  M/32
// waves; wave w owns features [32w, 32w+32) and their running state
// (S_w: two accumulator tiles, rows = features, lane = value column; z_w).
// It starts from the sum of the earlier segments' states (index order).  Per
// chunk each wave forms its features' share of
//   num = phi(Q) S + tril(P) V,   den = phi(Q) z + tril(P) 1,   P = phi(Q) phi(K)^T,
// then adds the chunk's keys to S_w and z_w; the shares are summed in wave
// order in LDS and y = num / den is written.  Two barriers per chunk.
// ---------------------------------------------------------------------------
template <int KIND, int M>
__global__ __launch_bounds__(2 * M) void k_lin_causal(const uint16_t* __restrict__ Q,
                                                      const uint16_t* __restrict__ K,
                                                      const uint16_t* __restrict__ V,
                                                      const uint16_t* __restrict__ W,
                                                      const float* __restrict__ part_S,
                                                      const float* __restrict__ part_z, float* __restrict__ out,
                                                      int H, int n, int segs, int span) {
  constexpr int NW = M / 32, NT = 2 * M;
  constexpr int VPT = (256 + NT - 1) / NT;   // 16-byte chunks of the 32 x 64 V tile per thread
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][32 * 64];
  constexpr int PLD = kD + 4;   // padded partial rows: the two lane halves' rows (4 apart) use different banks
  __shared__ __attribute__((aligned(16))) float part[NW][32][PLD];
  __shared__ float dpart[NW][32];
  __shared__ __attribute__((aligned(16))) float zl[NW][32];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, h = lane >> 5;
  const int bh = blockIdx.x / segs, sg = blockIdx.x % segs, hh = bh % H;
  const int t0 = sg * span, t1 = min(n, t0 + span);
  const int fb = 32 * wave;
  const uint16_t* Wh = KIND == kRelu ? W + static_cast<size_t>(hh) * M * kD : nullptr;
  u32x4 wop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) wop[ks] = w_operand<KIND>(Wh, fb, lane, ks);

  // the state of the keys before this segment
  f32x16 S[2];
  {
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) S[dt][i] = 0.f;
    float z = 0.f;
    for (int s = 0; s < sg; ++s) {
      const float* PS = part_S + (static_cast<size_t>(bh) * segs + s) * M * kD;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[dt][i] += PS[(fb + drow(i, lane)) * kD + 32 * dt + (lane & 31)];
      z += part_z[(static_cast<size_t>(bh) * segs + s) * M + fb + (lane & 31)];
    }
    if (lane < 32) zl[wave][lane] = z;
  }

  const size_t rowbase = static_cast<size_t>(bh) * n;
  u32x4 xq[4], xk[4], vp[VPT];
  auto fetch = [&](int c0) {
    const int row = c0 + (lane & 31);
    const bool ok = row < t1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      xq[ks] = ok ? *reinterpret_cast<const u32x4*>(Q + (rowbase + row) * kD + 16 * ks + 8 * h) : u32x4{0u, 0u, 0u, 0u};
      xk[ks] = ok ? *reinterpret_cast<const u32x4*>(K + (rowbase + row) * kD + 16 * ks + 8 * h) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = t + NT * i, r = c >> 3, ch = c & 7;
      vp[i] = (c < 256 && c0 + r < t1) ? *reinterpret_cast<const u32x4*>(V + (rowbase + c0 + r) * kD + 8 * ch)
                                       : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto stage_v = [&](int par) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = t + NT * i;
      if (c < 256) *reinterpret_cast<u32x4*>(vt[par] + swz(c >> 3, c & 7)) = vp[i];
    }
  };

  if (t0 < t1) {
    fetch(t0);
    stage_v(0);
  }
  __syncthreads();
  int par = 0;
  for (int c0 = t0; c0 < t1; c0 += 32, par ^= 1) {
    const u32x4 cq[4] = {xq[0], xq[1], xq[2], xq[3]};
    const u32x4 ck[4] = {xk[0], xk[1], xk[2], xk[3]};
    if (c0 + 32 < t1) fetch(c0 + 32);
    // features of the chunk's queries and keys (FT: lane = token) and keys (TF: lane = feature)
    f32x16 pq = {}, pk = {}, pkt = {};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      pq = mfma_bf16(as_bf16x8(wop[ks]), as_bf16x8(cq[ks]), pq);
      pk = mfma_bf16(as_bf16x8(wop[ks]), as_bf16x8(ck[ks]), pk);
      pkt = mfma_bf16(as_bf16x8(ck[ks]), as_bf16x8(wop[ks]), pkt);
    }
    const bool key_ok = c0 + (lane & 31) < t1;
    float phq[16], phk[16], phkt[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      phq[i] = phi_of<KIND>(pq[i]);
      phk[i] = key_ok ? phi_of<KIND>(pk[i]) : 0.f;
      phkt[i] = c0 + drow(i, lane) < t1 ? phi_of<KIND>(pkt[i]) : 0.f;
    }
    u32x4 qhi[2], qlo[2], khi[2], klo[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      split8(phq, kb, qhi[kb], qlo[kb]);
      split8(phk, kb, khi[kb], klo[kb]);
    }
    // P^T = phi(K) phi(Q)^T over this wave's features: lane = query, register = key
    f32x16 pt = {};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      pt = mfma_bf16(as_bf16x8(khi[kb]), as_bf16x8(qhi[kb]), pt);
      pt = mfma_bf16(as_bf16x8(khi[kb]), as_bf16x8(qlo[kb]), pt);
      pt = mfma_bf16(as_bf16x8(klo[kb]), as_bf16x8(qhi[kb]), pt);
    }
    float den = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (drow(i, lane) > (lane & 31)) pt[i] = 0.f;   // keys after the query
      den += pt[i];
    }
    // carry term against the state before the chunk, and the chunk term
    f32x16 num[2] = {};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 phi_, plo_;
      split8(pt, kb, phi_, plo_);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        u32x4 shi_, slo_;
        split8(S[dt], kb, shi_, slo_);
        num[dt] = mfma_bf16(as_bf16x8(qhi[kb]), as_bf16x8(shi_), num[dt]);
        num[dt] = mfma_bf16(as_bf16x8(qhi[kb]), as_bf16x8(slo_), num[dt]);
        num[dt] = mfma_bf16(as_bf16x8(qlo[kb]), as_bf16x8(shi_), num[dt]);
        const u32x4 vb = v_operand(vt[par], 16 * kb, dt, lane);
        num[dt] = mfma_bf16(as_bf16x8(phi_), as_bf16x8(vb), num[dt]);
        num[dt] = mfma_bf16(as_bf16x8(plo_), as_bf16x8(vb), num[dt]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 zz = *reinterpret_cast<const f32x4*>(&zl[wave][8 * j + 4 * h]);
#pragma unroll
      for (int e = 0; e < 4; ++e) den = fmaf(phq[4 * j + e], zz[e], den);
    }
    den = pair_sum(den);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) part[wave][drow(i, lane)][32 * dt + (lane & 31)] = num[dt][i];
    if (lane < 32) dpart[wave][lane] = den;
    // the chunk's keys join the state
    float zs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 ahi, alo;
      split8(phkt, kb, ahi, alo);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const u32x4 vb = v_operand(vt[par], 16 * kb, dt, lane);
        S[dt] = mfma_bf16(as_bf16x8(ahi), as_bf16x8(vb), S[dt]);
        S[dt] = mfma_bf16(as_bf16x8(alo), as_bf16x8(vb), S[dt]);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) zs += phkt[i];
    zs = pair_sum(zs);
    if (lane < 32) zl[wave][lane] += zs;
    if (c0 + 32 < t1) stage_v(par ^ 1);
    __syncthreads();
    {
      // thread -> one query and CPQ consecutive columns: the waves' shares summed
      // in wave order, one reciprocal per query
      constexpr int CPQ = 32 * kD / NT;
      const int q = t / (kD / CPQ), cb = (t % (kD / CPQ)) * CPQ, r = c0 + q;
      if (r < t1) {
        float dsum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) dsum += dpart[w][q];
        const float rq = dsum > 0.f ? 1.f / dsum : 0.f;   // y = 0 for a query without weight
#pragma unroll
        for (int j = 0; j < CPQ / 4; ++j) {
          f32x4 acc4 = *reinterpret_cast<const f32x4*>(&part[0][q][cb + 4 * j]);
#pragma unroll
          for (int w = 1; w < NW; ++w) {
            const f32x4 p4 = *reinterpret_cast<const f32x4*>(&part[w][q][cb + 4 * j]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc4[e] += p4[e];
          }
          *reinterpret_cast<f32x4*>(out + (rowbase + r) * kD + cb + 4 * j) =
              f32x4{acc4[0] * rq, acc4[1] * rq, acc4[2] * rq, acc4[3] * rq};
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace

// Key ranges per (b, h): about one workgroup per CU at m >= 128 (4 or 8 waves
// each), two at m = 64 (2 waves each; its 16 KB range states keep the causal
// carry reads small).
int lin_splits(int BH, int n, int m) {
  const int target = m >= 128 ? 256 : 512;
  int s = (target + BH - 1) / BH;
  const int tiles = (n + 63) / 64;
  if (s > tiles) s = tiles;
  return s < 1 ? 1 : s;
}

LinPlan lin_plan(int B, int H, int n, int m, int kind, int causal) {
  LinPlan p{};
  p.B = B;
  p.H = H;
  p.n = n;
  p.m = m;
  p.kind = kind;
  p.causal = causal;
  const int BH = B * H;
  int s = lin_splits(BH, n, m);
  p.span = ((n + s - 1) / s + 63) / 64 * 64;
  p.splits = (n + p.span - 1) / p.span;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = bf16k::align_up(off + bytes, 256);
    return o;
  };
  p.off_part_S = take(static_cast<size_t>(BH) * p.splits * m * kD * 4);
  p.off_part_z = take(static_cast<size_t>(BH) * p.splits * m * 4);
  if (!causal) {
    p.off_sop = take(static_cast<size_t>(BH) * m * kD * 2 * 2);
    p.off_z = take(static_cast<size_t>(BH) * m * 4);
  }
  p.off_end = off;
  return p;
}

namespace {
template <int KIND, int M>
hipError_t launch_km(const LinPlan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     const uint16_t* W, float* out, void* ws, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  float* pS = reinterpret_cast<float*>(base + p.off_part_S);
  float* pz = reinterpret_cast<float*>(base + p.off_part_z);
  const int BH = p.B * p.H;
  auto kst = k_lin_state<KIND, M>;
  FAVOR_LAUNCH("k_lin_state", kst, dim3(BH * p.splits), dim3(2 * M), 0, s, k, v, W, pS, pz, p.H, p.n, p.splits,
               p.span);
  if (p.causal) {
    auto kc = k_lin_causal<KIND, M>;
    FAVOR_LAUNCH("k_lin_causal", kc, dim3(BH * p.splits), dim3(2 * M), 0, s, q, k, v, W, pS, pz, out, p.H, p.n,
                 p.splits, p.span);
  } else {
    u32x4* sop = reinterpret_cast<u32x4*>(base + p.off_sop);
    float* zz = reinterpret_cast<float*>(base + p.off_z);
    FAVOR_LAUNCH("k_lin_merge", k_lin_merge, dim3(BH * (M / 16)), dim3(128), 0, s, pS, pz, sop, zz, BH, M,
                 p.splits);
    const int ntiles = (p.n + 31) / 32;
    int qblocks = (256 + BH - 1) / BH;
    const int per = (ntiles + 7) / 8;   // workgroups that still have a tile for every wave
    if (qblocks > per) qblocks = per;
    if (qblocks < 1) qblocks = 1;
    auto ko = k_lin_output<KIND, M>;
    FAVOR_LAUNCH("k_lin_output", ko, dim3(BH * qblocks), dim3(512), 0, s, q, W, sop, zz, out, BH, p.H, p.n,
                 qblocks);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_linear_bf16(const LinPlan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const uint16_t* W, float* out, void* ws, hipStream_t s) {
  if (p.kind == kElu1) {
    if (p.m != kD) return hipErrorInvalidValue;
    return launch_km<kElu1, kD>(p, q, k, v, W, out, ws, s);
  }
  if (p.kind != kRelu) return hipErrorInvalidValue;
  switch (p.m) {
    case 64: return launch_km<kRelu, 64>(p, q, k, v, W, out, ws, s);
    case 128: return launch_km<kRelu, 128>(p, q, k, v, W, out, ws, s);
    case 256: return launch_km<kRelu, 256>(p, q, k, v, W, out, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lin
}  // namespace favor
