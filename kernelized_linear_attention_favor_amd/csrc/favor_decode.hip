// Streaming decode for FAVOR+ attention on gfx950: the causal prefix sums
// carried in a state from call to call (Performer for vision, How It Works,
// Step 2: each token adds its key features and value to running sums S and z,
// and reads them with its query; inclusive, as the causal path).
//
// State per (b, h) and feature f (fp32): S_f = sum_j 2^(e_jf - c_f) v_j,
// z_f = sum_j 2^(e_jf - c_f) and c_f, with e_jf = log2e (w_f.k_j - |k_j|^2/2).
// The feature map's 1/sqrt(m) and every factor common to a query row cancel
// in y_t = sum_f 2^(a_tf + c_f) S_f / sum_f 2^(a_tf + c_f) z_f, a_tf = log2e w_f.q_t.
//
// k_decode<M, CC>: one workgroup per (b, h) and slice of CC value columns
// (64 / CC workgroups per head, independent of one another: each keeps its own
// copy of the per-feature shift c_f and sum z_f, computed identically); thread
// f holds feature f's row of the slice, S_f[c0 .. c0+CC).  The T tokens go in
// blocks of 32:
//   * block set-up: the key and query logits of the block's tokens against the
//     head's M features, W k_t and W q_t, are one dense product per block
//     (32 tokens x 64 dims x M features) on bf16 MFMA with fp32 accumulation,
//     written to LDS; |k_t|^2 comes from the same key operand registers; the
//     block's values go to LDS as fp32; the next block's loads are issued.
//   * per token, thread f: the key joins feature f (c_f, z_f and its S row);
//     with g_f = a_f + c_f + log2 z_f and the wave's maximum G_w of it, each
//     wave sums r_f = 2^(g_f - G_w) / z_f times S_f over its 64 features with
//     a transposing butterfly (lane permutes, no LDS), and 2^(g_f - G_w).
//     Nothing crosses waves inside the token loop (no barrier): the state is
//     per feature and each wave keeps its own reference G_w.
//   * after the block: the waves' shares meet in LDS, rescaled to G = max G_w,
//   y = sum_f 2^(g_f - G) S_f / z_f  /  sum_f 2^(g_f - G).
// Every slice workgroup of a head reads z and c at its start, so they are
// written back only once all of them have: each takes a ticket from the head's
// counter in the state as soon as its threads hold z and c, and the one that
// drew the last ticket writes z and c at its end and clears the counter.
#include <math.h>

#include "favor_internal.h"
#include "favor_mfma.h"

namespace favor {
namespace {

constexpr int kDd = 64;   // head dimension of the decode path
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Lane permutes within rows of 16 (quad permutes, half-row and row mirrors:
// no lane reads outside its row, so the bound-control zero never applies);
// written so that the compiler folds them into the consuming add / max.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, true);
}
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;

// Sum / max of x over lanes l and l ^ 16, then l and l ^ 32 (register halves
// swapped between rows): the same operands in the same order on every lane.
__device__ __forceinline__ float sum_rows(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ int max_rows(int x) {
  auto r = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(x), static_cast<uint32_t>(x), false, false);
  x = max(static_cast<int>(r[0]), static_cast<int>(r[1]));
  r = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(x), static_cast<uint32_t>(x), false, false);
  return max(static_cast<int>(r[0]), static_cast<int>(r[1]));
}

// Maximum / sum over the 64 lanes, returned to every lane.  The maximum runs
// on integer keys that order like the floats (finite values; the key of a
// negative float flips its magnitude bits).
__device__ __forceinline__ float wave_max(float x) {
  const int b = __float_as_int(x);
  int k = b ^ ((b >> 31) & 0x7fffffff);
  k = max(k, dpp_i<kXor1>(k));
  k = max(k, dpp_i<kXor2>(k));
  k = max(k, dpp_i<kHalfMirror>(k));
  k = max(k, dpp_i<kMirror>(k));
  k = max_rows(k);
  return __int_as_float(k ^ ((k >> 31) & 0x7fffffff));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kXor1>(x);
  x += dpp<kXor2>(x);
  x += dpp<kHalfMirror>(x);
  x += dpp<kMirror>(x);
  return sum_rows(x);
}

// One halving step of the column butterfly across lane bit B: lanes with the
// bit clear keep column i (its sum over the lane pair), lanes with it set keep
// column i + h.  Bits 5 and 4 swap register halves between lanes (no select);
// bits 3 .. 0 pair the lanes with a mirror or quad permute.
template <int B>
__device__ __forceinline__ void halve(float& lo, float hi, bool up) {
  if constexpr (B == 5) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    lo = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else if constexpr (B == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    lo = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    constexpr int ctrl = B == 3 ? kMirror : B == 2 ? kHalfMirror : B == 1 ? kXor2 : kXor1;
    const float a = lo + dpp<ctrl>(lo);
    const float b = hi + dpp<ctrl>(hi);
    lo = up ? b : a;
  }
}

// Sum of x[i] over the wave's 64 lanes for each column i < CC: lane l ends with
// column l >> (6 - log2 CC), summed over all 64 lanes.
template <int CC>
__device__ __forceinline__ float column_sums(float (&x)[CC], int lane) {
  constexpr int LB = __builtin_ctz(CC);   // halving levels: lane bits 5 .. 6-LB
#pragma unroll
  for (int lv = 0; lv < LB; ++lv) {
    const int h = CC >> (lv + 1);
    const int bit = 5 - lv;
    const bool up = (lane >> bit) & 1;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      switch (bit) {
        case 5: halve<5>(x[i], x[i + h], up); break;
        case 4: halve<4>(x[i], x[i + h], up); break;
        case 3: halve<3>(x[i], x[i + h], up); break;
        case 2: halve<2>(x[i], x[i + h], up); break;
        case 1: halve<1>(x[i], x[i + h], up); break;
        default: halve<0>(x[i], x[i + h], up); break;
      }
    }
  }
  float y = x[0];
  // the remaining lane bits (6-LB-1 .. 0) hold partial sums of the same column
  if constexpr (LB <= 5) y += dpp<kXor1>(y);
  if constexpr (LB <= 4) y += dpp<kXor2>(y);
  if constexpr (LB <= 3) y += dpp<kHalfMirror>(y);
  if constexpr (LB <= 2) y += dpp<kMirror>(y);
  if constexpr (LB == 1) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    y = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (LB == 0) y = sum_rows(y);
  return y;
}

constexpr int kTB = 32;    // tokens per block: the row tile of one MFMA

template <int M, int CC>
struct DecSmem {
  static constexpr int NW = M / 64;
  static constexpr int LD = M + 4;   // padded logit rows: the two lane halves of an MFMA store hit different banks
  float eL[kTB][LD];                 // W k_t of the block (unscaled)
  float aL[kTB][LD];                 // W q_t of the block (unscaled)
  float vL[kTB][kDd];                // values of the block
  float part[kTB][NW][CC];           // per-wave column sums of the numerator, per token of the block
  float wdn[kTB][NW];                // per-wave sums of the denominator, per token of the block
  float wmx[kTB][NW];                // per-wave maxima of g (the shares' reference), per token
  uint32_t ticket;                   // this workgroup's place among the head's slices
};

template <int M, int CC>
__global__ __launch_bounds__(M) void k_decode(const uint16_t* __restrict__ Q,
                                              const uint16_t* __restrict__ K,
                                              const uint16_t* __restrict__ V,
                                              const uint16_t* __restrict__ W,
                                              float* __restrict__ state, float* __restrict__ out,
                                              int BH, int H, int T) {
  constexpr int NW = M / 64;
  constexpr int NS = kDd / CC;          // column slices per head
  constexpr int VW = kTB * 32 / M;      // value words (bf16 pairs) each thread stages per block
  constexpr int GB = 6 - __builtin_ctz(CC);   // lane l holds column l >> GB after the butterfly
  __shared__ __attribute__((aligned(16))) DecSmem<M, CC> sm;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // Workgroups go to the 8 XCDs round-robin by index, so with BH a multiple of
  // 8 the NS slices of one (b, h) share an XCD and its L2: the state rows, z, c
  // and W of the head are fetched from memory once, not once per slice.
  const int bh = blockIdx.x % BH, cs = blockIdx.x / BH, hh = bh % H;
  const int c0 = cs * CC;

  // W as the MFMA B operand (16 dims x 32 features per tile, two tiles per wave)
  u32x4 wop[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint16_t* wr = W + (static_cast<size_t>(hh) * M + 64 * wave + 32 * j + (lane & 31)) * kDd + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) wop[j][ks] = *reinterpret_cast<const u32x4*>(wr + 16 * ks);
  }

  // the state: feature t's row slice of S, its z and c
  float S[CC];
  float* Sg = state + (static_cast<size_t>(bh) * M + t) * kDd + c0;
#pragma unroll
  for (int j = 0; j < CC / 4; ++j) {
    const f32x4 r = reinterpret_cast<const f32x4*>(Sg)[j];
    S[4 * j] = r[0];
    S[4 * j + 1] = r[1];
    S[4 * j + 2] = r[2];
    S[4 * j + 3] = r[3];
  }
  float* zg = state + static_cast<size_t>(BH) * M * kDd + static_cast<size_t>(bh) * M + t;
  float z = zg[0], c = zg[static_cast<size_t>(BH) * M];
  uint32_t* cnt = reinterpret_cast<uint32_t*>(state + static_cast<size_t>(BH) * M * (kDd + 2)) + bh;
  uint32_t ticket = 0;

  const size_t tok_base = static_cast<size_t>(bh) * T;
  u32x4 qop[4], kop[4];
  uint32_t vw[VW];
  auto load_block = [&](int tok0) {
    const int row = tok0 + (lane & 31);
    const bool ok = row < T;
    const size_t off = (tok_base + row) * kDd + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qop[ks] = ok ? *reinterpret_cast<const u32x4*>(Q + off + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
      kop[ks] = ok ? *reinterpret_cast<const u32x4*>(K + off + 16 * ks) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < VW; ++i) {
      const int w = t + M * i, tt = w >> 5, pr = w & 31;
      vw[i] = tok0 + tt < T ? *reinterpret_cast<const uint32_t*>(V + (tok_base + tok0 + tt) * kDd + 2 * pr) : 0u;
    }
  };

  load_block(0);
  for (int tok0 = 0; tok0 < T; tok0 += kTB) {
    const int nb = T - tok0 < kTB ? T - tok0 : kTB;
    // |k|^2 of token lane % 32: each lane half holds 32 of its 64 dims
    float kk = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float lo = bf16_lo(kop[ks][s]), hi = bf16_hi(kop[ks][s]);
        kk = fmaf(lo, lo, kk);
        kk = fmaf(hi, hi, kk);
      }
    kk = pair_sum(kk);
    // logits of the block: rows = tokens, columns = this wave's 64 features
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x16 ae = {}, aa = {};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        ae = mfma_bf16(as_bf16x8(kop[ks]), as_bf16x8(wop[j][ks]), ae);
        aa = mfma_bf16(as_bf16x8(qop[ks]), as_bf16x8(wop[j][ks]), aa);
      }
      const int fcol = 64 * wave + 32 * j + (lane & 31);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (row < nb) {
          sm.eL[row][fcol] = ae[i];
          sm.aL[row][fcol] = aa[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < VW; ++i) {
      const int w = t + M * i, tt = w >> 5, pr = w & 31;
      *reinterpret_cast<f32x2*>(&sm.vL[tt][2 * pr]) = f32x2{bf16_lo(vw[i]), bf16_hi(vw[i])};
    }
    if (tok0 + kTB < T) load_block(tok0 + kTB);

    if (tok0 == 0) {
      // every thread holds its z and c before the barrier; then the workgroup
      // takes its ticket (the result is read at the end)
      asm volatile("" ::"v"(z), "v"(c));
    }
    __syncthreads();
    if constexpr (NS > 1) {
      if (tok0 == 0 && t == 0) ticket = atomicAdd(cnt, 1u);
    }

    // Per token: the key joins feature t (the shift follows the largest
    // exponent), then the query reads the wave's features relative to the
    // wave's maximum.  Hardware exp2 / log2 / reciprocal: every exp2 argument
    // is <= 0 (a result below the normal range only drops a term under 2^-126
    // of the largest one, which is 1), and z >= 1 since the key that set c
    // counts 1.
    auto join = [&](int tt) {
      const float kkt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kk), tt));
      const float e = kLog2e * fmaf(-0.5f, kkt, sm.eL[tt][t]);
      const float a = kLog2e * sm.aL[tt][t];
      const float cn = fmaxf(c, e);
      const float scf = fast_exp2(c - cn);   // 1 if the shift stays, 0 from the empty state
      const float p = fast_exp2(e - cn);
      z = fmaf(z, scf, p);
      c = cn;
#pragma unroll
      for (int j = 0; j < CC / 4; ++j) {
        const f32x4 vv = *reinterpret_cast<const f32x4*>(&sm.vL[tt][c0 + 4 * j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) S[4 * j + i] = fmaf(p, vv[i], S[4 * j + i] * scf);
      }
      return a + c + __builtin_amdgcn_logf(z);   // g
    };
    auto read = [&](float g, float zt, const float (&Sx)[CC], int tt) {
      const float gw = wave_max(g);
      const float om = fast_exp2(g - gw);
      const float r = om * fast_rcp(zt);
      float x[CC];
#pragma unroll
      for (int i = 0; i < CC; ++i) x[i] = r * Sx[i];
      const float col = column_sums<CC>(x, lane);
      const float dw = wave_sum(om);
      if ((lane & ((1 << GB) - 1)) == 0) sm.part[tt][wave][lane >> GB] = col;
      if (lane == 0) {
        sm.wdn[tt][wave] = dw;
        sm.wmx[tt][wave] = gw;
      }
    };
    int tt = 0;
    if constexpr (CC <= 16) {
      // two tokens at a time: token tt's read and token tt+1's join are
      // independent and interleave
      for (; tt + 1 < nb; tt += 2) {
        const float gA = join(tt);
        const float zA = z;
        float SA[CC];
#pragma unroll
        for (int i = 0; i < CC; ++i) SA[i] = S[i];
        const float gB = join(tt + 1);
        read(gA, zA, SA, tt);
        read(gB, z, S, tt + 1);
      }
    }
    for (; tt < nb; ++tt) {
      const float g = join(tt);
      read(g, z, S, tt);
    }
    __syncthreads();
    // the block's outputs: the waves' shares rescaled to the largest reference
    // and summed in wave order
    for (int o = t; o < nb * CC; o += M) {
      const int tt = o / CC, cc = o % CC;
      float gm = sm.wmx[tt][0];
#pragma unroll
      for (int w = 1; w < NW; ++w) gm = fmaxf(gm, sm.wmx[tt][w]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float sw = exp2f(sm.wmx[tt][w] - gm);
        num = fmaf(sm.part[tt][w][cc], sw, num);
        den = fmaf(sm.wdn[tt][w], sw, den);
      }
      out[(tok_base + tok0 + tt) * kDd + c0 + cc] = num / den;
    }
  }

#pragma unroll
  for (int j = 0; j < CC / 4; ++j)
    reinterpret_cast<f32x4*>(Sg)[j] = f32x4{S[4 * j], S[4 * j + 1], S[4 * j + 2], S[4 * j + 3]};
  if constexpr (NS > 1) {
    if (t == 0) sm.ticket = ticket;
    __syncthreads();
    if (sm.ticket != NS - 1) return;
    if (t == 0) *cnt = 0u;
  }
  zg[0] = z;
  zg[static_cast<size_t>(BH) * M] = c;
}

// The empty state: S = 0, z = 0, c = -inf, finish counters 0.
__global__ void k_state_reset(float* __restrict__ state, size_t n_s, size_t n_z, size_t n_bh) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t j = i; j < n_s + 2 * n_z + n_bh; j += stride)
    state[j] = (j < n_s + n_z || j >= n_s + 2 * n_z) ? 0.f : kNegInf;
}

}  // namespace

size_t state_floats(int B, int H, int d, int m) {
  return static_cast<size_t>(B) * H * (static_cast<size_t>(m) * (d + 2) + 1);
}

hipError_t launch_state_reset(float* state, int B, int H, int d, int m, hipStream_t s) {
  const size_t n_bh = static_cast<size_t>(B) * H;
  const size_t n_s = n_bh * m * d, n_z = n_bh * m;
  const size_t total = n_s + 2 * n_z + n_bh;
  const int blocks = static_cast<int>((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  FAVOR_LAUNCH("k_state_reset", k_state_reset, dim3(blocks), dim3(256), 0, s, state, n_s, n_z, n_bh);
  return hipGetLastError();
}

template <int M, int CC>
hipError_t launch_decode_mc(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* W,
                            float* state, float* out, int BH, int H, int T, hipStream_t s) {
  auto kern = k_decode<M, CC>;
  FAVOR_LAUNCH("k_decode", kern, dim3(BH * (kDd / CC)), dim3(M), 0, s, q, k, v, W, state, out, BH, H, T);
  return hipGetLastError();
}

template <int M>
hipError_t launch_decode_m(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* W,
                           float* state, float* out, int BH, int H, int T, int cc, hipStream_t s) {
  switch (cc) {
    case 8: return launch_decode_mc<M, 8>(q, k, v, W, state, out, BH, H, T, s);
    case 16: return launch_decode_mc<M, 16>(q, k, v, W, state, out, BH, H, T, s);
    case 32: return launch_decode_mc<M, 32>(q, k, v, W, state, out, BH, H, T, s);
    default: return launch_decode_mc<M, 64>(q, k, v, W, state, out, BH, H, T, s);
  }
}

// Columns per workgroup: the narrowest slice (most workgroups per head, the
// shortest per-token path) while the grid stays within about four workgroups
// per compute unit; wider slices repeat the per-feature work fewer times.
int decode_columns(int BH) {
  int cc = 8;
  while (cc < kDd && static_cast<long long>(BH) * (kDd / cc) > 1024) cc *= 2;
  return cc;
}

hipError_t launch_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* W,
                         float* state, float* out, int B, int H, int T, int m, hipStream_t s) {
  const int BH = B * H;
  const int cc = decode_columns(BH);
  switch (m) {
    case 64: return launch_decode_m<64>(q, k, v, W, state, out, BH, H, T, cc, s);
    case 128: return launch_decode_m<128>(q, k, v, W, state, out, BH, H, T, cc, s);
    case 256: return launch_decode_m<256>(q, k, v, W, state, out, BH, H, T, cc, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace favor
