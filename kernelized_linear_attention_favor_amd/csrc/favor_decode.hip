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
// k_decode: one workgroup per (b, h), thread f = feature f holding S_f (64
// floats), z_f and c_f in registers for the whole call; the T tokens are taken
// in order.  Per token: q, k, v to LDS; each feature's key exponent e_f and
// query exponent a_f (fp32 dot products against its W row); the key joins the
// state (c_f rises to e_f when e_f exceeds it, rescaling S_f and z_f); the row
// reads the state as a softmax over features, g_f = a_f + c_f + log2 z_f:
//   y = sum_f 2^(g_f - G) S_f / z_f  /  sum_f 2^(g_f - G),   G = max_f g_f,
// with the sums over features done per wave by recursive halving (lane l ends
// with value column l) and across waves through LDS.
#include <math.h>

#include "favor_internal.h"
#include "favor_mfma.h"

namespace favor {
namespace {

constexpr int kDd = 64;   // head dimension of the decode path
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Sum over the 64 lanes of a wave of r * S[0..63] (one 64-vector per lane);
// lane l returns the sum of element l.  Each halving step keeps one half of
// the current index range (the upper one on lanes with that bit set) and adds
// the partner's copy of it; the first step forms the products as it goes.
__device__ __forceinline__ float wave_vec_sum(float r, const float (&S)[kDd], int lane) {
  float x[kDd / 2];
  {
    const bool up = (lane & 32) != 0;
#pragma unroll
    for (int i = 0; i < kDd / 2; ++i) {
      const float lo = r * S[i], hi = r * S[i + kDd / 2];
      x[i] = (up ? hi : lo) + __shfl_xor(up ? lo : hi, 32);
    }
  }
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) {
    const bool up = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < o; ++i) {
      const float keep = up ? x[i + o] : x[i];
      const float give = up ? x[i] : x[i + o];
      x[i] = keep + __shfl_xor(give, o);
    }
  }
  return x[0];
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int M>
__global__ __launch_bounds__(M, 1) void k_decode(const uint16_t* __restrict__ Q,
                                              const uint16_t* __restrict__ K,
                                              const uint16_t* __restrict__ V,
                                              const uint16_t* __restrict__ W,
                                              float* __restrict__ state, float* __restrict__ out,
                                              int BH, int H, int T) {
  constexpr int NWV = M / 64;
  __shared__ __attribute__((aligned(16))) float qkv[3][kDd];
  __shared__ __attribute__((aligned(16))) float red[NWV][kDd];
  __shared__ float wmx[NWV], wdn[NWV];
  const int f = threadIdx.x, lane = f & 63, wave = f >> 6;
  const int bh = blockIdx.x, hh = bh % H;

  float* Sg = state + (static_cast<size_t>(bh) * M + f) * kDd;
  float* zg = state + static_cast<size_t>(BH) * M * kDd + static_cast<size_t>(bh) * M + f;
  float* cg = zg + static_cast<size_t>(BH) * M;
  float S[kDd];
#pragma unroll
  for (int j = 0; j < kDd / 4; ++j) {
    const f32x4 t = reinterpret_cast<const f32x4*>(Sg)[j];
    S[4 * j] = t[0];
    S[4 * j + 1] = t[1];
    S[4 * j + 2] = t[2];
    S[4 * j + 3] = t[3];
  }
  float z = *zg, c = *cg;
  // the feature's W row, kept as bf16 pairs
  u32x4 w[kDd / 8];
  {
    const u32x4* wr = reinterpret_cast<const u32x4*>(W + (static_cast<size_t>(hh) * M + f) * kDd);
#pragma unroll
    for (int j = 0; j < kDd / 8; ++j) w[j] = wr[j];
  }

  for (int t = 0; t < T; ++t) {
    const size_t tok = static_cast<size_t>(bh) * T + t;
    for (int i = f; i < 96; i += M) {   // q, k, v of the token as fp32: 3 vectors x 32 bf16 pairs
      const int vec = i >> 5, pr = i & 31;
      const uint16_t* src = (vec == 0 ? Q : vec == 1 ? K : V) + tok * kDd + 2 * pr;
      const uint32_t u = *reinterpret_cast<const uint32_t*>(src);
      qkv[vec][2 * pr] = bf16_lo(u);
      qkv[vec][2 * pr + 1] = bf16_hi(u);
    }
    __syncthreads();
    float e = 0.f, kk = 0.f, a = 0.f;
#pragma unroll
    for (int j = 0; j < kDd / 4; ++j) {
      const f32x4 kq = *reinterpret_cast<const f32x4*>(&qkv[1][4 * j]);
      const f32x4 qq = *reinterpret_cast<const f32x4*>(&qkv[0][4 * j]);
      const uint32_t w01 = w[j >> 1][2 * (j & 1)], w23 = w[j >> 1][2 * (j & 1) + 1];
      const float wv[4] = {bf16_lo(w01), bf16_hi(w01), bf16_lo(w23), bf16_hi(w23)};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e = fmaf(wv[i], kq[i], e);
        kk = fmaf(kq[i], kq[i], kk);
        a = fmaf(wv[i], qq[i], a);
      }
    }
    e = kLog2e * fmaf(-0.5f, kk, e);
    a *= kLog2e;
    // the key joins the state; the shift follows the largest exponent
    if (e > c) {
      const float sc = c == kNegInf ? 0.f : exp2f(c - e);
#pragma unroll
      for (int i = 0; i < kDd; ++i) S[i] *= sc;
      z *= sc;
      c = e;
    }
    const float p = exp2f(e - c);
#pragma unroll
    for (int j = 0; j < kDd / 4; ++j) {
      const f32x4 vq = *reinterpret_cast<const f32x4*>(&qkv[2][4 * j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) S[4 * j + i] = fmaf(p, vq[i], S[4 * j + i]);
    }
    z += p;
    // the query reads the state: a softmax over features (z > 0: this key is in)
    const float g = a + c + log2f(z);
    float gm = wave_max(g);
    if (lane == 0) wmx[wave] = gm;
    __syncthreads();
    gm = wmx[0];
#pragma unroll
    for (int i = 1; i < NWV; ++i) gm = fmaxf(gm, wmx[i]);
    const float om = exp2f(g - gm);
    const float r = om / z;
    const float num = wave_vec_sum(r, S, lane);
    const float den = wave_sum(om);
    red[wave][lane] = num;
    if (lane == 0) wdn[wave] = den;
    __syncthreads();
    if (wave == 0) {
      float nsum = red[0][lane], dsum = wdn[0];
#pragma unroll
      for (int i = 1; i < NWV; ++i) {
        nsum += red[i][lane];
        dsum += wdn[i];
      }
      out[tok * kDd + lane] = nsum / dsum;
    }
  }

#pragma unroll
  for (int j = 0; j < kDd / 4; ++j)
    reinterpret_cast<f32x4*>(Sg)[j] = f32x4{S[4 * j], S[4 * j + 1], S[4 * j + 2], S[4 * j + 3]};
  *zg = z;
  *cg = c;
}

// The empty state: S = 0, z = 0, c = -inf.
__global__ void k_state_reset(float* __restrict__ state, size_t n_s, size_t n_z) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t j = i; j < n_s + 2 * n_z; j += stride)
    state[j] = j < n_s + n_z ? 0.f : kNegInf;
}

}  // namespace

size_t state_floats(int B, int H, int d, int m) {
  return static_cast<size_t>(B) * H * m * (d + 2);
}

hipError_t launch_state_reset(float* state, int B, int H, int d, int m, hipStream_t s) {
  const size_t n_s = static_cast<size_t>(B) * H * m * d, n_z = static_cast<size_t>(B) * H * m;
  const size_t total = n_s + 2 * n_z;
  const int blocks = static_cast<int>((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  FAVOR_LAUNCH("k_state_reset", k_state_reset, dim3(blocks), dim3(256), 0, s, state, n_s, n_z);
  return hipGetLastError();
}

hipError_t launch_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* W,
                         float* state, float* out, int B, int H, int T, int m, hipStream_t s) {
  const int BH = B * H;
  switch (m) {
    case 64:
      FAVOR_LAUNCH("k_decode", k_decode<64>, dim3(BH), dim3(64), 0, s, q, k, v, W, state, out, BH, H, T);
      break;
    case 128:
      FAVOR_LAUNCH("k_decode", k_decode<128>, dim3(BH), dim3(128), 0, s, q, k, v, W, state, out, BH, H, T);
      break;
    case 256:
      FAVOR_LAUNCH("k_decode", k_decode<256>, dim3(BH), dim3(256), 0, s, q, k, v, W, state, out, BH, H, T);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace favor
