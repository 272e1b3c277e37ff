// Orthogonal random features drawn on the device (Performer for vision, Kernel
// Choices: QR of random projection matrices gives orthogonal features with
// lower variance; Performer notes, FAVOR+: the random directions w_f).
//
// Random numbers: Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", 2011), written from its published
// definition, with key (seed, step) and counter (i, block, head, kind); block i
// of a stream gives normals 4i .. 4i+3 by two Box-Muller pairs (words 0-1, then
// 2-3; cos then sin), each word mapped to (0, 1) by its top 53 bits.
//
// Per head and block b of d rows (one workgroup; column j held by 4 threads,
// a quarter of its rows each, their partial sums combined by lane shuffles):
//   G[r][c] = normal r*d + c of stream kind 0  ->  LDS  ->  columns in registers;
//   modified Gram-Schmidt in fp64 (R's diagonal comes out positive, the QR that
//   makes Q unique): q_k is published through LDS, every later column removes
//   its component;
//   s_j = |g_j|, g_j = normals j*d .. j*d + d-1 of stream kind 1 (chi(d));
//   W[h][b*d + j][:] = s_j q_j  (rows below m), written as fp32 or as bf16,
//   each rounded once from fp64 to nearest even (bf16 through an fp32 value
//   rounded to odd, which keeps the second rounding exact: Boldo and
//   Melquiond, "Emulation of FMA and correctly rounded sums: proved
//   algorithms using rounding to odd", 2008).
#include <math.h>

#include "favor_internal.h"
#include "favor_mfma.h"

namespace favor {
namespace draw {
namespace {

constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;

// One Philox4x64-10 block, in place on the counter words.
__device__ __forceinline__ void philox4x64_10(uint64_t& c0, uint64_t& c1, uint64_t& c2, uint64_t& c3,
                                              uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t lo0 = kM0 * c0, hi0 = __umul64hi(kM0, c0);
    const uint64_t lo1 = kM1 * c2, hi1 = __umul64hi(kM1, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += kW0;
    k1 += kW1;
  }
}

__device__ __forceinline__ double unit(uint64_t w) {
  return (static_cast<double>(w >> 11) + 0.5) * 0x1p-53;
}

// Normals 4i .. 4i+3 of stream (head, block, kind) into dst[0..3].  The angle
// 2 pi u goes through sincospi(2u): the same cosine and sine, without reducing
// a multiple of pi.
__device__ __forceinline__ void normals4(uint64_t seed, uint64_t step, int head, int block, int kind,
                                         uint64_t i, double* dst) {
  uint64_t c0 = i, c1 = static_cast<uint64_t>(block), c2 = static_cast<uint64_t>(head),
           c3 = static_cast<uint64_t>(kind);
  philox4x64_10(c0, c1, c2, c3, seed, step);
  double sn, cs;
  double r = sqrt(-2.0 * log(unit(c0)));
  sincospi(2.0 * unit(c1), &sn, &cs);
  dst[0] = r * cs;
  dst[1] = r * sn;
  r = sqrt(-2.0 * log(unit(c2)));
  sincospi(2.0 * unit(c3), &sn, &cs);
  dst[2] = r * cs;
  dst[3] = r * sn;
}

// Sum over the 4 lanes 4j .. 4j+3 (the threads of one column), returned to all four.
__device__ __forceinline__ double quad_sum(double x) {
  x += __shfl_xor(x, 1);
  return x + __shfl_xor(x, 2);
}

// fp64 -> fp32 rounded to odd: truncate toward zero and, if anything was
// dropped, set the last bit.
__device__ __forceinline__ float round_to_odd_f32(double x) {
  float f = static_cast<float>(x);
  if (static_cast<double>(f) != x) {
    if (fabs(static_cast<double>(f)) > fabs(x)) f = __uint_as_float(__float_as_uint(f) - 1u);
    f = __uint_as_float(__float_as_uint(f) | 1u);
  }
  return f;
}

template <int D>
__global__ __launch_bounds__(256) void k_draw_features(uint64_t seed, uint64_t step, void* __restrict__ W,
                                                       int out_f32, int m, int nblocks) {
  constexpr int RPT = D / 4;   // rows of a column per thread
  __shared__ double buf[D * D];
  __shared__ double qk[2][D];
  const int t = threadIdx.x, j = t >> 2, p = t & 3;   // column j, row quarter p
  const bool col = j < D;
  const int h = blockIdx.x / nblocks, b = blockIdx.x % nblocks;
  const int rows = min(D, m - b * D);

  for (int i = t; i < D * D / 4; i += 256) normals4(seed, step, h, b, 0, static_cast<uint64_t>(i), &buf[4 * i]);
  __syncthreads();
  double a[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) a[r] = col ? buf[(RPT * p + r) * D + j] : 0.0;
  __syncthreads();
  for (int i = t; i < D * D / 4; i += 256) normals4(seed, step, h, b, 1, static_cast<uint64_t>(i), &buf[4 * i]);
  __syncthreads();
  double s = 0.0;
  if (col) {
#pragma unroll
    for (int c = 0; c < RPT; ++c) s = fma(buf[j * D + RPT * p + c], buf[j * D + RPT * p + c], s);
  }
  s = sqrt(quad_sum(s));

  for (int k = 0; k < D; ++k) {
    double nn = 0.0;
#pragma unroll
    for (int r = 0; r < RPT; ++r) nn = fma(a[r], a[r], nn);
    nn = quad_sum(nn);   // all lanes take part in the shuffles
    if (j == k) {
      const double rkk = sqrt(nn);
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        a[r] /= rkk;
        qk[k & 1][RPT * p + r] = a[r];
      }
    }
    __syncthreads();   // q_k published; q_{k-1}'s readers are done with it
    double dot = 0.0;
#pragma unroll
    for (int r = 0; r < RPT; ++r) dot = fma(qk[k & 1][RPT * p + r], a[r], dot);
    dot = quad_sum(dot);
    if (col && j > k) {
#pragma unroll
      for (int r = 0; r < RPT; ++r) a[r] = fma(-dot, qk[k & 1][RPT * p + r], a[r]);
    }
  }

  if (j < rows) {
    const size_t row = static_cast<size_t>(h) * m + b * D + j;
    if (out_f32) {
      float* o = static_cast<float*>(W) + row * D + RPT * p;
#pragma unroll
      for (int c = 0; c < RPT; ++c) o[c] = static_cast<float>(s * a[c]);
    } else {
      uint32_t* o = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(W) + row * D + RPT * p);
#pragma unroll
      for (int c = 0; c < RPT; c += 2)
        o[c / 2] = pack_bf16(round_to_odd_f32(s * a[c]), round_to_odd_f32(s * a[c + 1]));
    }
  }
}

}  // namespace

bool draw_supported(int d) { return d == 16 || d == 32 || d == 64; }

hipError_t launch_draw_features(uint64_t seed, uint64_t step, void* W, int out_f32, int H, int m, int d,
                                hipStream_t s) {
  const int nb = (m + d - 1) / d;
  switch (d) {
    case 16: {
      auto k = k_draw_features<16>;
      FAVOR_LAUNCH("k_draw_features", k, dim3(H * nb), dim3(256), 0, s, seed, step, W, out_f32, m, nb);
      break;
    }
    case 32: {
      auto k = k_draw_features<32>;
      FAVOR_LAUNCH("k_draw_features", k, dim3(H * nb), dim3(256), 0, s, seed, step, W, out_f32, m, nb);
      break;
    }
    case 64: {
      auto k = k_draw_features<64>;
      FAVOR_LAUNCH("k_draw_features", k, dim3(H * nb), dim3(256), 0, s, seed, step, W, out_f32, m, nb);
      break;
    }
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace draw
}  // namespace favor
