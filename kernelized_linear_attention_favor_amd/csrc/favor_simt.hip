// fp32 (SIMT) kernels: the exact feature map, and FAVOR+ attention with fp32
// inputs and fp32 arithmetic throughout.
//
// Method (Performer notes: FAVOR+, Kernel Attention View, Normalization;
// Performer for vision: How It Works, Steps 1-2):
//   phi(x) = exp(W x - |x|^2/2) / sqrt(m),  S = Phi(K)^T V,  z = Phi(K)^T 1,
//   y_i = phi(q_i)^T S / phi(q_i)^T z   (causal: S, z summed over keys j <= i).
//
// Stabilised evaluation used by the attention kernels (all exact rewrites):
//  * keys: e_jf = w_f.k_j - |k_j|^2/2 is shifted by a per-feature constant c_f
//    shared by every key of the (batch, head), so S_f and z_f are both scaled
//    by exp(-c_f); c_f is carried along explicitly.
//  * queries: the factor exp(-|q_i|^2/2)/sqrt(m) is the same for every feature
//    of row i and cancels in the ratio, as does 1/sqrt(m) on the key side.
//  * with yhat_f = S_f / z_f and beta_f = c_f + log(z_f - in c_f units),
//        y_i = sum_f softmax_f(w_f.q_i + beta_f) * yhat_f,
//    a softmax over features whose row maximum is subtracted before exp.
#include "favor_internal.h"

#include <math.h>

namespace favor {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float load_as_f32(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_as_f32(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}

// ---------------------------------------------------------------------------
// Exact feature map.  One block computes a 32-token x 64-feature tile.
// Threads: feature lane fl = tid % 64, token group tg = tid / 64 (8 tokens each).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_feature_map(const T* __restrict__ x,
                                                     const T* __restrict__ W,
                                                     float* __restrict__ phi, int H, int n, int d,
                                                     int m, float inv_sqrt_m) {
  extern __shared__ float sm[];
  const int ldx = d + 1;
  float* xs = sm;                // [32][d+1]
  float* wsh = xs + 32 * ldx;    // [64][d+1]
  float* half_sq = wsh + 64 * ldx;  // [32]
  const int bh = blockIdx.z;
  const int h = bh % H;
  const int t0 = blockIdx.x * 32;
  const int f0 = blockIdx.y * 64;
  const T* xb = x + static_cast<size_t>(bh) * n * d;
  const T* wb = W + static_cast<size_t>(h) * m * d;
  for (int idx = threadIdx.x; idx < 32 * d; idx += 256) {
    const int r = idx / d, c = idx - r * d;
    const int t = t0 + r;
    xs[r * ldx + c] = (t < n) ? load_as_f32(xb, static_cast<size_t>(t) * d + c) : 0.f;
  }
  for (int idx = threadIdx.x; idx < 64 * d; idx += 256) {
    const int r = idx / d, c = idx - r * d;
    const int f = f0 + r;
    wsh[r * ldx + c] = (f < m) ? load_as_f32(wb, static_cast<size_t>(f) * d + c) : 0.f;
  }
  __syncthreads();
  if (threadIdx.x < 32) {
    float s = 0.f;
    for (int c = 0; c < d; ++c) s = fmaf(xs[threadIdx.x * ldx + c], xs[threadIdx.x * ldx + c], s);
    half_sq[threadIdx.x] = 0.5f * s;
  }
  __syncthreads();
  const int fl = threadIdx.x & 63;
  const int tg = threadIdx.x >> 6;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int c = 0; c < d; ++c) {
    const float w = wsh[fl * ldx + c];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(xs[(tg * 8 + i) * ldx + c], w, acc[i]);
  }
  const int f = f0 + fl;
  if (f < m) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = tg * 8 + i;
      const int t = t0 + r;
      if (t < n) phi[(static_cast<size_t>(bh) * n + t) * m + f] = expf(acc[i] - half_sq[r]) * inv_sqrt_m;
    }
  }
}

template <typename T>
hipError_t launch_fm(const T* x, const T* W, float* phi, int B, int H, int n, int d, int m,
                     hipStream_t s) {
  const size_t lds = static_cast<size_t>(96 * (d + 1) + 32) * sizeof(float);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_feature_map<T>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  dim3 grid((n + 31) / 32, (m + 63) / 64, B * H);
  FAVOR_LAUNCH("k_feature_map", k_feature_map<T>, grid, dim3(256), lds, s, x, W, phi, H, n, d, m,
                     1.0f / sqrtf(static_cast<float>(m)));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 attention, non-causal.
// Pass A: per (split, b, h) -- per-feature max c_f of the key exponents over
// the split, then z_f = sum exp(e - c_f), S_f = sum exp(e - c_f) v.
// Pass B: per (b, h) -- combine splits in fixed order; yhat = S/z,
// beta = c + log z.
// Pass C: per 64 queries -- softmax over features of w_f.q + beta_f, times yhat.
// ---------------------------------------------------------------------------
constexpr int kF32Tile = 16;   // tokens staged per step in pass A
constexpr int kF32Splits = 8;  // key-range splits per (b, h)

struct F32Ws {
  float* c;     // [BH][splits][m]
  float* z;     // [BH][splits][m]
  float* S;     // [BH][splits][m][d]
  float* yhat;  // [BH][m][d]
  float* beta;  // [BH][m]
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

F32Ws carve_f32(void* ws, int BH, int d, int m) {
  char* p = static_cast<char*>(ws);
  F32Ws w;
  size_t o = 0;
  w.c = reinterpret_cast<float*>(p + o);
  o = align256(o + sizeof(float) * BH * kF32Splits * m);
  w.z = reinterpret_cast<float*>(p + o);
  o = align256(o + sizeof(float) * BH * kF32Splits * m);
  w.S = reinterpret_cast<float*>(p + o);
  o = align256(o + sizeof(float) * BH * kF32Splits * m * d);
  w.yhat = reinterpret_cast<float*>(p + o);
  o = align256(o + sizeof(float) * BH * m * d);
  w.beta = reinterpret_cast<float*>(p + o);
  return w;
}

__global__ __launch_bounds__(256) void k_state_f32(const float* __restrict__ k,
                                                   const float* __restrict__ v,
                                                   const float* __restrict__ W, F32Ws ws, int H,
                                                   int n, int d, int m, int span) {
  extern __shared__ float sm[];
  const int ld = d + 1;
  float* S = sm;                        // [m][d+1]
  float* ks = S + static_cast<size_t>(m) * ld;  // [tile][d]
  float* vs = ks + kF32Tile * d;        // [tile][d]
  float* nk = vs + kF32Tile * d;        // [tile]
  const int split = blockIdx.x;
  const int bh = blockIdx.y;
  const int h = bh % H;
  const int j0 = split * span;
  const int j1 = min(n, j0 + span);
  const float* kb = k + static_cast<size_t>(bh) * n * d;
  const float* vb = v + static_cast<size_t>(bh) * n * d;
  const float* wb = W + static_cast<size_t>(h) * m * d;
  const int nf = (m + 255) / 256;  // features per thread (<= 2)
  float cmax[2] = {-INFINITY, -INFINITY};
  float zf[2] = {0.f, 0.f};
  for (int idx = threadIdx.x; idx < m * ld; idx += 256) S[idx] = 0.f;
  for (int pass = 0; pass < 2; ++pass) {
    for (int jt = j0; jt < j1; jt += kF32Tile) {
      const int cnt = min(kF32Tile, j1 - jt);
      __syncthreads();
      for (int idx = threadIdx.x; idx < cnt * d; idx += 256) {
        ks[idx] = kb[static_cast<size_t>(jt) * d + idx];
        vs[idx] = vb[static_cast<size_t>(jt) * d + idx];
      }
      __syncthreads();
      if (threadIdx.x < cnt) {
        float s = 0.f;
        for (int c = 0; c < d; ++c) s = fmaf(ks[threadIdx.x * d + c], ks[threadIdx.x * d + c], s);
        nk[threadIdx.x] = 0.5f * s;
      }
      __syncthreads();
      for (int a = 0; a < nf; ++a) {
        const int f = threadIdx.x + 256 * a;
        if (f >= m) break;
        const float* wf = wb + static_cast<size_t>(f) * d;
        for (int j = 0; j < cnt; ++j) {
          float e = 0.f;
          for (int c = 0; c < d; ++c) e = fmaf(wf[c], ks[j * d + c], e);
          e -= nk[j];
          if (pass == 0) {
            cmax[a] = fmaxf(cmax[a], e);
          } else {
            const float p = expf(e - cmax[a]);
            zf[a] += p;
            float* Sf = S + static_cast<size_t>(f) * ld;
            for (int c = 0; c < d; ++c) Sf[c] = fmaf(p, vs[j * d + c], Sf[c]);
          }
        }
      }
    }
  }
  __syncthreads();
  const size_t base = (static_cast<size_t>(bh) * kF32Splits + split) * m;
  for (int a = 0; a < nf; ++a) {
    const int f = threadIdx.x + 256 * a;
    if (f >= m) break;
    ws.c[base + f] = cmax[a];
    ws.z[base + f] = zf[a];
    for (int c = 0; c < d; ++c) ws.S[(base + f) * d + c] = S[static_cast<size_t>(f) * ld + c];
  }
}

__global__ __launch_bounds__(256) void k_merge_f32(F32Ws ws, int d, int m) {
  const int bh = blockIdx.x;
  for (int f = threadIdx.x; f < m; f += 256) {
    float cm = -INFINITY;
    for (int s = 0; s < kF32Splits; ++s)
      cm = fmaxf(cm, ws.c[(static_cast<size_t>(bh) * kF32Splits + s) * m + f]);
    float z = 0.f;
    float scale[kF32Splits];
    for (int s = 0; s < kF32Splits; ++s) {
      const size_t i = (static_cast<size_t>(bh) * kF32Splits + s) * m + f;
      const float cs = ws.c[i];
      scale[s] = (cs == -INFINITY) ? 0.f : expf(cs - cm);
      z = fmaf(scale[s], ws.z[i], z);
    }
    const float invz = 1.0f / z;
    for (int c = 0; c < d; ++c) {
      float acc = 0.f;
      for (int s = 0; s < kF32Splits; ++s)
        acc = fmaf(scale[s], ws.S[((static_cast<size_t>(bh) * kF32Splits + s) * m + f) * d + c], acc);
      ws.yhat[(static_cast<size_t>(bh) * m + f) * d + c] = acc * invz;
    }
    ws.beta[static_cast<size_t>(bh) * m + f] = cm + logf(z);
  }
}

// 64 queries per block; thread (query r = tid/4, part p = tid%4).
__global__ __launch_bounds__(256) void k_output_f32(const float* __restrict__ q,
                                                    const float* __restrict__ W, F32Ws ws,
                                                    float* __restrict__ out, int H, int n, int d,
                                                    int m) {
  extern __shared__ float sm[];
  const int ld = d + 1;
  float* qs = sm;                   // [64][d+1]
  float* wbuf = qs + 64 * ld;       // [64][65] weights of the current feature chunk
  float* ych = wbuf + 64 * 65;      // [64][d]  yhat rows of the chunk
  const int bh = blockIdx.y;
  const int h = bh % H;
  const int i0 = blockIdx.x * 64;
  const float* qb = q + static_cast<size_t>(bh) * n * d;
  const float* wb = W + static_cast<size_t>(h) * m * d;
  const float* yb = ws.yhat + static_cast<size_t>(bh) * m * d;
  const float* bb = ws.beta + static_cast<size_t>(bh) * m;
  for (int idx = threadIdx.x; idx < 64 * d; idx += 256) {
    const int r = idx / d, c = idx - r * d;
    qs[r * ld + c] = (i0 + r < n) ? qb[static_cast<size_t>(i0 + r) * d + c] : 0.f;
  }
  __syncthreads();
  const int r = threadIdx.x >> 2;
  const int p = threadIdx.x & 3;
  const float* qr = qs + r * ld;
  // row maximum of w_f.q + beta_f
  float M = -INFINITY;
  for (int f = p; f < m; f += 4) {
    const float* wf = wb + static_cast<size_t>(f) * d;
    float a = bb[f];
    for (int c = 0; c < d; ++c) a = fmaf(wf[c], qr[c], a);
    M = fmaxf(M, a);
  }
  M = fmaxf(M, __shfl_xor(M, 1));
  M = fmaxf(M, __shfl_xor(M, 2));
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;
  float den = 0.f;
  const int ncol = (d + 3 - p) / 4;  // columns c = p + 4 i
  for (int f0 = 0; f0 < m; f0 += 64) {
    const int cnt = min(64, m - f0);
    __syncthreads();
    for (int ff = p; ff < cnt; ff += 4) {
      const int f = f0 + ff;
      const float* wf = wb + static_cast<size_t>(f) * d;
      float a = bb[f];
      for (int c = 0; c < d; ++c) a = fmaf(wf[c], qr[c], a);
      wbuf[r * 65 + ff] = expf(a - M);
    }
    for (int idx = threadIdx.x; idx < cnt * d; idx += 256) ych[idx] = yb[static_cast<size_t>(f0) * d + idx];
    __syncthreads();
    for (int ff = 0; ff < cnt; ++ff) {
      const float u = wbuf[r * 65 + ff];
      den += u;
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if (i < ncol) acc[i] = fmaf(u, ych[ff * d + p + 4 * i], acc[i]);
    }
  }
  if (i0 + r < n) {
    const float inv = 1.0f / den;
    float* o = out + (static_cast<size_t>(bh) * n + i0 + r) * d;
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (i < ncol) o[p + 4 * i] = acc[i] * inv;
  }
}

// ---------------------------------------------------------------------------
// fp32 causal attention: one block per (b, h) walks the tokens in order,
// keeping the running per-feature state (c_f, z_f, S_f) in LDS.  For token j:
//   e_f = w_f.k_j - |k_j|^2/2;  if e_f > c_f, rescale (S_f, z_f) to c_f = e_f;
//   z_f += exp(e_f - c_f);  S_f += exp(e_f - c_f) v_j;
//   y_j = sum_f softmax_f(w_f.q_j + c_f + log z_f) * (S_f / z_f).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_max(float x, float* red) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ __launch_bounds__(256) void k_causal_f32(const float* __restrict__ q,
                                                    const float* __restrict__ k,
                                                    const float* __restrict__ v,
                                                    const float* __restrict__ W,
                                                    float* __restrict__ out, int H, int n, int d,
                                                    int m) {
  extern __shared__ float sm[];
  const int ld = d + 1;
  float* S = sm;                                  // [m][d+1]
  float* zc = S + static_cast<size_t>(m) * ld;    // [m] running z_f
  float* u = zc + m;                              // [m] weights for the current query
  float* row = u + m;                             // [3][d] q_j, k_j, v_j
  float* num = row + 3 * d;                       // [d+1] numerator, denominator
  float* red = num + d + 1;                       // [4] block reduction
  const int bh = blockIdx.x;
  const int h = bh % H;
  const float* qb = q + static_cast<size_t>(bh) * n * d;
  const float* kb = k + static_cast<size_t>(bh) * n * d;
  const float* vb = v + static_cast<size_t>(bh) * n * d;
  const float* wb = W + static_cast<size_t>(h) * m * d;
  const int nf = (m + 255) / 256;
  float cf[2] = {-INFINITY, -INFINITY};
  for (int idx = threadIdx.x; idx < m * ld; idx += 256) S[idx] = 0.f;
  for (int f = threadIdx.x; f < m; f += 256) zc[f] = 0.f;
  for (int j = 0; j < n; ++j) {
    __syncthreads();
    for (int c = threadIdx.x; c < d; c += 256) {
      row[c] = qb[static_cast<size_t>(j) * d + c];
      row[d + c] = kb[static_cast<size_t>(j) * d + c];
      row[2 * d + c] = vb[static_cast<size_t>(j) * d + c];
    }
    __syncthreads();
    float nk = 0.f;
    for (int c = 0; c < d; ++c) nk = fmaf(row[d + c], row[d + c], nk);
    nk *= 0.5f;
    float amax = -INFINITY;
    float a_own[2];
    for (int t = 0; t < nf; ++t) {
      const int f = threadIdx.x + 256 * t;
      a_own[t] = -INFINITY;
      if (f >= m) break;
      const float* wf = wb + static_cast<size_t>(f) * d;
      float e = 0.f, a = 0.f;
      for (int c = 0; c < d; ++c) {
        e = fmaf(wf[c], row[d + c], e);
        a = fmaf(wf[c], row[c], a);
      }
      e -= nk;
      float* Sf = S + static_cast<size_t>(f) * ld;
      if (e > cf[t]) {
        const float sc = (cf[t] == -INFINITY) ? 0.f : expf(cf[t] - e);
        zc[f] *= sc;
        for (int c = 0; c < d; ++c) Sf[c] *= sc;
        cf[t] = e;
      }
      const float p = expf(e - cf[t]);
      zc[f] += p;
      for (int c = 0; c < d; ++c) Sf[c] = fmaf(p, row[2 * d + c], Sf[c]);
      a += cf[t];
      a_own[t] = a;
      amax = fmaxf(amax, a + logf(zc[f]));
    }
    const float M = block_max(amax, red);
    for (int t = 0; t < nf; ++t) {
      const int f = threadIdx.x + 256 * t;
      if (f >= m) break;
      u[f] = expf(a_own[t] - M);
    }
    __syncthreads();
    for (int c = threadIdx.x; c <= d; c += 256) {
      float acc = 0.f;
      if (c < d) {
        for (int f = 0; f < m; ++f) acc = fmaf(u[f], S[static_cast<size_t>(f) * ld + c], acc);
      } else {
        for (int f = 0; f < m; ++f) acc = fmaf(u[f], zc[f], acc);
      }
      num[c] = acc;  // num[d] holds the denominator
    }
    __syncthreads();
    for (int c = threadIdx.x; c < d; c += 256)
      out[(static_cast<size_t>(bh) * n + j) * d + c] = num[c] / num[d];
  }
}

}  // namespace

hipError_t launch_feature_map_f32(const float* x, const float* W, float* phi, int B, int H, int n,
                                  int d, int m, hipStream_t s) {
  return launch_fm<float>(x, W, phi, B, H, n, d, m, s);
}
hipError_t launch_feature_map_bf16(const uint16_t* x, const uint16_t* W, float* phi, int B, int H,
                                   int n, int d, int m, hipStream_t s) {
  return launch_fm<uint16_t>(x, W, phi, B, H, n, d, m, s);
}

size_t f32_workspace_bytes(int B, int H, int n, int d, int m) {
  (void)n;
  const size_t BH = static_cast<size_t>(B) * H;
  size_t o = 0;
  o = align256(o + sizeof(float) * BH * kF32Splits * m);
  o = align256(o + sizeof(float) * BH * kF32Splits * m);
  o = align256(o + sizeof(float) * BH * kF32Splits * m * d);
  o = align256(o + sizeof(float) * BH * m * d);
  o = align256(o + sizeof(float) * BH * m);
  return o;
}

static hipError_t set_lds(const void* fn, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

hipError_t launch_attention_f32(const float* q, const float* k, const float* v, const float* W,
                                float* out, int B, int H, int n, int d, int m, void* wsp,
                                hipStream_t s) {
  const int BH = B * H;
  F32Ws ws = carve_f32(wsp, BH, d, m);
  const int span = (n + kF32Splits - 1) / kF32Splits;
  const size_t ldsA = sizeof(float) * (static_cast<size_t>(m) * (d + 1) + 2 * kF32Tile * d + kF32Tile);
  hipError_t e = set_lds(reinterpret_cast<const void*>(&k_state_f32), ldsA);
  if (e != hipSuccess) return e;
  FAVOR_LAUNCH("k_state_f32", k_state_f32, dim3(kF32Splits, BH), dim3(256), ldsA, s, k, v, W, ws, H, n, d,
                     m, span);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  FAVOR_LAUNCH("k_merge_f32", k_merge_f32, dim3(BH), dim3(256), 0, s, ws, d, m);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t ldsC = sizeof(float) * (64 * (d + 1) + 64 * 65 + 64 * d);
  e = set_lds(reinterpret_cast<const void*>(&k_output_f32), ldsC);
  if (e != hipSuccess) return e;
  FAVOR_LAUNCH("k_output_f32", k_output_f32, dim3((n + 63) / 64, BH), dim3(256), ldsC, s, q, W, ws, out, H,
                     n, d, m);
  return hipGetLastError();
}

hipError_t launch_attention_causal_f32(const float* q, const float* k, const float* v,
                                       const float* W, float* out, int B, int H, int n, int d,
                                       int m, hipStream_t s) {
  const size_t lds = sizeof(float) * (static_cast<size_t>(m) * (d + 1) + 2 * m + 4 * d + 1 + 4);
  hipError_t e = set_lds(reinterpret_cast<const void*>(&k_causal_f32), lds);
  if (e != hipSuccess) return e;
  FAVOR_LAUNCH("k_causal_f32", k_causal_f32, dim3(B * H), dim3(256), lds, s, q, k, v, W, out, H, n, d, m);
  return hipGetLastError();
}

}  // namespace favor
