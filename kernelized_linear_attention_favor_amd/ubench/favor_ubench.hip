// Instruction-rate probes (include/favor_ubench.h): throughput of v_exp_f32
// and v_fma_f32 on the vector units, alone and interleaved.  Eight independent
// chains per thread keep the pipeline full, so the rate measured is issue
// throughput, not latency.
#include <hip/hip_runtime.h>

#include "../../include/favor_ubench.h"

namespace {

__global__ __launch_bounds__(1024) void k_exp2(float* __restrict__ out, int iters) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  float x[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] = 0.5f + 0.01f * c + 1e-7f * (g & 255);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = __builtin_amdgcn_exp2f(-x[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += x[c];
  out[g] = s;
}

__global__ __launch_bounds__(1024) void k_fma(float* __restrict__ out, int iters) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  float x[8];
  const float a = 0.999f, b = 1e-3f * (1 + (g & 7));
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] = 0.5f + 0.01f * c;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = fmaf(x[c], a, b);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += x[c];
  out[g] = s;
}

__global__ __launch_bounds__(1024) void k_mix(float* __restrict__ out, int iters) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  float x[8], y[8];
  const float a = 0.999f, b = 1e-3f * (1 + (g & 7));
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    x[c] = 0.5f + 0.01f * c;
    y[c] = 0.25f + 0.01f * c;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      x[c] = __builtin_amdgcn_exp2f(-x[c]);
      y[c] = fmaf(y[c], a, b);
      y[c] = fmaf(y[c], a, b);
      y[c] = fmaf(y[c], a, b);
      y[c] = fmaf(y[c], a, b);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += x[c] + y[c];
  out[g] = s;
}

int launch(void (*k)(float*, int), float* out, int blocks, int threads, int iters, hipStream_t s) {
  if (!out || blocks < 1 || threads < 64 || threads > 1024 || threads % 64 != 0 || iters < 1) return 1;
  hipLaunchKernelGGL(k, dim3(blocks), dim3(threads), 0, s, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // namespace

extern "C" {
int favor_ubench_exp2(float* out, int blocks, int threads, int iters, hipStream_t stream) {
  return launch(k_exp2, out, blocks, threads, iters, stream);
}
int favor_ubench_fma(float* out, int blocks, int threads, int iters, hipStream_t stream) {
  return launch(k_fma, out, blocks, threads, iters, stream);
}
int favor_ubench_mix(float* out, int blocks, int threads, int iters, hipStream_t stream) {
  return launch(k_mix, out, blocks, threads, iters, stream);
}
}
