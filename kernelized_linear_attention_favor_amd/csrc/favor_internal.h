// Internal declarations shared by the libfavor host layer and its HIP kernels.
// Nothing here is part of the public ABI (include/favor.h).
#pragma once

#include <atomic>

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace favor {

// Kernel timing hooks (no-ops unless favor_profile_enable() is active on the
// calling thread).  name must be a string literal.
void prof_begin(hipStream_t s, const char* name);
void prof_end(hipStream_t s);

// Kernel launch bracketed by the timing hooks.
#define FAVOR_LAUNCH(name, kernel, grid, block, lds, stream, ...)                 \
  do {                                                                        \
    ::favor::prof_begin(stream, name);                                        \
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);        \
    ::favor::prof_end(stream);                                                \
  } while (0)

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- fp32 path
// Launchers for the fp32 (SIMT) kernels.  All return hipGetLastError().
hipError_t launch_feature_map_f32(const float* x, const float* W, float* phi, int B, int H, int n,
                                  int d, int m, hipStream_t s);
hipError_t launch_feature_map_bf16(const uint16_t* x, const uint16_t* W, float* phi, int B, int H,
                                   int n, int d, int m, hipStream_t s);

// Non-causal fp32 attention.  Workspace layout is private to the launcher;
// f32_workspace_bytes gives its size.
size_t f32_workspace_bytes(int B, int H, int n, int d, int m);
hipError_t launch_attention_f32(const float* q, const float* k, const float* v, const float* W,
                                float* out, int B, int H, int n, int d, int m, void* ws,
                                hipStream_t s);
hipError_t launch_attention_causal_f32(const float* q, const float* k, const float* v,
                                       const float* W, float* out, int B, int H, int n, int d,
                                       int m, hipStream_t s);

// ---------------------------------------------------------------- bf16 path
// Shapes: d in {32, 64}; m a multiple of 16 up to 512 (features are handled in
// 32-feature tiles, m rounded up to ma = 32 ceil(m / 32), the tail masked);
// causal chunk in {16, 32, 64, 128}.
constexpr int kMaxFeatures = 512;
constexpr int kDefaultChunk = 64;
bool bf16_supported(int d, int m);
bool chunk_supported(int chunk);

// A group of feature slices of equal width launched together (the causal walk).
struct SliceGroup {
  int first_slice, nslices, nw, fbase;   // nw waves (32 features each) per slice
};

struct Bf16Plan {
  int B, H, n, d, m, ma;   // ma: m rounded up to a multiple of 32 (state rows per range)
  int causal, chunk;
  int splits;     // key ranges per (b,h): state splits (non-causal) or segments (causal)
  int span;       // tokens per split / segment (multiple of 64)
  int nslices;    // causal: feature slices (1 unless m exceeds one walk's width)
  int ngroups;    // causal: launch groups of slices (1 or 2)
  SliceGroup groups[2];
  // workspace carve-up (byte offsets)
  size_t off_part_S, off_part_zc, off_vmax, off_yhat, off_beta, off_sigma, off_pnum, off_pdl, off_end;
};
Bf16Plan bf16_plan(int B, int H, int n, int d, int m, int causal, int chunk = kDefaultChunk);
hipError_t launch_attention_bf16(const Bf16Plan& p, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const uint16_t* W, float* out, void* ws,
                                 hipStream_t s);
// The causal chunk walk specialised for d = 64, m in {64, 128, 256} and chunks
// of 64 (k_causal_chunks); other shapes take the general walk (walk::).
bool causal_chunks_shape(const Bf16Plan& p);
// Bounded wait of the causal chunk kernel's key-tile hand-over (polls before
// the waiting wave computes the tile itself).
constexpr int kHandoverSpinDefault = 4096;
extern std::atomic<int> g_handover_spin;

hipError_t launch_causal_chunks(const Bf16Plan& p, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const uint16_t* W, const float* part_S,
                                const float* part_zc, const float* vmax, float* out,
                                hipStream_t s);
// The state pass (k_kv_state) over the plan's key ranges for every feature:
// partial states for the merge, or, with yhat non-null (one key range per
// (b, h)), the merge's outputs yhat, beta and sigma directly.
hipError_t launch_kv_all(const Bf16Plan& p, const uint16_t* k, const uint16_t* v, const uint16_t* W, float* pS,
                         float* pzc, float* pvm, hipStream_t s, uint16_t* yhat = nullptr, float* beta = nullptr,
                         float* sigma = nullptr);

namespace walk {
struct Args;
hipError_t launch_walk_c16(const Args& a, int nw, int nsl, hipStream_t s);
hipError_t launch_walk_c32(const Args& a, int nw, int nsl, hipStream_t s);
hipError_t launch_walk_c64(const Args& a, int nw, int nsl, hipStream_t s);
hipError_t launch_walk_c128(const Args& a, int nw, int nsl, hipStream_t s);
hipError_t launch_causal(const Bf16Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* W, const float* part_S, const float* part_zc, const float* vmax,
                         float* out, float* pnum, float* pdl, hipStream_t s);
}  // namespace walk

// ---------------------------------------------------------------- decode
// State of the keys of a non-causal plan's ranges, merged (k_kv_state + k_state_merge).
hipError_t launch_state_bf16(const Bf16Plan& p, const uint16_t* k, const uint16_t* v,
                             const uint16_t* W, void* ws, float* state, hipStream_t s);
size_t state_floats(int B, int H, int d, int m);
hipError_t launch_state_reset(float* state, int B, int H, int d, int m, hipStream_t s);
hipError_t launch_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* W,
                         float* state, float* out, int B, int H, int T, int m, hipStream_t s);

// ------------------------------------------- deterministic feature maps
namespace lin {
struct LinPlan {
  int B, H, n, m;
  int kind;       // 1 = ReLU features of W, 2 = elu(x) + 1 (m = d)
  int causal;
  int splits;     // key ranges per (b,h): state splits (non-causal) or segments (causal)
  int span;       // tokens per split / segment (multiple of 64)
  size_t off_part_S, off_part_z, off_sop, off_z, off_end;
};
LinPlan lin_plan(int B, int H, int n, int m, int kind, int causal);
hipError_t launch_linear_bf16(const LinPlan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const uint16_t* W, float* out, void* ws, hipStream_t s);
}  // namespace lin

// --------------------------------------------------- random feature draws
namespace draw {
bool draw_supported(int d);
hipError_t launch_draw_features(uint64_t seed, uint64_t step, void* W, int out_f32, int H, int m, int d,
                                hipStream_t s);
}  // namespace draw

// ------------------------------------------------------------ backward pass
namespace bw {
struct BwPlan {
  int B, H, n, m, causal;
  int splits, span;   // key / query ranges per (b,h) (multiple of 64 tokens)
  size_t off_cpart, off_part, off_pvec, off_part2, off_pvec2, off_stiles, off_rtiles, off_z, off_rho, off_cfin,
      off_aux, off_end;
};
BwPlan bw_plan(int B, int H, int n, int m, int causal);
hipError_t launch_backward_bf16(const BwPlan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const uint16_t* W, const float* y, const float* dy, float* dq, float* dk, float* dv,
                                void* ws, hipStream_t s);
}  // namespace bw

}  // namespace favor
