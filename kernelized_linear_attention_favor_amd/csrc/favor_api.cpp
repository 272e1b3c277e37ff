// libfavor host layer: argument checks, dispatch, scratch, status codes.
// Every check runs before anything is queued on the stream, so a failing call
// launches nothing and writes nothing.
#include "../../include/favor.h"

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "favor_internal.h"

namespace favor {
namespace {
struct ProfRec {
  const char* name;
  hipEvent_t start, stop;
};
struct Profiler {
  bool on = false;
  bool failed = false;
  char only[64] = "";   // record only kernels of this name (empty: all)
  bool open = false;    // the last prof_begin recorded a start event
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) failed = true;
    return e;
  }
};
thread_local Profiler g_prof;
}  // namespace

void prof_begin(hipStream_t s, const char* name) {
  g_prof.open = false;
  if (!g_prof.on) return;
  if (g_prof.only[0] && strcmp(g_prof.only, name) != 0) return;
  g_prof.open = true;
  ProfRec r{name, g_prof.get(), g_prof.get()};
  if (r.start && hipEventRecord(r.start, s) != hipSuccess) g_prof.failed = true;
  g_prof.recs.push_back(r);
}

void prof_end(hipStream_t s) {
  if (!g_prof.on || !g_prof.open || g_prof.recs.empty()) return;
  g_prof.open = false;
  hipEvent_t e = g_prof.recs.back().stop;
  if (e && hipEventRecord(e, s) != hipSuccess) g_prof.failed = true;
}
}  // namespace favor

namespace {

thread_local char g_last_error[512] = "";

favor_status_t fail(favor_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

favor_status_t ok() {
  g_last_error[0] = '\0';
  return FAVOR_OK;
}

favor_status_t hip_fail(hipError_t e, const char* where) {
  return fail(FAVOR_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

favor_status_t check_sizes(int B, int H, int n, int d, int m) {
  if (B < 1 || H < 1 || n < 1 || d < 1 || m < 1)
    return fail(FAVOR_ERR_INVALID_ARGUMENT, "sizes must be >= 1 (B=%d H=%d n=%d d=%d m=%d)", B, H,
                n, d, m);
  const long long elems = static_cast<long long>(B) * H * n * (d > m ? d : m);
  if (elems > (1LL << 40))
    return fail(FAVOR_ERR_UNSUPPORTED, "problem too large (B*H*n*max(d,m) = %lld)", elems);
  return FAVOR_OK;
}

favor_status_t check_ptrs(const void* a, const void* b, const void* c, const void* d,
                          const void* e, size_t align) {
  const void* ps[5] = {a, b, c, d, e};
  const char* names[5] = {"q", "k", "v", "W", "out"};
  for (int i = 0; i < 5; ++i) {
    if (!ps[i]) return fail(FAVOR_ERR_INVALID_ARGUMENT, "%s is null", names[i]);
    if (!aligned(ps[i], align))
      return fail(FAVOR_ERR_UNSUPPORTED, "%s is not %zu-byte aligned", names[i], align);
  }
  return FAVOR_OK;
}

favor_status_t check_f32_limits(int d, int m) {
  if (d > 128 || m > 512 || static_cast<long long>(m) * d > 16384)
    return fail(FAVOR_ERR_UNSUPPORTED, "fp32 path needs d <= 128, m <= 512, m*d <= 16384 (d=%d m=%d)",
                d, m);
  return FAVOR_OK;
}

favor_status_t check_bf16(const void* q, const void* k, const void* v, const void* W, float* out,
                          int B, int H, int n, int d, int m) {
  favor_status_t st = check_sizes(B, H, n, d, m);
  if (st != FAVOR_OK) return st;
  if ((st = check_ptrs(q, k, v, W, out, 16)) != FAVOR_OK) return st;
  if (!favor::bf16_supported(d, m))
    return fail(FAVOR_ERR_UNSUPPORTED,
                "bf16 attention supports d in {32, 64} and m a multiple of 16 from 16 to 512 (d=%d m=%d)", d, m);
  return FAVOR_OK;
}

// The shapes of the decode, deterministic feature-map and backward kernels.
bool fixed_shape(int d, int m) { return d == 64 && (m == 64 || m == 128 || m == 256); }

favor_status_t check_fixed(const void* q, const void* k, const void* v, const void* W, float* out,
                           int B, int H, int n, int d, int m, const char* what) {
  favor_status_t st = check_sizes(B, H, n, d, m);
  if (st != FAVOR_OK) return st;
  if ((st = check_ptrs(q, k, v, W, out, 16)) != FAVOR_OK) return st;
  if (!fixed_shape(d, m))
    return fail(FAVOR_ERR_UNSUPPORTED, "%s supports d = 64 and m in {64, 128, 256} (d=%d m=%d)", what, d, m);
  return FAVOR_OK;
}

// Stream-ordered scratch: allocated and freed on the caller's stream.
struct StreamScratch {
  void* p = nullptr;
  hipStream_t s;
  explicit StreamScratch(hipStream_t st) : s(st) {}
  hipError_t alloc(size_t bytes) { return hipMallocAsync(&p, bytes, s); }
  ~StreamScratch() {
    if (p) (void)hipFreeAsync(p, s);
  }
};

favor_status_t run_bf16(const void* q, const void* k, const void* v, const void* W, float* out,
                        int B, int H, int n, int d, int m, int causal, void* ws, size_t ws_bytes,
                        hipStream_t stream, int chunk = favor::kDefaultChunk) {
  favor::Bf16Plan plan = favor::bf16_plan(B, H, n, d, m, causal, chunk);
  StreamScratch own(stream);
  if (!ws) {
    hipError_t e = own.alloc(plan.off_end);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(FAVOR_ERR_OUT_OF_MEMORY, "scratch allocation of %zu bytes failed: %s",
                  plan.off_end, hipGetErrorString(e));
    }
    e = hipMemsetAsync(own.p, 0, plan.off_end, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync(scratch)");
    ws = own.p;
  } else if (ws_bytes < plan.off_end) {
    return fail(FAVOR_ERR_OUT_OF_MEMORY, "workspace has %zu bytes, needs %zu", ws_bytes,
                plan.off_end);
  } else if (!aligned(ws, 256)) {
    return fail(FAVOR_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");
  }
  hipError_t e = favor::launch_attention_bf16(
      plan, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(W), out, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "bf16 attention launch");
  return ok();
}

favor_status_t check_state_shape(const float* state, int B, int H, int d, int m) {
  if (B < 1 || H < 1 || d < 1 || m < 1)
    return fail(FAVOR_ERR_INVALID_ARGUMENT, "sizes must be >= 1 (B=%d H=%d d=%d m=%d)", B, H, d, m);
  if (!state) return fail(FAVOR_ERR_INVALID_ARGUMENT, "state is null");
  if (!aligned(state, 16)) return fail(FAVOR_ERR_UNSUPPORTED, "state is not 16-byte aligned");
  if (!fixed_shape(d, m))
    return fail(FAVOR_ERR_UNSUPPORTED, "decode supports d = 64 and m in {64, 128, 256} (d=%d m=%d)",
                d, m);
  return FAVOR_OK;
}

favor_status_t check_phi(const void* q, const void* k, const void* v, const void* W, float* out,
                         int B, int H, int n, int d, int m, int causal, int phi) {
  if (causal != 0 && causal != 1)
    return fail(FAVOR_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
  if (phi != FAVOR_PHI_RELU && phi != FAVOR_PHI_ELU1)
    return fail(FAVOR_ERR_INVALID_ARGUMENT, "unknown feature map %d", phi);
  favor_status_t st = check_sizes(B, H, n, d, m);
  if (st != FAVOR_OK) return st;
  const void* Wc = phi == FAVOR_PHI_ELU1 ? q : W;   // elu(x) + 1 takes no W
  if ((st = check_ptrs(q, k, v, Wc, out, 16)) != FAVOR_OK) return st;
  if (phi == FAVOR_PHI_ELU1 && (d != 64 || m != d))
    return fail(FAVOR_ERR_UNSUPPORTED, "elu(x)+1 features need d = m = 64 (d=%d m=%d)", d, m);
  if (phi == FAVOR_PHI_RELU && !fixed_shape(d, m))
    return fail(FAVOR_ERR_UNSUPPORTED, "ReLU features support d = 64 and m in {64, 128, 256} (d=%d m=%d)",
                d, m);
  return FAVOR_OK;
}

// Fixed scratch for favor_attention_noalloc: one array per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory; the device address of each GPU's copy comes from hipGetSymbolAddress
// (taken once per device, with that device current) and only that address is
// ever handed to kernels.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's scratch array (nullptr on failure, with
// the HIP error in *err).
void* scratch_for_current_device(hipError_t* err, int* dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  *dev_out = dev;
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  ScratchSlot& sl = g_scratch[dev];
  std::call_once(sl.once, [&sl] {
    void* p = nullptr;
    sl.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (sl.err == hipSuccess) sl.ptr = p;
  });
  *err = sl.err;
  return sl.err == hipSuccess ? sl.ptr : nullptr;
}

}  // namespace

extern "C" {

int favor_version(void) { return 10000; }

favor_status_t favor_profile_enable(void) { return favor_profile_enable_only(nullptr); }

favor_status_t favor_set_handover_spin_limit(int limit) {
  if (limit < 0) return fail(FAVOR_ERR_INVALID_ARGUMENT, "spin limit %d is negative", limit);
  favor::g_handover_spin.store(limit, std::memory_order_relaxed);
  return ok();
}

favor_status_t favor_profile_enable_only(const char* name) {
  auto& P = favor::g_prof;
  if (name && strlen(name) >= sizeof(P.only))
    return fail(FAVOR_ERR_INVALID_ARGUMENT, "kernel name longer than %zu characters", sizeof(P.only) - 1);
  P.only[0] = '\0';
  if (name) strcpy(P.only, name);
  P.on = true;
  return ok();
}

int favor_profile_collect(const char** names, int* counts, double* total_ms, int capacity) {
  auto& P = favor::g_prof;
  std::vector<const char*> uniq;
  std::vector<int> cnt;
  std::vector<double> tot;
  bool failed = P.failed;
  for (auto& r : P.recs) {
    float ms = 0.f;
    if (!r.start || !r.stop || hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      failed = true;
    }
    size_t i = 0;
    while (i < uniq.size() && strcmp(uniq[i], r.name) != 0) ++i;
    if (i == uniq.size()) {
      uniq.push_back(r.name);
      cnt.push_back(0);
      tot.push_back(0.0);
    }
    cnt[i] += 1;
    tot[i] += ms;
    if (r.start) P.pool.push_back(r.start);
    if (r.stop) P.pool.push_back(r.stop);
  }
  P.recs.clear();
  P.on = false;
  P.open = false;
  P.only[0] = '\0';
  P.failed = false;
  for (size_t i = 0; i < uniq.size() && static_cast<int>(i) < capacity; ++i) {
    if (names) names[i] = uniq[i];
    if (counts) counts[i] = cnt[i];
    if (total_ms) total_ms[i] = tot[i];
  }
  if (failed) return -1;
  return static_cast<int>(uniq.size());
}

const char* favor_status_string(favor_status_t s) {
  switch (s) {
    case FAVOR_OK: return "FAVOR_OK";
    case FAVOR_ERR_INVALID_ARGUMENT: return "FAVOR_ERR_INVALID_ARGUMENT";
    case FAVOR_ERR_UNSUPPORTED: return "FAVOR_ERR_UNSUPPORTED";
    case FAVOR_ERR_HIP: return "FAVOR_ERR_HIP";
    case FAVOR_ERR_OUT_OF_MEMORY: return "FAVOR_ERR_OUT_OF_MEMORY";
  }
  return "FAVOR_ERR_UNKNOWN";
}

const char* favor_last_error(void) { return g_last_error; }

favor_status_t favor_feature_map(const void* x, const void* W, float* phi, int B, int H, int n,
                                 int d, int m, hipStream_t stream) {
  favor_status_t st = check_sizes(B, H, n, d, m);
  if (st != FAVOR_OK) return st;
  if (!x || !W || !phi) return fail(FAVOR_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned(x, 4) || !aligned(W, 4) || !aligned(phi, 4))
    return fail(FAVOR_ERR_UNSUPPORTED, "pointers must be 4-byte aligned");
  if (d > 256 || m > 1024) return fail(FAVOR_ERR_UNSUPPORTED, "feature map needs d <= 256, m <= 1024");
  hipError_t e = favor::launch_feature_map_bf16(static_cast<const uint16_t*>(x),
                                                static_cast<const uint16_t*>(W), phi, B, H, n, d,
                                                m, stream);
  if (e != hipSuccess) return hip_fail(e, "feature map launch");
  return ok();
}

favor_status_t favor_feature_map_f32(const float* x, const float* W, float* phi, int B, int H,
                                     int n, int d, int m, hipStream_t stream) {
  favor_status_t st = check_sizes(B, H, n, d, m);
  if (st != FAVOR_OK) return st;
  if (!x || !W || !phi) return fail(FAVOR_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned(x, 4) || !aligned(W, 4) || !aligned(phi, 4))
    return fail(FAVOR_ERR_UNSUPPORTED, "pointers must be 4-byte aligned");
  if (d > 256 || m > 1024) return fail(FAVOR_ERR_UNSUPPORTED, "feature map needs d <= 256, m <= 1024");
  hipError_t e = favor::launch_feature_map_f32(x, W, phi, B, H, n, d, m, stream);
  if (e != hipSuccess) return hip_fail(e, "feature map launch");
  return ok();
}

favor_status_t favor_attention(const void* q, const void* k, const void* v, const void* W,
                               float* out, int B, int H, int n, int d, int m, int causal,
                               hipStream_t stream) {
  if (causal != 0 && causal != 1)
    return fail(FAVOR_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
  favor_status_t st = check_bf16(q, k, v, W, out, B, H, n, d, m);
  if (st != FAVOR_OK) return st;
  return run_bf16(q, k, v, W, out, B, H, n, d, m, causal, nullptr, 0, stream);
}

favor_status_t favor_attention_causal(const void* q, const void* k, const void* v, const void* W,
                                      float* out, int B, int H, int n, int d, int m, int chunk,
                                      hipStream_t stream) {
  if (chunk != 0 && !favor::chunk_supported(chunk))
    return fail(chunk < 0 ? FAVOR_ERR_INVALID_ARGUMENT : FAVOR_ERR_UNSUPPORTED,
                "chunk must be 0 (default, %d) or one of 16, 32, 64, 128 (got %d)", favor::kDefaultChunk, chunk);
  favor_status_t st = check_bf16(q, k, v, W, out, B, H, n, d, m);
  if (st != FAVOR_OK) return st;
  return run_bf16(q, k, v, W, out, B, H, n, d, m, 1, nullptr, 0, stream, chunk == 0 ? favor::kDefaultChunk : chunk);
}

size_t favor_workspace_bytes(int B, int H, int n, int d, int m, int causal) {
  if (B < 1 || H < 1 || n < 1 || !favor::bf16_supported(d, m) || (causal != 0 && causal != 1))
    return 0;
  return favor::bf16_plan(B, H, n, d, m, causal).off_end;
}

favor_status_t favor_attention_ws(const void* q, const void* k, const void* v, const void* W,
                                  float* out, int B, int H, int n, int d, int m, int causal,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  if (causal != 0 && causal != 1)
    return fail(FAVOR_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
  favor_status_t st = check_bf16(q, k, v, W, out, B, H, n, d, m);
  if (st != FAVOR_OK) return st;
  if (!ws) return fail(FAVOR_ERR_INVALID_ARGUMENT, "ws is null");
  return run_bf16(q, k, v, W, out, B, H, n, d, m, causal, ws, ws_bytes, stream);
}

favor_status_t favor_attention_noalloc(const void* q, const void* k, const void* v, const void* W, float* out,
                                       int B, int H, int n, int d, int m, int causal, hipStream_t stream) {
  if (causal != 0 && causal != 1)
    return fail(FAVOR_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
  favor_status_t st = check_bf16(q, k, v, W, out, B, H, n, d, m);
  if (st != FAVOR_OK) return st;
  const favor::Bf16Plan plan = favor::bf16_plan(B, H, n, d, m, causal);
  if (plan.off_end > kNoAllocScratchBytes)
    return fail(FAVOR_ERR_UNSUPPORTED,
                "favor_attention_noalloc: this shape needs %zu bytes of scratch, above the fixed %zu-byte "
                "array (use favor_attention_ws with a caller-owned workspace)",
                plan.off_end, kNoAllocScratchBytes);
  hipError_t e = hipSuccess;
  int dev = -1;
  void* ws = scratch_for_current_device(&e, &dev);
  if (!ws) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  e = favor::launch_attention_bf16(plan, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                   static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(W), out, ws,
                                   stream);
  if (e != hipSuccess) return hip_fail(e, "bf16 attention launch");
  return ok();
}

size_t favor_state_bytes(int B, int H, int d, int m) {
  if (B < 1 || H < 1 || !fixed_shape(d, m)) return 0;
  return sizeof(float) * favor::state_floats(B, H, d, m);
}


favor_status_t favor_state_reset(float* state, int B, int H, int d, int m, hipStream_t stream) {
  favor_status_t st = check_state_shape(state, B, H, d, m);
  if (st != FAVOR_OK) return st;
  hipError_t e = favor::launch_state_reset(state, B, H, d, m, stream);
  if (e != hipSuccess) return hip_fail(e, "state reset launch");
  return ok();
}

favor_status_t favor_state_from_keys(const void* k, const void* v, const void* W, float* state,
                                     int B, int H, int n, int d, int m, hipStream_t stream) {
  favor_status_t st = check_state_shape(state, B, H, d, m);
  if (st != FAVOR_OK) return st;
  if ((st = check_sizes(B, H, n, d, m)) != FAVOR_OK) return st;
  const void* ps[3] = {k, v, W};
  const char* names[3] = {"k", "v", "W"};
  for (int i = 0; i < 3; ++i) {
    if (!ps[i]) return fail(FAVOR_ERR_INVALID_ARGUMENT, "%s is null", names[i]);
    if (!aligned(ps[i], 16)) return fail(FAVOR_ERR_UNSUPPORTED, "%s is not 16-byte aligned", names[i]);
  }
  const favor::Bf16Plan plan = favor::bf16_plan(B, H, n, d, m, 0);
  StreamScratch own(stream);
  hipError_t e = own.alloc(plan.off_end);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(FAVOR_ERR_OUT_OF_MEMORY, "scratch allocation of %zu bytes failed: %s", plan.off_end,
                hipGetErrorString(e));
  }
  e = favor::launch_state_bf16(plan, static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                               static_cast<const uint16_t*>(W), own.p, state, stream);
  if (e != hipSuccess) return hip_fail(e, "state launch");
  return ok();
}

favor_status_t favor_decode(const void* q, const void* k, const void* v, const void* W,
                            float* state, float* out, int B, int H, int T, int d, int m,
                            hipStream_t stream) {
  favor_status_t st = check_state_shape(state, B, H, d, m);
  if (st != FAVOR_OK) return st;
  if ((st = check_sizes(B, H, T, d, m)) != FAVOR_OK) return st;
  if ((st = check_ptrs(q, k, v, W, out, 16)) != FAVOR_OK) return st;
  hipError_t e = favor::launch_decode(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(W),
                                      state, out, B, H, T, m, stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

favor_status_t favor_attention_f32(const float* q, const float* k, const float* v, const float* W,
                                   float* out, int B, int H, int n, int d, int m, int causal,
                                   hipStream_t stream) {
  if (causal != 0 && causal != 1)
    return fail(FAVOR_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
  favor_status_t st = check_sizes(B, H, n, d, m);
  if (st != FAVOR_OK) return st;
  if ((st = check_ptrs(q, k, v, W, out, 4)) != FAVOR_OK) return st;
  if ((st = check_f32_limits(d, m)) != FAVOR_OK) return st;
  hipError_t e;
  if (causal) {
    e = favor::launch_attention_causal_f32(q, k, v, W, out, B, H, n, d, m, stream);
    if (e != hipSuccess) return hip_fail(e, "fp32 causal launch");
    return ok();
  }
  StreamScratch own(stream);
  const size_t bytes = favor::f32_workspace_bytes(B, H, n, d, m);
  e = own.alloc(bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(FAVOR_ERR_OUT_OF_MEMORY, "scratch allocation of %zu bytes failed", bytes);
  }
  e = favor::launch_attention_f32(q, k, v, W, out, B, H, n, d, m, own.p, stream);
  if (e != hipSuccess) return hip_fail(e, "fp32 attention launch");
  return ok();
}

favor_status_t favor_attention_causal_f32(const float* q, const float* k, const float* v,
                                          const float* W, float* out, int B, int H, int n, int d,
                                          int m, int chunk, hipStream_t stream) {
  if (chunk < 0) return fail(FAVOR_ERR_INVALID_ARGUMENT, "chunk must be >= 0 (got %d)", chunk);
  return favor_attention_f32(q, k, v, W, out, B, H, n, d, m, 1, stream);
}

}  // extern "C"

extern "C" {

size_t favor_workspace_bytes_phi(int B, int H, int n, int d, int m, int causal, int phi) {
  if (phi == FAVOR_PHI_EXP) return favor_workspace_bytes(B, H, n, d, m, causal);
  if (B < 1 || H < 1 || n < 1 || d != 64 || (causal != 0 && causal != 1)) return 0;
  if (phi == FAVOR_PHI_ELU1 && m != d) return 0;
  if (phi == FAVOR_PHI_RELU && !fixed_shape(d, m)) return 0;
  if (phi != FAVOR_PHI_RELU && phi != FAVOR_PHI_ELU1) return 0;
  return favor::lin::lin_plan(B, H, n, m, phi, causal).off_end;
}

favor_status_t favor_attention_phi(const void* q, const void* k, const void* v, const void* W,
                                   float* out, int B, int H, int n, int d, int m, int causal, int phi,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  if (phi == FAVOR_PHI_EXP)
    return ws ? favor_attention_ws(q, k, v, W, out, B, H, n, d, m, causal, ws, ws_bytes, stream)
              : favor_attention(q, k, v, W, out, B, H, n, d, m, causal, stream);
  favor_status_t st = check_phi(q, k, v, W, out, B, H, n, d, m, causal, phi);
  if (st != FAVOR_OK) return st;
  const favor::lin::LinPlan plan = favor::lin::lin_plan(B, H, n, m, phi, causal);
  StreamScratch own(stream);
  if (!ws) {
    hipError_t e = own.alloc(plan.off_end);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(FAVOR_ERR_OUT_OF_MEMORY, "scratch allocation of %zu bytes failed: %s", plan.off_end,
                  hipGetErrorString(e));
    }
    ws = own.p;
  } else if (ws_bytes < plan.off_end) {
    return fail(FAVOR_ERR_OUT_OF_MEMORY, "workspace has %zu bytes, needs %zu", ws_bytes, plan.off_end);
  } else if (!aligned(ws, 256)) {
    return fail(FAVOR_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");
  }
  hipError_t e = favor::lin::launch_linear_bf16(plan, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                                static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(W),
                                                out, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "feature-map attention launch");
  return ok();
}

}  // extern "C"

extern "C" {

favor_status_t favor_draw_features(unsigned long long seed, unsigned long long step, void* W, int out_dtype,
                                   int H, int m, int d, hipStream_t stream) {
  if (H < 1 || m < 1 || d < 1)
    return fail(FAVOR_ERR_INVALID_ARGUMENT, "sizes must be >= 1 (H=%d m=%d d=%d)", H, m, d);
  if (!W) return fail(FAVOR_ERR_INVALID_ARGUMENT, "W is null");
  if (out_dtype != FAVOR_OUT_BF16 && out_dtype != FAVOR_OUT_F32)
    return fail(FAVOR_ERR_INVALID_ARGUMENT, "out_dtype must be FAVOR_OUT_BF16 or FAVOR_OUT_F32 (got %d)", out_dtype);
  if (!favor::draw::draw_supported(d)) return fail(FAVOR_ERR_UNSUPPORTED, "d must be 16, 32 or 64 (got %d)", d);
  if (!aligned(W, 4)) return fail(FAVOR_ERR_UNSUPPORTED, "W is not 4-byte aligned");
  if (static_cast<long long>(H) * ((m + d - 1) / d) > (1LL << 30))
    return fail(FAVOR_ERR_UNSUPPORTED, "too many blocks (H=%d m=%d)", H, m);
  hipError_t e = favor::draw::launch_draw_features(seed, step, W, out_dtype == FAVOR_OUT_F32, H, m, d, stream);
  if (e != hipSuccess) return hip_fail(e, "feature draw launch");
  return ok();
}

}  // extern "C"

extern "C" {

size_t favor_backward_workspace_bytes(int B, int H, int n, int d, int m, int causal) {
  if (B < 1 || H < 1 || n < 1 || (causal != 0 && causal != 1) || !fixed_shape(d, m)) return 0;
  return favor::bw::bw_plan(B, H, n, m, causal).off_end;
}

favor_status_t favor_attention_backward(const void* q, const void* k, const void* v, const void* W, const float* y,
                                        const float* dy, float* dq, float* dk, float* dv, int B, int H, int n, int d,
                                        int m, int causal, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (causal != 0 && causal != 1)
    return fail(FAVOR_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", causal);
  favor_status_t st = check_fixed(q, k, v, W, dq, B, H, n, d, m, "the backward pass");
  if (st != FAVOR_OK) return st;
  const void* more[5] = {y, dy, dk, dv, dq};
  const char* names[5] = {"y", "dy", "dk", "dv", "dq"};
  for (int i = 0; i < 5; ++i) {
    if (!more[i]) return fail(FAVOR_ERR_INVALID_ARGUMENT, "%s is null", names[i]);
    if (!aligned(more[i], 16)) return fail(FAVOR_ERR_UNSUPPORTED, "%s is not 16-byte aligned", names[i]);
  }
  const favor::bw::BwPlan plan = favor::bw::bw_plan(B, H, n, m, causal);
  StreamScratch own(stream);
  if (!ws) {
    hipError_t e = own.alloc(plan.off_end);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(FAVOR_ERR_OUT_OF_MEMORY, "scratch allocation of %zu bytes failed: %s", plan.off_end,
                  hipGetErrorString(e));
    }
    ws = own.p;
  } else if (ws_bytes < plan.off_end) {
    return fail(FAVOR_ERR_OUT_OF_MEMORY, "workspace has %zu bytes, needs %zu", ws_bytes, plan.off_end);
  } else if (!aligned(ws, 256)) {
    return fail(FAVOR_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");
  }
  hipError_t e = favor::bw::launch_backward_bf16(
      plan, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
      static_cast<const uint16_t*>(W), y, dy, dq, dk, dv, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return ok();
}

}  // extern "C"
