/*
 * libfavor -- FAVOR+ (Performer) linear attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every entry point takes plain device pointers, sizes and a HIP stream.
 *
 * The operation (Performer notes: sections Kernel Attention View, Normalization
 * and FAVOR+; lesson "Linear Attention and the Performer": Code; Performer for
 * vision: How It Works, Steps 1 and 2):
 *
 *   phi(x)  = exp(W x - |x|^2 / 2) / sqrt(m)          positive random features
 *   S       = Phi(K)^T V,   z = Phi(K)^T 1             key/value summary
 *   y_i     = phi(q_i)^T S / phi(q_i)^T z              non-causal output
 *   y_i     = phi(q_i)^T S_i / phi(q_i)^T z_i,         causal output, with
 *             S_i, z_i summing keys j <= i only        (prefix sums, inclusive)
 *
 * The library applies no 1/sqrt(d) temperature: the caller folds it into q and
 * k.  The same W serves queries and keys.  d_v = d.
 *
 * Layouts (all row-major, innermost last, no padding):
 *   q, k, v, x, out : [B, H, n, d]
 *   W               : [H, m, d]   one feature matrix per head, shared by the batch
 *   phi             : [B, H, n, m]
 * bf16 entry points take q, k, v, x, W as bfloat16 bit patterns (uint16) and
 * write float32 results; the _f32 twins take float32 inputs.
 *
 * Ownership: the caller allocates every input, output and workspace and keeps
 * them alive until the work queued on `stream` has finished.  The library
 * never frees caller memory.  The self-allocating entries take scratch from
 * hipMallocAsync/hipFreeAsync on `stream`.  stream may be 0 (null stream).
 *
 * Errors: arguments are checked before anything is queued; on error nothing is
 * launched and no output is written.  Launch failures return FAVOR_ERR_HIP.
 * Kernels run asynchronously: device faults surface at the caller's next
 * synchronisation.  NaN/Inf inputs are not checked and propagate.
 * favor_last_error() returns a thread-local description of the last failure.
 *
 * Determinism: for a fixed shape, device and library build, results are
 * bitwise reproducible (all cross-workgroup reductions run in a fixed order;
 * no floating-point atomics).
 */
#ifndef FAVOR_H_
#define FAVOR_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FAVOR_OK = 0,
  FAVOR_ERR_INVALID_ARGUMENT = 1, /* null pointer, non-positive size, bad flag */
  FAVOR_ERR_UNSUPPORTED = 2,      /* valid but outside what the library implements */
  FAVOR_ERR_HIP = 3,              /* a HIP call or kernel launch failed */
  FAVOR_ERR_OUT_OF_MEMORY = 4     /* scratch allocation failed, or workspace too small */
} favor_status_t;

/* Version as major*10000 + minor*100 + patch. */
int favor_version(void);
const char* favor_status_string(favor_status_t s);
/* Thread-local text for the last failing call on this thread ("" if none). */
const char* favor_last_error(void);

/*
 * favor_feature_map -- the positive random-feature map itself (Performer
 * notes, FAVOR+: phi in R^m whose inner products estimate exp(q.k)):
 *   phi[b,h,i,:] = exp(W[h] x[b,h,i,:] - |x[b,h,i,:]|^2 / 2) / sqrt(m), fp32.
 * Exact (no stabilising shift), so very large |x| can overflow or underflow
 * fp32 exactly as the formula does.
 *   x   : bf16 [B,H,n,d]         W : bf16 [H,m,d]        phi : fp32 [B,H,n,m]
 * Supported: 1 <= d <= 256, 1 <= m <= 1024.  Pointers 4-byte aligned.
 */
favor_status_t favor_feature_map(const void* x, const void* W, float* phi,
                                 int B, int H, int n, int d, int m, hipStream_t stream);
favor_status_t favor_feature_map_f32(const float* x, const float* W, float* phi,
                                     int B, int H, int n, int d, int m, hipStream_t stream);

/*
 * favor_attention -- FAVOR+ attention, y = Phi(Q) S / (Phi(Q) z) (Performer
 * notes, Normalization).  causal = 0: every query sees every key.  causal = 1:
 * query i sees keys j <= i (Performer for vision, Step 2); identical to
 * favor_attention_causal with chunk = 0.
 *   q, k, v : bf16 [B,H,n,d]     W : bf16 [H,m,d]        out : fp32 [B,H,n,d]
 * bf16 path: d in {32, 64}; m any multiple of 16 from 16 to 512 (m is the
 * estimator's accuracy knob, Performer notes, FAVOR+); pointers 16-byte
 * aligned; otherwise FAVOR_ERR_UNSUPPORTED.  The causal form uses chunks of 64
 * tokens.  Scratch is allocated stream-ordered on `stream` (see
 * favor_attention_ws to supply it).
 */
favor_status_t favor_attention(const void* q, const void* k, const void* v, const void* W,
                               float* out, int B, int H, int n, int d, int m, int causal,
                               hipStream_t stream);

/*
 * favor_attention_causal -- causal FAVOR+ by chunked prefix sums (Performer for
 * vision, How It Works, Step 2): the sequence is cut into chunks of `chunk`
 * tokens; each chunk combines the running key/value state of all earlier
 * chunks with the masked pairwise weights inside the chunk.  chunk == 0 picks
 * the default (64).  Supported chunk: 16, 32, 64, 128 (any other positive
 * value: FAVOR_ERR_UNSUPPORTED; negative: FAVOR_ERR_INVALID_ARGUMENT).  Every
 * chunk length gives the same sums up to rounding; it sets how many keys join
 * the running state at once and how large the masked pairwise block is.  Same
 * shapes and limits as favor_attention.
 */
favor_status_t favor_attention_causal(const void* q, const void* k, const void* v,
                                      const void* W, float* out, int B, int H, int n, int d,
                                      int m, int chunk, hipStream_t stream);

/*
 * fp32 twins: identical semantics with float32 q, k, v, W.  Arithmetic in fp32
 * throughout.  Limits: 1 <= d <= 128, 1 <= m <= 512, m*d <= 16384; pointers
 * 4-byte aligned.  The causal fp32 entry walks tokens one by one per (b,h); it
 * is meant for checking, not speed.
 */
favor_status_t favor_attention_f32(const float* q, const float* k, const float* v,
                                   const float* W, float* out, int B, int H, int n, int d,
                                   int m, int causal, hipStream_t stream);
favor_status_t favor_attention_causal_f32(const float* q, const float* k, const float* v,
                                          const float* W, float* out, int B, int H, int n,
                                          int d, int m, int chunk, hipStream_t stream);

/*
 * Caller-owned scratch for the bf16 attention path.  favor_workspace_bytes
 * returns the size favor_attention_ws needs for a shape (0 if the shape is not
 * supported; causal = 1 sizes the default chunk of 64).  The workspace needs
 * no initialisation: every call writes each scratch word before reading it.
 * Two calls that share one workspace must not overlap in time (same stream is
 * fine).
 */
size_t favor_workspace_bytes(int B, int H, int n, int d, int m, int causal);
favor_status_t favor_attention_ws(const void* q, const void* k, const void* v, const void* W,
                                  float* out, int B, int H, int n, int d, int m, int causal,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * favor_attention_noalloc -- favor_attention (same arguments, same kernels,
 * bitwise the same output) for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It calls no allocator.  Its scratch is one fixed array of 64 MiB
 * (67108864 bytes) per GPU, a static device array of the library that each GPU
 * it runs on holds until the process ends; a shape whose scratch
 * (favor_workspace_bytes) exceeds it returns FAVOR_ERR_UNSUPPORTED and launches
 * nothing.  No part of the array needs to start at zero (every call writes each
 * scratch word before reading it).  All calls on one GPU share that GPU's array:
 * calls that overlap in time on one GPU (different streams, or threads without
 * ordering) race and give undefined results; calls ordered on one stream are
 * safe.
 */
favor_status_t favor_attention_noalloc(const void* q, const void* k, const void* v, const void* W,
                                       float* out, int B, int H, int n, int d, int m, int causal,
                                       hipStream_t stream);

/*
 * Deterministic feature maps on the same state / output / causal structure
 * (Performer for vision, What Is Performer? and Kernel Choices: ReLU features of
 * the random projections; quiz page on linear attention variants, comparison
 * table: the Linear Transformer's elu(x)+1):
 *   FAVOR_PHI_EXP   phi(x) = exp(W x - |x|^2/2) / sqrt(m)   (favor_attention)
 *   FAVOR_PHI_RELU  phi(x) = max(W x, 0) / sqrt(m), W [H,m,d] bf16, m in {64,128,256}
 *   FAVOR_PHI_ELU1  phi(x) = elu(x) + 1 on x itself: m must equal d; W is not read
 *                   (may be NULL)
 * y_i = phi(q_i)^T S / phi(q_i)^T z, non-causal or causal (j <= i) as for
 * favor_attention; a query whose features are all zero (possible only with
 * ReLU) gets y_i = 0.  bf16 q, k, v [B,H,n,d] with d = 64, fp32 out.
 *
 * favor_workspace_bytes_phi -- scratch bytes favor_attention_phi needs for a
 *   shape (0 if unsupported).
 * favor_attention_phi -- ws / ws_bytes as for favor_attention_ws, or ws = NULL
 *   for scratch allocated stream-ordered on `stream`.  An unknown phi is
 *   FAVOR_ERR_INVALID_ARGUMENT; FAVOR_PHI_EXP forwards to favor_attention(_ws).
 */
typedef enum { FAVOR_PHI_EXP = 0, FAVOR_PHI_RELU = 1, FAVOR_PHI_ELU1 = 2 } favor_phi_t;
size_t favor_workspace_bytes_phi(int B, int H, int n, int d, int m, int causal, int phi);
favor_status_t favor_attention_phi(const void* q, const void* k, const void* v, const void* W,
                                   float* out, int B, int H, int n, int d, int m, int causal, int phi,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Orthogonal random features drawn on the device (Performer for vision, Kernel
 * Choices: orthogonal features by QR of random projection matrices; Performer
 * notes, FAVOR+).  Writes W [H, m, d] (bf16 or fp32, row-major) for the key
 * (seed, step): a new step gives an independent draw (redraw per call or per
 * training step), the same key the same W, bit for bit.
 *
 * Definition (an oracle reproduces it from this text): Philox4x64-10 with key
 * (seed, step) and counter (i, block, head, kind) gives 4 words; words (0, 1)
 * and (2, 3) each give a Box-Muller pair (r cos t, r sin t), r = sqrt(-2 ln u1),
 * t = 2 pi u2, u = ((word >> 11) + 0.5) * 2^-53: normals 4i .. 4i+3 of stream
 * (head, block, kind).  For each head and block b < ceil(m/d): G[r][c] = normal
 * r*d + c of kind 0; G = Q R with R's diagonal positive; row b*d + j of W (if
 * below m) is |g_j| Q[:, j], g_j = normals j*d .. j*d + d-1 of kind 1.  Computed
 * in fp64; the fp32 or bf16 output is the fp64 value rounded once to the nearest
 * representable value (ties to even).
 *
 * d in {16, 32, 64} (else FAVOR_ERR_UNSUPPORTED); W 4-byte aligned, caller-owned.
 */
typedef enum { FAVOR_OUT_BF16 = 0, FAVOR_OUT_F32 = 1 } favor_out_t;
favor_status_t favor_draw_features(unsigned long long seed, unsigned long long step, void* W, int out_dtype,
                                   int H, int m, int d, hipStream_t stream);

/*
 * Backward pass (training): gradients dq, dk, dv of a scalar loss L for its
 * upstream gradient dy = dL/dy, y = favor_attention(q, k, v, W, causal).
 * The pages mention training and gradients but print no formulas; these follow
 * from the forward (Performer notes, Kernel Attention View, Normalization and
 * FAVOR+) by the chain rule, with dphi_f(x)/dx = phi_f(x) (w_f - x).  W is a
 * fixed random draw and gets no gradient.
 *
 * Inputs: q, k, v bf16 [B,H,n,d], W bf16 [H,m,d], y (the forward output) and
 * dy fp32 [B,H,n,d].  Outputs dq, dk, dv fp32 [B,H,n,d] (caller-owned, fully
 * written).  d = 64, m in {64,128,256}; every pointer 16-byte aligned.  ws /
 * ws_bytes as for favor_attention_ws (ws = NULL: scratch allocated stream-
 * ordered on `stream`).  causal = 1: query i's sums run over keys j <= i (the
 * prefix sums of the causal forward), so key j's gradient collects queries
 * i >= j.  Bit-for-bit reproducible for a fixed shape.
 */
size_t favor_backward_workspace_bytes(int B, int H, int n, int d, int m, int causal);
favor_status_t favor_attention_backward(const void* q, const void* k, const void* v, const void* W, const float* y,
                                        const float* dy, float* dq, float* dk, float* dv, int B, int H, int n, int d,
                                        int m, int causal, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Streaming decode -- the causal prefix sums carried from call to call
 * (Performer for vision, How It Works, Step 2: each token adds its key
 * features and value to running sums S, z and reads them with its query).
 *
 * A state holds, for each (b,h) and feature f, over the keys j absorbed so far:
 *   S_f = sum_j 2^(e_jf - c_f) v_j   (d floats),   z_f = sum_j 2^(e_jf - c_f),   c_f,
 * with e_jf = log2(e) (w_f.k_j - |k_j|^2/2): the key/value summary S = Phi(K)^T V
 * and z = Phi(K)^T 1 (Performer notes, Kernel Attention View and Normalization)
 * up to the factor 2^c_f / sqrt(m) per feature, which is carried (c_f) or
 * cancels in y (1/sqrt(m)).  Layout: fp32, favor_state_bytes(B,H,d,m) bytes:
 *   S [B,H,m,d], then z [B,H,m], then c [B,H,m] (log2 units), then one uint32
 *   per (b,h) that favor_decode uses as a finish counter (zero between calls;
 *   favor_state_reset and favor_state_from_keys set it to zero).
 * The empty state is S = 0, z = 0, c = -inf.  Shapes: d == 64, m in {64,128,256}
 * (the bf16 path); q, k, v, W bf16; state and out 16-byte aligned.  Calls on
 * one state must be ordered (one stream, or events between streams).
 *
 * favor_state_bytes  -- bytes of a state (0 if the shape is not supported).
 * favor_state_reset  -- write the empty state.
 * favor_state_from_keys -- replace the state by that of the n keys k, v
 *   ([B,H,n,d]; e.g. a prompt), computed in parallel over the keys.  Scratch is
 *   allocated stream-ordered on `stream`.
 * favor_decode -- T new tokens per (b,h) (q, k, v: [B,H,T,d]), in order: token
 *   t's key and value join the state, then y_t = phi(q_t)^T S / phi(q_t)^T z
 *   (inclusive, as in favor_attention with causal = 1) goes to out
 *   (fp32 [B,H,T,d]).  The state is updated in place; a sequence decoded in any
 *   split into calls gives the same outputs, bit for bit.  Each (b,h) is walked
 *   in token order by 64/CC workgroups, one per slice of CC value columns (CC =
 *   8 for up to 128 heads, wider for more).
 */
size_t favor_state_bytes(int B, int H, int d, int m);
favor_status_t favor_state_reset(float* state, int B, int H, int d, int m, hipStream_t stream);
favor_status_t favor_state_from_keys(const void* k, const void* v, const void* W, float* state,
                                     int B, int H, int n, int d, int m, hipStream_t stream);
favor_status_t favor_decode(const void* q, const void* k, const void* v, const void* W,
                            float* state, float* out, int B, int H, int T, int d, int m,
                            hipStream_t stream);

/*
 * Diagnostics: per-kernel timing with HIP events.  favor_profile_enable()
 * starts recording on the calling thread: every kernel the library launches
 * from that thread is bracketed by two HIP events recorded on the launch
 * stream.  favor_profile_collect() waits for those events, writes up to
 * `capacity` entries (kernel name, launch count, total milliseconds; names
 * are static strings owned by the library), stops recording, clears the
 * record and returns the number of distinct kernels (which may exceed
 * capacity).  Returns -1 if a HIP event call failed.
 * favor_profile_enable_only(name) does the same for the kernels of that one
 * name only (the names favor_profile_collect reports, e.g. "k_output"), so
 * that the events of the others stay out of the stream; NULL means all.  The
 * string is copied.
 */
favor_status_t favor_profile_enable(void);
favor_status_t favor_profile_enable_only(const char* name);
int favor_profile_collect(const char** names, int* counts, double* total_ms, int capacity);

/*
 * Test hook for the causal kernel at d = 64, chunk 64, m in {64, 128, 256}
 * (Performer for vision, How It Works, Step 2: the chunked prefix sums).  In
 * each chunk the waves of the second query tile receive the first key tile's
 * features from the waves of the first, guarded by a per-chunk flag; a
 * waiting wave polls the flag at most `limit` times, then (if the tile has
 * not been claimed) abandons the hand-over and computes the tile itself.
 * Both ways give the same output.  Default 4096; 0 abandons every chunk
 * whose tile is not already claimed, which is how tests reach that path.
 * Process-wide, read at each launch.  limit < 0: FAVOR_ERR_INVALID_ARGUMENT.
 */
favor_status_t favor_set_handover_spin_limit(int limit);

#ifdef __cplusplus
}
#endif
#endif /* FAVOR_H_ */
