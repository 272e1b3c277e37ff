// bf16-input causal FAVOR+ attention on gfx950 (prefix-sum form, chunk 64).
//
// The method (Performer for vision, How It Works, Step 2; Performer notes,
// Normalization): query i aggregates keys j <= i,
//     y_i = phi(q_i)^T S_i / phi(q_i)^T z_i,  S_i = sum_{j<=i} phi(k_j) v_j^T,
//     z_i = sum_{j<=i} phi(k_j).
// Each (b, h) sequence is cut into segments (one workgroup each) and each
// segment into chunks of 64 tokens:
//   phase 1 (k_kv_state, shared with the non-causal path): per-segment state
//            (S, z, per-feature shift c) of the segment's own keys;
//   phase 2 (k_causal_chunks): each segment's workgroup first merges the
//            states of all segments before it, in index order, into its carry;
//            then it walks the segment's chunks in order.  Query i of
//            chunk t sums two terms,
//     carry  phi(q_i)^T S and phi(q_i)^T z over the keys before the chunk, as a
//            softmax over features with weights phi(q_i)_f z_f and values
//            yhat_f = S_f / z_f (the state the non-causal output uses), and
//     chunk  sum_{j in t, j <= i} (phi(q_i)^T phi(k_j)) v_j, from the chunk's own
//            kernel matrix with one exponent shift per query and per key,
//   each with its own log2 scale; the two are brought to the larger scale of
//   the row before they are added, then S += Phi(K_t)^T V_t and z += Phi(K_t)^T 1.
//   Normalising the chunk term per key (not per feature) keeps it exact for the
//   first rows of a chunk, whose visible keys may be far smaller than the ones
//   after them.  Factors common to a row (exp(-|q|^2/2), 1/sqrt(m)) cancel.
#include <math.h>

#include <atomic>

#include "favor_bf16_common.h"
#include "favor_internal.h"
#include "favor_mfma.h"

namespace favor {

// Polls of the key-tile hand-over wait before the query tile 1 wave gives up
// (see cs_query_phase); set through favor_set_handover_spin_limit.
std::atomic<int> g_handover_spin{kHandoverSpinDefault};

namespace {

using namespace bf16k;

// ---------------------------------------------------------------------------
// phase 3
// ---------------------------------------------------------------------------
// Hand-over flag values (per chunk c: value + c; chunks fit in 2^28).
constexpr int kGive = 1, kNoGive = -(1 << 28), kClaim = 1 << 28, kAbandon = 2 << 28;

template <int NW>
struct CsSmem {
  static constexpr int M = NW * 32;
  static constexpr int YS = M + 8;   // fp16 per row of the transposed yhat' table (padded)
  uint16_t w[M * kD];                // W rows (swizzled like the token tiles)
  uint16_t ysh[kD * YS];             // yhat_f (units of sigma_v), [value column][feature slot], fp16
  uint16_t k[kKT * kD];              // chunk tiles, bf16, swizzled
  uint16_t v[kKT * kD];              // values / sigma_v, fp16
  uint16_t q[kKT * kD];
  float knorm[kKT];                  // -|k|^2/2 in log2 units; -inf past the segment end
  float gam[M];                      // log2 of the running feature sums z_f (with shift)
  float colmax[NW][kD];              // prologue scratch (|v| maxima, carry z and c), then
                                     // G_f = 2^(gam_f - Gm) (M) and per-wave max gam (NW)
  float np[NW][32 * kD];             // per wave: partial numerators [query][value, swizzled]
  float dp[NW][32];                  // per wave: partial denominators
  float lp[NW][32];                  // per wave: log2 scale of the partials
  float xs[NW][32];                  // per wave: per-feature scalars, lane -> register layout
  int hflag[NW / 2];                 // per feature group: key tile 0 hand-over state (kGive ...)
  float htile[NW / 2];               // ... and its shift
  __device__ float* gexp() { return &colmax[0][0]; }
  __device__ const float* gexp() const { return &colmax[0][0]; }
  __device__ float* gwmax() { return &colmax[0][0] + M; }
};

template <int NW>
struct CsRegs {
  static constexpr int R = (kKT * 8) / (NW * 64);
  u32x4 k[R], v[R], q[R];
};

template <int NW>
__device__ __forceinline__ void cs_load(CsRegs<NW>& r, const uint16_t* Kb, const uint16_t* Vb,
                                        const uint16_t* Qb, int t0, int ntok, int tid) {
#pragma unroll
  for (int i = 0; i < CsRegs<NW>::R; ++i) {
    const int c = tid + NW * 64 * i;
    const size_t off = static_cast<size_t>(min(t0 + (c >> 3), ntok - 1)) * kD + (c & 7) * 8;
    r.k[i] = *reinterpret_cast<const u32x4*>(Kb + off);
    r.v[i] = *reinterpret_cast<const u32x4*>(Vb + off);
    r.q[i] = *reinterpret_cast<const u32x4*>(Qb + off);
  }
}

// Tiles to LDS (values times vinv as fp16); per key -|k|^2/2 (log2 units), or
// -inf for keys past the end.
template <int NW>
__device__ __forceinline__ void cs_stage(CsSmem<NW>& sm, const CsRegs<NW>& r, int tid, int nvalid,
                                         float vinv) {
#pragma unroll
  for (int i = 0; i < CsRegs<NW>::R; ++i) {
    const int c = tid + NW * 64 * i;
    const int key = c >> 3, ch = c & 7;
    *reinterpret_cast<u32x4*>(&sm.k[swz(key, ch)]) = r.k[i];
    u32x4 vh;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      vh[w] = pack_f16(bf16_lo_as_f32(r.v[i][w]) * vinv, bf16_hi_as_f32(r.v[i][w]) * vinv);
    *reinterpret_cast<u32x4*>(&sm.v[swz(key, ch)]) = vh;
    *reinterpret_cast<u32x4*>(&sm.q[swz(key, ch)]) = r.q[i];
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = bf16_lo_as_f32(r.k[i][w]), b = bf16_hi_as_f32(r.k[i][w]);
      s = fmaf(a, a, s);
      s = fmaf(b, b, s);
    }
    s = sum8(s);
    if (ch == 0) sm.knorm[key] = key < nvalid ? -0.5f * kLog2e * s : -kFInf;
  }
}

// D[row, token] = w_row . x_token for one 32-row tile of W (A operand, rows
// from LDS) against 32 tokens (B operand xB).
__device__ __forceinline__ f32x16 w_proj(const uint16_t* w, int row, int half, const u32x4 (&xB)[4]) {
  f32x16 acc = {};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    acc = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(&w[swz(row, 2 * kb + half)])),
                    as_bf16x8(xB[kb]), acc);
  return acc;
}

__device__ __forceinline__ void tile_rows(const uint16_t* t, int row, int half, u32x4 (&xB)[4]) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) xB[kb] = *reinterpret_cast<const u32x4*>(&t[swz(row, 2 * kb + half)]);
}

// Lane offsets of a row operand (16 bytes of row `col`, chunk 2 kb + half) in
// a swizzled tile; rows 16 apart share the swizzle, so a row base that is a
// multiple of 16 is an immediate offset.
struct RowAddr {
  int c[4];
};
__device__ __forceinline__ RowAddr row_addr(int lane) {
  RowAddr r;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) r.c[kb] = swz(lane & 31, 2 * kb + (lane >> 5));
  return r;
}
// w_proj / tile_rows for row base + col, base a multiple of 16.
__device__ __forceinline__ f32x16 w_proj_at(const uint16_t* w, int base, const RowAddr& ra, const u32x4 (&xB)[4]) {
  f32x16 acc = {};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    acc = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(w + base * 64 + ra.c[kb])), as_bf16x8(xB[kb]), acc);
  return acc;
}
__device__ __forceinline__ void tile_rows_at(const uint16_t* t, int base, const RowAddr& ra, u32x4 (&xB)[4]) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) xB[kb] = *reinterpret_cast<const u32x4*>(t + base * 64 + ra.c[kb]);
}

// Row of D-layout register i inside a 32 x 32 tile, for lane half `half`.
__device__ __forceinline__ int drow(int i, int half) { return 8 * (i >> 2) + 4 * half + (i & 3); }

// Carry weights u_if = 2^(a_if + gam_f - mc_i) and mc_i straight from the
// projections (the rarely taken path; kept out of line so that its registers
// do not weigh on the common path).
struct CarryW {
  u32x4 ua[2][2];
  float mc;
};
template <int NW>
__device__ __attribute__((noinline)) CarryW carry_weights_exact(const CsSmem<NW>& sm, int f0, int qt,
                                                                int lane) {
  const int col = lane & 31, half = lane >> 5;
  CarryW r;
  u32x4 xB[4];
  tile_rows(sm.q, 32 * qt + col, half, xB);
  float mc = -kFInf;
#pragma unroll
  for (int ft = 0; ft < 2; ++ft) {
    const f32x16 pr = w_proj(sm.w, f0 + 32 * ft + col, half, xB);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 g = *reinterpret_cast<const f32x4*>(&sm.gam[f0 + 32 * ft + 8 * g4 + 4 * half]);
#pragma unroll
      for (int j = 0; j < 4; ++j) mc = fmaxf(mc, fmaf(pr[4 * g4 + j], kLog2e, g[j]));
    }
  }
  mc = pair_max(mc);
#pragma unroll
  for (int ft = 0; ft < 2; ++ft) {
    const f32x16 pr = w_proj(sm.w, f0 + 32 * ft + col, half, xB);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 g = *reinterpret_cast<const f32x4*>(&sm.gam[f0 + 32 * ft + 8 * g4 + 4 * half]);
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const int i = 4 * g4 + j;
        r.ua[ft][g4 >> 1][2 * (g4 & 1) + (j >> 1)] =
            pack_f16(fast_exp2(fmaf(pr[i], kLog2e, g[j]) - mc),
                     fast_exp2(fmaf(pr[i + 1], kLog2e, g[j + 1]) - mc));
      }
    }
  }
  r.mc = mc;
  return r;
}

// Query side of one chunk for the wave's 32 queries (tile qt) and 64 features
// (group fg): partial numerator, denominator and their log2 scale L_i.
//   carry:  u_if = 2^(a_if + gam_f - mc_i) (fp16), mc_i = max_f (a_if + gam_f);
//           sum_f u_if yhat_f and sum_f u_if, both times 2^(mc_i - L_i)
//   chunk:  P_ij = sum_f 2^(a_if - alpha_i) 2^(b_jf + n_j - T)   (bf16 hi/lo, three
//           MFMAs per 16 features), alpha_i = max_f a_if, T = the key tile's
//           largest beta_j (or, on the diagonal tile with a wide beta spread,
//           per-key shifts and a per-row factor, see below), times
//           2^(alpha_i + T - L_i);  sum_j P_ij v_j and sum_j P_ij
// with a_if = log2e w_f.q_i, b_jf = log2e w_f.k_j, n_j = -log2e |k_j|^2/2,
// L_i = max(mc_i, alpha_i + T + log2 max_j P_ij) over the tiles.  The factor
// exp(-|q_i|^2/2) / sqrt(m) common to every term of a row is left out.
template <int NW, int QT>
__device__ __forceinline__ void cs_query_phase(CsSmem<NW>& sm, int wave, int lane, float Gm,
                                               int chunk, int spin) {
  constexpr int YS = CsSmem<NW>::YS;
  const float* gexp = sm.gexp();
  constexpr int qt = QT;
  const int col = lane & 31, half = lane >> 5;
  const int f0 = 64 * (wave % (NW / 2));

  const RowAddr ra = row_addr(lane);
  u32x4 xB[4];
  tile_rows_at(sm.q, 32 * qt, ra, xB);
  f32x16 pa[2];
  pa[0] = w_proj_at(sm.w, f0, ra, xB);
  pa[1] = w_proj_at(sm.w, f0 + 32, ra, xB);
  // query features 2^(a_if - alpha_i), alpha_i = max_f a_if (the maximum of
  // the raw projections, scaled afterwards: rounding is monotone), in place
  float amax = -kFInf;
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, pa[ft][i]);
  amax = pair_max(amax) * kLog2e;
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int i = 0; i < 16; ++i) pa[ft][i] = fast_exp2(fmaf(pa[ft][i], kLog2e, -amax));
  // carry weights u_if = 2^(a_if + gam_f - mc_i) (fp16, A operand: lane =
  // query, k = feature), mc_i = max_f (a_if + gam_f).  From the features
  // above: u_if = 2^(a_if - alpha_i) G_f / max_f (...), G_f = 2^(gam_f - Gm)
  // (published with the state, Gm = max_f gam_f), so mc_i = alpha_i + Gm +
  // log2 max_f (...).  When some row's maximum product falls below 2^-60
  // (its strongest state features are far from its own), the weights are
  // taken from the projections directly, after the chunk term (where fewer
  // registers are live).
  u32x4 ua[2][2];
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) ua[ft][kb2] = u32x4{0u, 0u, 0u, 0u};
  float mc = -kFInf;
  bool exact_carry = false;   // wave-uniform
  if (Gm != -kFInf) {         // else no keys before this chunk: no carry
    float pmx = 0.f;
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 G = *reinterpret_cast<const f32x4*>(&gexp[f0 + 32 * ft + 8 * g4 + 4 * half]);
#pragma unroll
        for (int j = 0; j < 4; ++j) pmx = fmaxf(pmx, pa[ft][4 * g4 + j] * G[j]);
      }
    pmx = pair_max(pmx);
    exact_carry = __ballot(!(pmx >= 0x1p-60f)) != 0;
    if (!exact_carry) {
      const float kap = fast_rcp(pmx);
      mc = __log2f(pmx) + amax + Gm;
#pragma unroll
      for (int ft = 0; ft < 2; ++ft)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 G = *reinterpret_cast<const f32x4*>(&gexp[f0 + 32 * ft + 8 * g4 + 4 * half]);
#pragma unroll
          for (int j = 0; j < 4; j += 2) {
            const int i = 4 * g4 + j;
            ua[ft][g4 >> 1][2 * (g4 & 1) + (j >> 1)] =
                pack_f16(pa[ft][i] * G[j] * kap, pa[ft][i + 1] * G[j + 1] * kap);
          }
        }
    }
  }

  // query features of the chunk term, bf16 hi + lo (B operand: k = feature, n = query)
  u32x4 ahi[2][2], alo[2][2];
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t h_, l_;
        split_bf16_trunc(pa[ft][8 * kb2 + 2 * w], pa[ft][8 * kb2 + 2 * w + 1], h_, l_);
        ahi[ft][kb2][w] = h_;
        alo[ft][kb2][w] = l_;
      }

  // P^T[key, query] for key tiles kt <= qt (lane = query, registers = keys).
  // Key features carry one exponent shift per key:
  //   shared: n_j - T, T = max_j beta_j over the tile, beta_j = bmax_j + n_j
  //           (n_j = -log2e |k_j|^2/2, bmax_j the key's largest log2e w_f.k_j over
  //           the first 32 of the features).  Every row of the tile then has
  //           the common scale 2^T.  Always used for the tile below the
  //           diagonal, whose keys every query of the wave sees.
  //   per key: -bmax_j, then each entry times 2^(beta_j - B_i), B_i the largest
  //           beta among the keys <= i; used for the diagonal tile when some
  //           key's beta lies more than 2^kSpread below T (the first rows
  //           would otherwise see only keys far below the tile's scale).
  // s[kt] is the log2 scale of tile kt's entries for this lane's query row.
  constexpr float kSpread = 32.f;
  f32x16 pt[2] = {};
  float bj[2] = {-kFInf, -kFInf};
  float s[2] = {-kFInf, -kFInf};
  bool perkey = false;   // wave-uniform: the diagonal tile uses per-key shifts
  // Key tile 0 is the query tile 0 wave's diagonal tile and the query tile 1
  // wave's off-diagonal one, with the same shared shift unless the former
  // needs per-key shifts.  The tile 0 wave hands its operands over through the
  // tile 1 wave's partial slot (free until that wave's own partials), guarded
  // by a per-chunk flag whose values name the chunk:
  //   kGive + c   operands handed over       kNoGive + c  none (per-key shifts)
  //   kClaim + c  tile 0 is writing them     kAbandon + c tile 1 gave up waiting
  // The tile 0 wave claims the slot (compare-and-swap) before its first write
  // and writes nothing once tile 1 has abandoned the chunk; the tile 1 wave
  // abandons only a chunk that tile 0 has not claimed (the same compare-and-
  // swap), so the slot is never written by both.  A claimed hand-over is
  // straight-line code up to its release, so waiting for it always ends.
  const int grp = wave % (NW / 2);
  uint32_t* hand = reinterpret_cast<uint32_t*>(sm.np[NW / 2 + grp]);
  const int cgive = kGive + chunk, cnogive = kNoGive + chunk;
  const int cclaim = kClaim + chunk, cabandon = kAbandon + chunk;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int kt = qt == 1 ? 1 - kk : kk;   // the diagonal tile first
    if (kt > qt) continue;
    if (qt == 1 && kt == 0) {
      int f = 0;
      for (int it = 0;;) {
        f = __hip_atomic_load(&sm.hflag[grp], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (f == cgive || f == cnogive) break;
        if (f != cclaim && ++it >= spin) {
          // tile 0 has not claimed the slot: abandon the hand-over, unless the
          // flag moved meanwhile (then look again)
          int ok = 0;
          if (lane == 0) {
            int expect = f;
            ok = __hip_atomic_compare_exchange_strong(&sm.hflag[grp], &expect, cabandon, __ATOMIC_ACQ_REL,
                                                      __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
          if (__builtin_amdgcn_readfirstlane(ok)) {
            f = cabandon;
            break;
          }
          continue;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (f == cgive) {
        s[0] = sm.htile[grp];
#pragma unroll
        for (int ft = 0; ft < 2; ++ft)
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) {
            const int blk = 2 * (2 * ft + kb2);
            const u32x4 bhi = *reinterpret_cast<const u32x4*>(&hand[(blk * 64 + lane) * 4]);
            const u32x4 blo = *reinterpret_cast<const u32x4*>(&hand[((blk + 1) * 64 + lane) * 4]);
            pt[0] = mfma_bf16(as_bf16x8(bhi), as_bf16x8(ahi[ft][kb2]), pt[0]);
            pt[0] = mfma_bf16(as_bf16x8(blo), as_bf16x8(ahi[ft][kb2]), pt[0]);
            pt[0] = mfma_bf16(as_bf16x8(bhi), as_bf16x8(alo[ft][kb2]), pt[0]);
          }
        continue;
      }
    }
    tile_rows_at(sm.k, 32 * kt, ra, xB);
    float sh = 0.f;
    bool give = false;   // wave-uniform
#pragma unroll
    for (int ft = 0; ft < 2; ++ft) {
      const f32x16 pk = w_proj_at(sm.w, f0 + 32 * ft, ra, xB);
      if (ft == 0) {
        float bm = -kFInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) bm = fmaxf(bm, pk[i]);
        bm = pair_max(bm) * kLog2e;
        const float kn = sm.knorm[32 * kt + col];   // -inf past the segment end
        const float beta = bm + kn;
        const float T = max32_uniform(beta);
        bj[kt] = beta;
        if (kt == qt) perkey = __ballot(beta > -kFInf && beta < T - kSpread) != 0;
        const bool pk_shift = kt == qt && perkey;
        sh = pk_shift ? -bm : (T == -kFInf ? -kFInf : kn - T);
        s[kt] = T;
        give = qt == 0 && !perkey;
        if (give) {
          // claim the slot before the first write (fails once tile 1 abandoned the chunk)
          int ok = 0;
          if (lane == 0) {
            int expect = __hip_atomic_load(&sm.hflag[grp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            ok = expect != cabandon &&
                 __hip_atomic_compare_exchange_strong(&sm.hflag[grp], &expect, cclaim, __ATOMIC_ACQ_REL,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
          give = __builtin_amdgcn_readfirstlane(ok) != 0;
        }
      }
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        u32x4 bhi, blo;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t h_, l_;
          split_bf16_trunc(fast_exp2(fmaf(pk[8 * kb2 + 2 * w], kLog2e, sh)),
                           fast_exp2(fmaf(pk[8 * kb2 + 2 * w + 1], kLog2e, sh)), h_, l_);
          bhi[w] = h_;
          blo[w] = l_;
        }
        if (give) {
          const int blk = 2 * (2 * ft + kb2);
          *reinterpret_cast<u32x4*>(&hand[(blk * 64 + lane) * 4]) = bhi;
          *reinterpret_cast<u32x4*>(&hand[((blk + 1) * 64 + lane) * 4]) = blo;
        }
        pt[kt] = mfma_bf16(as_bf16x8(bhi), as_bf16x8(ahi[ft][kb2]), pt[kt]);
        pt[kt] = mfma_bf16(as_bf16x8(blo), as_bf16x8(ahi[ft][kb2]), pt[kt]);
        pt[kt] = mfma_bf16(as_bf16x8(bhi), as_bf16x8(alo[ft][kb2]), pt[kt]);
      }
    }
    if (qt == 0) {
      // the flag is released after the operands and the shift; an abandoned
      // chunk keeps its flag (tile 1 computes key tile 0 itself)
      if (give && lane == 0) sm.htile[grp] = s[0];
      if (lane == 0 && (give || perkey))
        __hip_atomic_store(&sm.hflag[grp], give ? cgive : cnogive, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }

  if (exact_carry) {
    const CarryW cw = carry_weights_exact<NW>(sm, f0, qt, lane);
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) ua[ft][kb2] = cw.ua[ft][kb2];
    mc = cw.mc;
  }

  // causal mask on the diagonal tile (keys after the query drop out), the
  // per-key factors where used, and each tile's row maximum
  float* scr = sm.np[wave];
  float rmx[2] = {0.f, 0.f};
  if (qt == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) rmx[0] = fmaxf(rmx[0], pt[0][i]);
    rmx[0] = pair_max(rmx[0]);
  }
  if (perkey) {
    // beta of the key in each register (lane -> register layout through the
    // wave's own partial slot, which is written only at the end)
    if (half == 0) scr[col] = bj[qt];
    s[qt] = prefix_max32(bj[qt], lane);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(&scr[8 * g4 + 4 * half]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * g4 + j;
        const float p = drow(i, half) <= col ? pt[qt][i] * fast_exp2(b4[j] - s[qt]) : 0.f;
        pt[qt][i] = p;
        rmx[qt] = fmaxf(rmx[qt], p);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = drow(i, half) <= col ? pt[qt][i] : 0.f;
      pt[qt][i] = p;
      rmx[qt] = fmaxf(rmx[qt], p);
    }
  }
  rmx[qt] = pair_max(rmx[qt]);
  float ic = -kFInf;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
    if (kt <= qt && rmx[kt] > 0.f) ic = fmaxf(ic, s[kt] + __log2f(rmx[kt]));
  const float L = fmaxf(mc, amax + ic);
  const float Ls = L == -kFInf ? 0.f : L;
  float fac[2] = {0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
    if (kt <= qt && rmx[kt] > 0.f) fac[kt] = fast_exp2(amax + s[kt] - Ls);
  const float cfac = mc == -kFInf ? 0.f : fast_exp2(mc - Ls);

  // Both terms accumulate into one numerator from fp16 weights already at the
  // row's scale L: the carry weights times cfac (packed fp16; a weight under
  // fp16 range is under 2^-24 of the row's largest and drops out), the chunk
  // weights times fac.  The denominator sums exactly the rounded weights the
  // numerator uses, in fp32 (v_dot2 over this lane's weights of its query,
  // then the two lanes of the query column).
  f32x16 np0 = {}, np1 = {};
  float dl = 0.f;
  const f16x2 ones2 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
  const f16x2 cf2 = {static_cast<_Float16>(cfac), static_cast<_Float16>(cfac)};
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const int kpos = f0 + 32 * ft + 16 * kb2 + 8 * half;
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(&sm.ysh[col * YS + kpos]);
      const u32x4 b1 = *reinterpret_cast<const u32x4*>(&sm.ysh[(32 + col) * YS + kpos]);
      u32x4 a;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t h = mul_f16x2(ua[ft][kb2][w], cf2);
        dl = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, h), ones2, dl, false);
        a[w] = h;
      }
      np0 = mfma_f16(as_f16x8(b0), as_f16x8(a), np0);
      np1 = mfma_f16(as_f16x8(b1), as_f16x8(a), np1);
    }
  const VOpAddr va = vop_addr(lane);
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    if (kt > qt) break;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      u32x4 a;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t h = pack_f16(pt[kt][8 * kb2 + 2 * w] * fac[kt], pt[kt][8 * kb2 + 2 * w + 1] * fac[kt]);
        dl = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, h), ones2, dl, false);
        a[w] = h;
      }
      const u32x4 v0 = v_operand_at(sm.v, 32 * kt + 16 * kb2, 0, va);
      const u32x4 v1 = v_operand_at(sm.v, 32 * kt + 16 * kb2, 1, va);
      np0 = mfma_f16(as_f16x8(v0), as_f16x8(a), np0);
      np1 = mfma_f16(as_f16x8(v1), as_f16x8(a), np1);
    }
  }

  // The products are formed transposed (value operand first): register
  // 4 g + j holds value column 8 g + 4 half + j (np1: 32 + that) of query
  // col, so each lane writes its query row's values four at a time.  The
  // row's 8-float blocks are XOR-swizzled by row & 7, so that the combine
  // step's reads of 8 rows hit different banks.
  {
    float* row = scr + col * kD + 4 * half;
    const int sw = (col & 7) << 3;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      *reinterpret_cast<f32x4*>(row + ((8 * g) ^ sw)) =
          f32x4{np0[4 * g], np0[4 * g + 1], np0[4 * g + 2], np0[4 * g + 3]};
      *reinterpret_cast<f32x4*>(row + ((32 + 8 * g) ^ sw)) =
          f32x4{np1[4 * g], np1[4 * g + 1], np1[4 * g + 2], np1[4 * g + 3]};
    }
  }
  const float dq = pair_sum(dl);   // the denominator of query col
  if (half == 0) {
    sm.dp[wave][col] = dq;
    sm.lp[wave][col] = L;
  }
}

// Power of two >= x (x >= 0); 1 for x = 0.
__device__ __forceinline__ float pow2_above(float x) {
  int ex = 0;
  if (x > 0.f && x <= 3.0e38f) frexpf(x, &ex);
  return ldexpf(1.0f, ex);
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void k_causal_chunks(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ W, const float* __restrict__ part_S,
    const float* __restrict__ part_zc, const float* __restrict__ seg_vmax,
    float* __restrict__ out, int H, int n, int nseg, int seglen, int has_carry, int spin) {
  constexpr int M = NW * 32;
  constexpr int YS = CsSmem<NW>::YS;
  constexpr int NQ = NW / 2;  // feature groups per query tile
  __shared__ __attribute__((aligned(16))) CsSmem<NW> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  // the segments of one (b, h) share an XCD: their prologues read the same
  // earlier segment states, which then pass through one L2
  const int wg = xcd_contiguous(blockIdx.x, gridDim.x);
  const int bh = wg / nseg;
  const int seg = wg - bh * nseg;
  const int hh = bh % H;
  const int s0 = seg * seglen;
  const int ntok = min(n, s0 + seglen) - s0;
  if (ntok <= 0) return;  // whole workgroup exits together
  const size_t tok0 = static_cast<size_t>(bh) * n + s0;
  const uint16_t* Kb = K + tok0 * kD;
  const uint16_t* Vb = V + tok0 * kD;
  const uint16_t* Qb = Q + tok0 * kD;
  float* Ob = out + tok0 * kD;

  for (int c = tid; c < M * 8; c += NW * 64) {
    const int f = c >> 3, ch = c & 7;
    *reinterpret_cast<u32x4*>(&sm.w[swz(f, ch)]) =
        *reinterpret_cast<const u32x4*>(W + (static_cast<size_t>(hh) * M + f) * kD + ch * 8);
  }

  // Values are staged as fp16 after scaling by 1 / sigma_v, a power of two
  // above the largest |v| of this and the earlier segments (from the state
  // pass when there is one, else from a pass over the segment's values).
  // Every S, yhat and partial numerator below is in units of sigma_v; yhat, a
  // weighted average of values up to the current chunk, stays inside (-1, 1).
  float vm;
  if (has_carry) {
    vm = 0.f;
    for (int s2 = 0; s2 <= seg; ++s2) vm = fmaxf(vm, seg_vmax[static_cast<size_t>(bh) * nseg + s2]);
  } else {
    vm = 0.f;
    for (int cc = tid; cc < ntok * 8; cc += NW * 64) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(Vb + static_cast<size_t>(cc >> 3) * kD + (cc & 7) * 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) vm = fmaxf(vm, fmaxf(fabsf(bf16_lo_as_f32(x[w])), fabsf(bf16_hi_as_f32(x[w]))));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) vm = fmaxf(vm, __shfl_xor(vm, o));
    if (lane == 0) sm.colmax[wave][0] = vm;
    __syncthreads();
    vm = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) vm = fmaxf(vm, sm.colmax[w][0]);
    __syncthreads();
  }
  const float vsig = pow2_above(vm);
  const float vinv = 1.0f / vsig;

  // Running state of the keys before the current chunk for the wave's 32
  // features: S (D layout, rows = features, lanes = value columns), z and the
  // shift c (lane = feature).  sum_j exp(w_f.k_j - |k_j|^2/2) = z_f 2^c_f.
  const int fk = 32 * wave + col;
  float c = -kFInf, z = 0.f;
  f32x16 sacc[2] = {};
  if (has_carry && seg > 0) {
    // Carry = ordered merge of the states of segments 0 .. seg-1 (from the
    // state pass).  Each partial, and the running state, is renormalised to
    // z = 1 by folding log2 z into its shift.  Two threads per feature, 32
    // value columns each; the result goes through the (still unused) partial
    // slots into the key side's register layout.
    const int f = tid >> 1, hq = tid & 1;
    float cr = -kFInf, zr = 0.f;
    f32x4 Sr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) Sr[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int s2 = 0; s2 < seg; ++s2) {
      const size_t base = static_cast<size_t>(bh) * nseg + s2;
      float cp = part_zc[base * 2 * M + M + f];
      const float zp = part_zc[base * 2 * M + f];
      const f32x4* src = reinterpret_cast<const f32x4*>(part_S + (base * M + f) * kD + 32 * hq);
      f32x4 r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = src[j];
      float bscale = 0.f;
      if (cp != -kFInf && zp > 0.f) {
        bscale = 1.0f / zp;
        cp += log2f(zp);
      } else {
        cp = -kFInf;
      }
      const float cn = fmaxf(cr, cp);
      const float a = (cr == -kFInf) ? 0.f : exp2f(cr - cn);
      const float b = (cp == -kFInf) ? 0.f : exp2f(cp - cn) * bscale;
      zr = fmaf(a, zr, b * zp);
#pragma unroll
      for (int j = 0; j < 8; ++j) Sr[j] = a * Sr[j] + b * r[j];
      cr = cn;
      if (zr > 0.f) {
        const float iz = 1.0f / zr;
        cr += log2f(zr);
        zr = 1.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) Sr[j] *= iz;
      }
    }
    float* cbuf = &sm.np[0][0];
    float* zcb = &sm.colmax[0][0];
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<f32x4*>(&cbuf[f * kD + 32 * hq + 4 * j]) = Sr[j];
    if (hq == 0) {
      zcb[f] = zr;
      zcb[M + f] = cr;
    }
    __syncthreads();
    z = zcb[fk];
    c = zcb[M + fk];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        sacc[dt][i] = cbuf[(32 * wave + drow(i, half)) * kD + 32 * dt + col] * vinv;
    __syncthreads();
  }

  const int nchunks = (ntok + kKT - 1) / kKT;
  CsRegs<NW> regs;
  cs_load<NW>(regs, Kb, Vb, Qb, 0, ntok, tid);

  float izr[16];   // 1/z of the feature held in D-layout register i
  float gam = -kFInf;
  // state summary: 1/z in the D layout (through the wave's scalar slots) and
  // gam = c + log2 z; z >= 1 whenever it is nonzero (the shift keeps the
  // largest key feature at 1 or above), so the hardware reciprocal is safe
  auto summarize = [&](int col, int half) {
    const float iz = z > 0.f ? fast_rcp(z) : 0.f;
    gam = z > 0.f ? c + __log2f(z) : -kFInf;
    if (half == 0) sm.xs[wave][col] = iz;
    const float gw = max32_uniform(gam);
    if (lane == 0) sm.gwmax()[wave] = gw;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 z4 = *reinterpret_cast<const f32x4*>(&sm.xs[wave][8 * g4 + 4 * half]);
#pragma unroll
      for (int j = 0; j < 4; ++j) izr[4 * g4 + j] = z4[j];
    }
  };
  // after a barrier (the previous chunk's readers are done): yhat, gam and
  // G_f = 2^(gam_f - Gm) to LDS; Gm = max_f gam_f (-inf before any key)
  float Gm = -kFInf;
  auto publish = [&](int col, int half) {
    Gm = -kFInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) Gm = fmaxf(Gm, sm.gwmax()[w]);
    if (half == 0) sm.gexp()[32 * wave + col] = gam == -kFInf ? 0.f : fast_exp2(gam - Gm);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int fr = 32 * wave + 8 * g4 + 4 * half;
      const int pos = (fr & ~15) | kblock_pos(fr & 15);
      const int i = 4 * g4;
      *reinterpret_cast<u32x2*>(&sm.ysh[col * YS + pos]) =
          u32x2{pack_f16(sacc[0][i] * izr[i], sacc[0][i + 1] * izr[i + 1]),
                pack_f16(sacc[0][i + 2] * izr[i + 2], sacc[0][i + 3] * izr[i + 3])};
      *reinterpret_cast<u32x2*>(&sm.ysh[(32 + col) * YS + pos]) =
          u32x2{pack_f16(sacc[1][i] * izr[i], sacc[1][i + 1] * izr[i + 1]),
                pack_f16(sacc[1][i + 2] * izr[i + 2], sacc[1][i + 3] * izr[i + 3])};
    }
    if (half == 0) sm.gam[32 * wave + col] = gam;
  };

  if (tid < NW / 2) sm.hflag[tid] = 0;
  summarize(col, half);
  lds_barrier();
  publish(col, half);
  cs_stage<NW>(sm, regs, tid, ntok, vinv);
  // Prefetch loads are issued on every path (past the end they re-read the
  // clamped last token), which keeps the compiler's wait before each stage
  // from also waiting on the output stores issued after the loads.
  cs_load<NW>(regs, Kb, Vb, Qb, kKT, ntok, tid);
  lds_barrier();

  for (int t = 0; t < nchunks; ++t) {
    const int t0 = t * kKT;
    // Lane-dependent LDS addresses are cheap to recompute; keeping them out of
    // loop-invariant registers leaves room for the accumulators.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int col = ln & 31, half = ln >> 5;
    const int fk = 32 * wave + col;
    const bool tile0 = wave < NW / 2;   // wave-uniform
    if (tile0)
      cs_query_phase<NW, 0>(sm, wave, ln, Gm, t, spin);
    else
      cs_query_phase<NW, 1>(sm, wave, ln, Gm, t, spin);
    // Query tile 1 carries twice tile 0's chunk term.  Its waves therefore
    // update their key state after the first barrier, while the tile 0 waves
    // combine the partials; a second barrier then lets the tiles be restaged.
    // (Every wave passes three barriers per chunk, at wave-uniform points.)
    if (!tile0) lds_barrier();

    // ---- key side: this chunk's keys into the wave's features (not after
    // the segment's last chunk, whose state nothing reads)
    const bool more = t + 1 < nchunks;
    if (more) {
      f32x16 pk[2];
      {
        const RowAddr ra = row_addr(ln);
        u32x4 wB[4];
        tile_rows_at(sm.w, 32 * wave, ra, wB);
  #pragma unroll
        for (int st = 0; st < 2; ++st) {
          f32x16 acc = {};
  #pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            acc = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.k[32 * st * 64 + ra.c[kb]])),
                            as_bf16x8(wB[kb]), acc);
  #pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 kn = *reinterpret_cast<const f32x4*>(&sm.knorm[32 * st + 8 * g4 + 4 * half]);
  #pragma unroll
            for (int j = 0; j < 4; ++j) acc[4 * g4 + j] = fmaf(acc[4 * g4 + j], kLog2e, kn[j]);
          }
          pk[st] = acc;
        }
      }
      float mx = -kFInf;
  #pragma unroll
      for (int st = 0; st < 2; ++st)
  #pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, pk[st][i]);
      mx = pair_max(mx);
      // raise the shift when this chunk's keys exceed it by more than 2^8
      const bool need = mx > c + 8.0f;
      if (__ballot(need) != 0) {
        const float cn = need ? mx : c;
        const float sc = need ? ((c == -kFInf) ? 0.f : exp2f(c - cn)) : 1.0f;
        z *= sc;
        c = cn;
        if (half == 0) sm.xs[wave][col] = sc;
  #pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 s4 = *reinterpret_cast<const f32x4*>(&sm.xs[wave][8 * g4 + 4 * half]);
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            sacc[0][4 * g4 + j] *= s4[j];
            sacc[1][4 * g4 + j] *= s4[j];
          }
        }
      }
      // S += Phi(K_t)^T V_t / sigma_v with fp16 key features (at most 2^8); z
      // sums the same rounded features in fp32 (v_dot2: this lane's keys, then
      // the two lanes of the feature column)
      const float cs = c == -kFInf ? 0.f : c;
      const f16x2 ones2 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
      const VOpAddr va = vop_addr(ln);
      float zp = 0.f;
  #pragma unroll
      for (int st = 0; st < 2; ++st)
  #pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          u32x4 a;
  #pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t h = pack_f16(fast_exp2(pk[st][8 * kb2 + 2 * w] - cs),
                                        fast_exp2(pk[st][8 * kb2 + 2 * w + 1] - cs));
            zp = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, h), ones2, zp, false);
            a[w] = h;
          }
  #pragma unroll
          for (int dt = 0; dt < 2; ++dt) {
            const u32x4 vb = v_operand_at(sm.v, 32 * st + 16 * kb2, dt, va);
            sacc[dt] = mfma_f16(as_f16x8(a), as_f16x8(vb), sacc[dt]);
          }
        }
      z += pair_sum(zp);
    }
    if (more) summarize(col, half);
    if (tile0) {
      lds_barrier();
      // ---- combine the partials of the chunk's rows and store
      for (int it = tid; it < kKT * 8; it += NW / 2 * 64) {
        const int qrow = it >> 3, d0 = (it & 7) * 8;
        if (t0 + qrow >= ntok) continue;
        const int qt = qrow >> 5, r = qrow & 31;
        float lmax = -kFInf;
#pragma unroll
        for (int g = 0; g < NQ; ++g) lmax = fmaxf(lmax, sm.lp[qt * NQ + g][r]);
        float den = 0.f;
        f32x4 n0 = {0.f, 0.f, 0.f, 0.f}, n1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < NQ; ++g) {
          const int w = qt * NQ + g;
          const float l = sm.lp[w][r];
          const float wt = l == -kFInf ? 0.f : fast_exp2(l - lmax);
          den = fmaf(wt, sm.dp[w][r], den);
          const int ds = d0 ^ ((r & 7) << 3);
          const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.np[w][r * kD + ds]);
          const f32x4 b = *reinterpret_cast<const f32x4*>(&sm.np[w][r * kD + ds + 4]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            n0[j] = fmaf(wt, a[j], n0[j]);
            n1[j] = fmaf(wt, b[j], n1[j]);
          }
        }
        const float inv = vsig * fast_rcp(den);
        f32x4* dst = reinterpret_cast<f32x4*>(Ob + static_cast<size_t>(t0 + qrow) * kD + d0);
        __builtin_nontemporal_store(n0 * inv, dst);
        __builtin_nontemporal_store(n1 * inv, dst + 1);
      }
    }
    lds_barrier();   // every key state updated and summarised
    if (more) {
      publish(col, half);
      cs_stage<NW>(sm, regs, tid, ntok - t0 - kKT, vinv);
      cs_load<NW>(regs, Kb, Vb, Qb, t0 + 2 * kKT, ntok, tid);
    }
    lds_barrier();
  }
}

template <int NW>
hipError_t launch_chunks(const Bf16Plan& p, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const uint16_t* W, const float* pS, const float* pzc,
                         const float* vmax, float* out, hipStream_t s) {
  FAVOR_LAUNCH("k_causal_output", k_causal_chunks<NW>, dim3(p.B * p.H * p.splits), dim3(NW * 64), 0,
               s, q, k, v, W, pS, pzc, vmax, out, p.H, p.n, p.splits, p.span, p.splits > 1 ? 1 : 0,
               g_handover_spin.load(std::memory_order_relaxed));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_causal_chunks(const Bf16Plan& p, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const uint16_t* W, const float* part_S,
                                const float* part_zc, const float* vmax, float* out,
                                hipStream_t s) {
  switch (p.m) {
    case 64: return launch_chunks<2>(p, q, k, v, W, part_S, part_zc, vmax, out, s);
    case 128: return launch_chunks<4>(p, q, k, v, W, part_S, part_zc, vmax, out, s);
    case 256: return launch_chunks<8>(p, q, k, v, W, part_S, part_zc, vmax, out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace favor
