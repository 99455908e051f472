// Register-resident gate prefix sums and centred chunk operands shared by the
// chunk-parallel kernels.
//
// Gate prefix (KDA blog 6.6; base 2 as in the pages' pipeline): thread t of an
// NTH-thread workgroup owns feature column c = t % KC of a [64 x KC] gate tile
// and the rows [seg*RS, seg*RS + RS), seg = t / KC.  The in-chunk inclusive sum
// G2 = log2(e) * cumsum(g) is formed in registers; one LDS exchange of segment
// totals joins the segments.
//
// Centring (ReWY paper section 3.3, "Centered factors", and Appendix 8): every
// sub-chunk J of 16 rows gets, per feature, a receiving reference rA_J and a
// sending reference rB_J: both its gate midpoint (max + min) / 2, or, for the
// features of a 16-feature block in which some feature's gate range over the
// sub-chunk exceeds CENTRE_MAX_RANGE, its first row (rA) and its last valid
// row (rB).  Operands are stored pre-scaled,
//   Ka[i] = beta_i k_i exp2(G_i - rA),  Qa[i] = s q_i exp2(G_i - rA),
//   Kc[j] = k_j exp2(rB - G_j),
// and a pair of sub-chunks I > J contributes through the per-feature factor
//   f_IJ = exp2(rA_I - rB_J) <= 1   (rA_I <= G at the first row of I <= G at the
//                                    last row of J <= rB_J for a decaying gate),
// so exp2(G_i - G_j) = exp2(G_i - rA_I) f_IJ exp2(rB_J - G_j) is never formed as
// a product of unbounded factors.  Midpoint-centred factors are bounded by
// 2^(range/2) <= 2^64.  On a diagonal pair the terms of a wide feature block are
// summed pairwise instead.
#pragma once
#include "chunk_common.hpp"

namespace rewy {

// Thread t < 4*KC owns feature column c = t % KC and sub-chunk seg = t / KC,
// i.e. the 16 rows [16 seg, 16 seg + 16); threads t >= 4*KC take no part.
template <int KC>
struct GateCols {
  static constexpr int NG = NSUB * KC;  // participating threads
  static constexpr int RS = SUB;        // rows per thread
  float G[RS];
  int c, seg;
  bool on;

  __device__ __forceinline__ void init(int tid) {
    on = tid < NG;
    c = tid % KC;
    seg = (tid / KC) % NSUB;
  }
  // Column pairs: slot s (0 or 1) of thread tid < 2 KC takes column
  // 2 (tid % (KC/2)) + s of sub-chunk tid / (KC/2), so a thread's two slots are
  // adjacent columns of the same 16 rows (element pairs are contiguous).
  __device__ __forceinline__ void init_pair(int tid, int s) {
    on = tid < 2 * KC;
    c = 2 * (tid % (KC / 2)) + s;
    seg = (tid / (KC / 2)) % NSUB;
  }
  // raw natural-log gates, features [k0, k0 + KC), of the chunk's n >= 1 rows,
  // through a bounds-checked buffer: rows past the end (and every row without
  // a gate) read as zero.  One unconditional load per row, so the loads' wait
  // falls at their first use.
  __device__ __forceinline__ void load(const Args& a, int64_t t0, int h, int n, int K, int k0) {
    const int H = a.H, r0 = seg * RS;
    const bool vec = a.gate == 2;
    const int64_t rs = vec ? (int64_t)H * K : H;  // row stride, elements
    const float* gb = vec ? a.g + (t0 * H + h) * K + k0 : a.g + t0 * H + h;
    const GBuf b = gbuf(gb, a.gate == 0 ? 0u : tile_bytes<float>(n, rs, vec ? KC : 1));
    const uint32_t rb = (uint32_t)(rs * 4), base = (uint32_t)r0 * rb + (vec ? c : 0) * 4;
#pragma unroll
    for (int r = 0; r < RS; ++r) G[r] = __uint_as_float(gld4(b, base + r * rb));
  }
  // Both slots of a column pair (init_pair: this slot's column c and the
  // column c + 1 of slot `odd`, the same rows), one 8-byte load per row.  The
  // range check of a buffer load is made per 4-byte word, so a scalar gate
  // (one word per row; the second word of each load is not used) reads its
  // last row like the others.
  __device__ __forceinline__ void load_pair(GateCols& odd, const Args& a, int64_t t0, int h, int n, int K) {
    const int H = a.H, r0 = seg * RS;
    const bool vec = a.gate == 2;
    const int64_t rs = vec ? (int64_t)H * K : H;  // row stride, elements
    const float* gb = vec ? a.g + (t0 * H + h) * K : a.g + t0 * H + h;
    const GBuf b = gbuf(gb, a.gate == 0 ? 0u : tile_bytes<float>(n, rs, vec ? KC : 1));
    const uint32_t rb = (uint32_t)(rs * 4), base = (uint32_t)r0 * rb + (vec ? c : 0) * 4;
#pragma unroll
    for (int r = 0; r < RS; ++r) {
      const uint2 x = gld8(b, base + r * rb);
      G[r] = __uint_as_float(x.x);
      odd.G[r] = __uint_as_float(vec ? x.y : x.x);
    }
  }
  // The gate formed in the kernel: the pre-activation x [.., K] (type X) of
  // this thread's column (features [0, KC), KC = K) and rows, raw bits kept
  // in G until kda_gate(); rows past the end read as zero.
  template <typename X>
  __device__ __forceinline__ void load_x(const Args& a, int64_t t0, int h, int n, int K) {
    const int H = a.H, r0 = seg * RS;
    const int64_t rs = (int64_t)H * K;
    const GBuf b = gbuf(reinterpret_cast<const X*>(a.gx) + (t0 * H + h) * K, tile_bytes<X>(n, rs, KC));
    const uint32_t rb = (uint32_t)(rs * (int64_t)sizeof(X)), base = (uint32_t)r0 * rb + c * (uint32_t)sizeof(X);
#pragma unroll
    for (int r = 0; r < RS; ++r)
      G[r] = __uint_as_float(sizeof(X) == 2 ? gld2(b, base + r * rb) : gld4(b, base + r * rb));
  }
  // x of a column pair (as load_pair), one 4-byte (bf16) or 8-byte (fp32)
  // load per row; raw bits kept in G until kda_gate()
  template <typename X>
  __device__ __forceinline__ void load_x_pair(GateCols& odd, const Args& a, int64_t t0, int h, int n, int K) {
    const int H = a.H, r0 = seg * RS;
    const int64_t rs = (int64_t)H * K;
    const GBuf b = gbuf(reinterpret_cast<const X*>(a.gx) + (t0 * H + h) * K, tile_bytes<X>(n, rs, KC));
    const uint32_t rb = (uint32_t)(rs * (int64_t)sizeof(X)), base = (uint32_t)r0 * rb + c * (uint32_t)sizeof(X);
#pragma unroll
    for (int r = 0; r < RS; ++r) {
      if constexpr (sizeof(X) == 2) {
        const uint32_t x = gld4(b, base + r * rb);
        G[r] = __uint_as_float(x & 0xffffu);
        odd.G[r] = __uint_as_float(x >> 16);
      } else {
        const uint2 x = gld8(b, base + r * rb);
        G[r] = __uint_as_float(x.x);
        odd.G[r] = __uint_as_float(x.y);
      }
    }
  }
  // g = -ea softplus(x + dtb) (lb = 0; GDN2 spec section 4.4) or the
  // bounded form g = lb sigmoid(ea (x + dtb)) (lb < 0; GDN2 spec section 3),
  // ea = exp(A_log) of the head, dtb = dt_bias of this column; rows past the
  // end are masked later
  template <typename X>
  __device__ __forceinline__ void kda_gate(float ea, float dtb, float lb) {
    auto zr = [&](int r) {
      const uint32_t u = __float_as_uint(G[r]);
      return (sizeof(X) == 2 ? __uint_as_float(u << 16) : __uint_as_float(u)) + dtb;
    };
    if (lb == 0.f) {  // uniform: one form per launch
#pragma unroll
      for (int r = 0; r < RS; ++r) G[r] = -ea * softplus(zr(r));
    } else {
#pragma unroll
      for (int r = 0; r < RS; ++r) G[r] = lb * sigmoid_f(ea * zr(r));
    }
  }
  // G2 = log2(e) * inclusive prefix over the chunk's n rows (rows past the end
  // add zero), in two halves around a barrier the caller places:
  // prefix_local() publishes the segment totals in sTot [NSUB][KC],
  // prefix_finish() adds the totals of earlier segments.
  // MASK: zero the rows past the end first (a gate formed from x, which is
  // nonzero there); a loaded g already reads as zero past the end.
  template <bool MASK>
  __device__ __forceinline__ void prefix_local(float* sTot, int n) {
    if constexpr (MASK)
#pragma unroll
      for (int r = 0; r < RS; ++r) G[r] = seg * RS + r < n ? G[r] : 0.f;
#pragma unroll
    for (int r = 1; r < RS; ++r) G[r] += G[r - 1];
    if (on) sTot[seg * KC + c] = G[RS - 1];
  }
  __device__ __forceinline__ void prefix_finish(const float* sTot) {
    float off = 0.f;
    if (on)
      for (int s = 0; s < seg; ++s) off += sTot[s * KC + c];
#pragma unroll
    for (int r = 0; r < RS; ++r) G[r] = (G[r] + off) * LOG2E;
  }
};

// Sub-chunk statistics from the register-resident prefix sums: midpoint, first
// row and last valid row per (J, feature) into sMid/sGf/sGl [NSUB][KC], G2 at
// the chunk's last valid row into sGn [KC], and sFlag[J][fb] (16-feature
// block fb, [NSUB][KC/16]) set when a feature of the block ranges over more
// than CENTRE_MAX_RANGE (sFlag zero on entry).  With gst non-null the
// record {first, last, midpoint, range} of every non-empty (J, feature) is also
// written to gst[J * KC + feature].  No barrier inside.
template <int KC>
__device__ __forceinline__ void subchunk_stats_regs(const GateCols<KC>& gc, int n, float* sMid,
                                                    float* sGf, float* sGl, float* sGn,
                                                    int* sFlag, f32x4* gst) {
  if (!gc.on) return;
  const int J = gc.seg, r0 = J * SUB;
  if (r0 >= n) return;
  const int last = min(r0 + SUB, n) - 1;
  // Rows past the chunk's end repeat the last valid row's G (the prefix adds
  // zeros there), so the extremes over all 16 rows are those over the valid
  // rows, and the last row holds the last valid value.  The extremes use
  // med3 against an infinity: the same max and min of two finite values
  // without the NaN quieting fmaxf/fminf add to each input.
  float mx = gc.G[0], mn = gc.G[0];
#pragma unroll
  for (int r = 1; r < SUB; ++r) {
    mx = __builtin_amdgcn_fmed3f(gc.G[r], mx, INFINITY);
    mn = __builtin_amdgcn_fmed3f(gc.G[r], mn, -INFINITY);
  }
  const float gl = gc.G[SUB - 1];
  const int idx = J * KC + gc.c;
  sMid[idx] = 0.5f * (mx + mn);
  sGf[idx] = gc.G[0];
  sGl[idx] = gl;
  if (last == n - 1) sGn[gc.c] = gl;
  if (mx - mn > CENTRE_MAX_RANGE) sFlag[J * (KC / SUB) + gc.c / SUB] = 1;  // benign race: same value
  if (gst) gst[idx] = f32x4{gc.G[0], gl, 0.5f * (mx + mn), mx - mn};
}

// References of sub-chunk J for feature k (after the statistics are visible).
__device__ __forceinline__ float ref_recv(const float* sMid, const float* sGf, const int* sFlag,
                                          int J, int KC, int k) {
  return sFlag[J * (KC / SUB) + k / SUB] ? sGf[J * KC + k] : sMid[J * KC + k];
}
__device__ __forceinline__ float ref_send(const float* sMid, const float* sGl, const int* sFlag,
                                          int J, int KC, int k) {
  return sFlag[J * (KC / SUB) + k / SUB] ? sGl[J * KC + k] : sMid[J * KC + k];
}

// Sub-chunk J has a wide feature block (some feature ranges over more than
// CENTRE_MAX_RANGE).
__device__ __forceinline__ bool flagged(const int* sFlag, int J, int nfb) {
  int any = 0;
  for (int b = 0; b < nfb; ++b) any |= sFlag[J * nfb + b];
  return any != 0;
}

// Pair factors fac[p][KC] = exp2(rA_I - rB_J) for the 10 pairs I >= J (pair_ij
// order).  On a diagonal pair: 1 for a feature of a centred block and 0 for a
// feature of a wide block, whose terms the pairwise sum supplies instead.
template <int KC>
__device__ __forceinline__ void pair_factors(const float* sMid, const float* sGf,
                                             const float* sGl, const int* sFlag, float* fac,
                                             int n, int tid, int nthr) {
  for (int idx = tid; idx < 10 * KC; idx += nthr) {
    const int p = idx / KC, k = idx - p * KC;
    int I, J;
    pair_ij(p, I, J);
    float f = 0.f;
    if (I * SUB < n)
      f = (I == J) ? (sFlag[J * (KC / SUB) + k / SUB] ? 0.f : 1.f)
                   : fexp2(ref_recv(sMid, sGf, sFlag, I, KC, k) -
                           ref_send(sMid, sGl, sFlag, J, KC, k));
    fac[idx] = f;
  }
}

// One score tile from pre-scaled operands (natural [token][feature] layout,
// pitch PK, bf16 or fp32), accumulated into accL / accC:
// L_IJ += Ka_I (Kc_J * f_IJ)^T and, with WITH_CQ, Cq_IJ += Qa_I (Kc_J * f_IJ)^T,
// the per-feature pair factor on the sending operand both products share
// (the triangles are cut by the caller).  A diagonal tile skips the factors
// unless `masked` (a flagged diagonal: f is 1 or 0 per feature).  One wave.
template <typename T, int K, bool WITH_CQ>
__device__ __forceinline__ void score_tile(const T* sKa, const T* sQa, const T* sKc, int PK,
                                           const float* f, int I, int J, bool masked,
                                           f32x4& accL, f32x4& accC) {
  constexpr bool BF = std::is_same_v<T, bf16>;
  const int l = lane_id();
  const bool plain = I == J && !masked;
  {
    const int ri = I * SUB + (l & 15), rj = J * SUB + (l & 15);
    for (int k0 = 0; k0 < K; k0 += MM<T>::KS) {
      typename MM<T>::frag ak, aq, bk;
      if constexpr (BF) {
        const int kb = k0 + (l >> 4) * 8;
        ak = *reinterpret_cast<const bf16x8*>(sKa + ri * PK + kb);
        if constexpr (WITH_CQ) aq = *reinterpret_cast<const bf16x8*>(sQa + ri * PK + kb);
        const bf16x8 kc = *reinterpret_cast<const bf16x8*>(sKc + rj * PK + kb);
        if (plain) {
          bk = kc;
        } else {  // the pair factor on the sending operand, which both products share
          const f32x4 f0 = *reinterpret_cast<const f32x4*>(f + kb);
          const f32x4 f1 = *reinterpret_cast<const f32x4*>(f + kb + 4);
#pragma unroll
          for (int e = 0; e < 8; ++e) bk[e] = (bf16)((float)kc[e] * (e < 4 ? f0[e] : f1[e - 4]));
        }
      } else {
        const int kk = k0 + (l >> 4);
        const float fe = plain ? 1.f : f[kk];
        ak = tof(sKa[ri * PK + kk]);
        if constexpr (WITH_CQ) aq = tof(sQa[ri * PK + kk]);
        bk = tof(sKc[rj * PK + kk]) * fe;
      }
      accL = mma(ak, bk, accL);
      if constexpr (WITH_CQ) accC = mma(aq, bk, accC);
    }
  }
}

// All score tiles of the pairs I >= J with rows < n, except the flagged
// diagonals (see pairwise_diag).  The callback st(I, J, accL, accC) receives
// each finished tile.  Called by all NW waves.
template <typename T, int K, bool WITH_CQ, int NW, typename Store>
__device__ __forceinline__ void score_tiles_pre(const T* sKa, const T* sQa, const T* sKc, int PK,
                                                const float* fac, const int* sFlag, int n,
                                                Store&& st) {
  const int w = wave_id();
  for (int p = w; p < 10; p += NW) {
    int I, J;
    pair_ij(p, I, J);
    if (I * SUB >= n || (I == J && flagged(sFlag, J, K / SUB))) continue;
    f32x4 accL = zero4(), accC = zero4();
    score_tile<T, K, WITH_CQ>(sKa, sQa, sKc, PK, fac + p * K, I, J, false, accL, accC);
    st(I, J, accL, accC);
  }
}

// Pairwise part of the diagonal tile of sub-chunk I (one wave): the terms of
// the features in wide 16-feature blocks (wide[fb] != 0),
//   L[i][j]  += beta_i sum_k k_ik k_jk exp2(G_ik - G_jk)      (j < i)
//   Cq[i][j] += s sum_k q_ik k_jk exp2(G_ik - G_jk)            (j <= i)
// with G_i - G_j summed from the raw gates between the two rows, so no factor
// exceeds 1, added to the centred blocks' terms already in accL / accC.  Reads
// q, k, g from global.  Lane l takes column j = l & 15 and the feature quarter
// l >> 4; results come back in the C-fragment layout.
// EW: the erase gate is a vector b (a.beta, [.., K], element type T), taken
// inside the sum over features instead of beta_i outside it.  GIN: the gate
// is formed from its pre-activation (softplus or bounded form, Args::gate_lb).
template <typename T, int K, bool WITH_CQ, bool EW = false, bool GIN = false>
__device__ __forceinline__ void pairwise_diag(const Args& a, int64_t t0, int h, int n, int I,
                                              const float* sBeta, const int* wide, f32x4& accL,
                                              f32x4& accC) {
  const int l = lane_id(), j = l & 15, qk = l >> 4, H = a.H;
  const T* kg = reinterpret_cast<const T*>(a.k);
  const T* qg = reinterpret_cast<const T*>(a.q);
  float pL[SUB], pC[SUB];
#pragma unroll
  for (int i = 0; i < SUB; ++i) pL[i] = pC[i] = 0.f;
  const float ea = GIN ? fexp2(a.a_log[h] * LOG2E) : 0.f;
  const int rj = I * SUB + j;
  if (rj < n) {
    for (int k = qk * (K / 4); k < (qk + 1) * (K / 4); ++k) {
      if (!wide[k / SUB]) continue;  // a centred block: its terms came from the MFMA tile
      const float kj = tof(kg[((t0 + rj) * H + h) * K + k]);
      float run = 0.f;
#pragma unroll
      for (int i = 0; i < SUB; ++i) {
        const int ri = I * SUB + i;
        if (i >= j && ri < n) {
          if (i > j) {
            float gi = 0.f;
            if constexpr (GIN) {
              const float z = tof(reinterpret_cast<const T*>(a.gx)[((t0 + ri) * H + h) * K + k]) +
                              a.dt_bias[(int64_t)h * K + k];
              gi = a.gate_lb == 0.f ? -ea * softplus(z) : a.gate_lb * sigmoid_f(ea * z);
            }
            else if (a.gate == 2) gi = a.g[((t0 + ri) * H + h) * K + k];
            else if (a.gate == 1) gi = a.g[(t0 + ri) * H + h];
            run += gi * LOG2E;
          }
          const float f = fexp2(run) * kj;
          float ki = tof(kg[((t0 + ri) * H + h) * K + k]);
          if constexpr (EW) ki *= tof(reinterpret_cast<const T*>(a.beta)[((t0 + ri) * H + h) * K + k]);
          pL[i] += ki * f;
          if constexpr (WITH_CQ) pC[i] += tof(qg[((t0 + ri) * H + h) * K + k]) * f;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < SUB; ++i) {
    pL[i] += __shfl_xor(pL[i], 16);
    pL[i] += __shfl_xor(pL[i], 32);
    if constexpr (WITH_CQ) {
      pC[i] += __shfl_xor(pC[i], 16);
      pC[i] += __shfl_xor(pC[i], 32);
    }
  }
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4)
    if (qk == g4)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        accL[r] += EW ? pL[4 * g4 + r] : sBeta[I * SUB + 4 * g4 + r] * pL[4 * g4 + r];
        accC[r] += a.scale * pC[4 * g4 + r];
      }
}

}  // namespace rewy
