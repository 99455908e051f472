// Per-chunk building blocks used by more than one chunk-parallel kernel:
// the base-2 in-chunk gate prefix sum, sub-chunk gate statistics, the centred
// intra-chunk score tiles and the blocked unit-lower-triangular inverse.
//
// Notation (ReWY paper, "The chunk system and conventional WY backward" and
// Appendix A): for one chunk of n <= 64 rows and one head,
//   G2 = log2(e) * in-chunk cumulative sum of g      (base-2 gates, KDA blog 6.6)
//   L  = tril_strict(E Y^T),  Cq = tril_incl(Qg Y^T),  A = (I + L)^-1
// with E = beta exp2(G2) K, Y = K exp2(-G2), Qg = s Q exp2(G2).
#pragma once
#include <algorithm>

#include "kernels.hpp"

namespace rewy {

// (I, J) sub-chunk pairs with J <= I; wave w takes pairs w, w+4, w+8.
__device__ __forceinline__ void pair_ij(int p, int& I, int& J) {
  // 0:(0,0) 1:(1,0) 2:(1,1) 3:(2,0) 4:(2,1) 5:(2,2) 6:(3,0) 7:(3,1) 8:(3,2) 9:(3,3)
  I = p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3;
  J = p - (I * (I + 1)) / 2;
}

// Rows [0, 64) of sG (pitch PG, K features) receive G2 for rows < n; rows >= n
// repeat the last valid value (zero increments).  Features [k0, k0 + KC) of the
// gate are read (vector gate), or the per-token scalar is broadcast (scalar
// gate), or zeros (no gate).
template <int KC>
__device__ __forceinline__ void load_gate_cumsum(float* sG, int PG, const Args& a, int64_t t0,
                                                 int h, int n, int K, int k0, int tid, int nthr) {
  const int H = a.H;
  if (a.gate == 2) {
    g2s<float, KC>(sG, PG, a.g + (t0 * H + h) * K + k0, (int64_t)H * K, n, CH, tid, nthr);
  } else {
    for (int idx = tid; idx < CH * KC; idx += nthr) {
      const int i = idx / KC, kk = idx - i * KC;
      sG[i * PG + kk] = (a.gate == 1 && i < n) ? a.g[(t0 + i) * H + h] : 0.f;
    }
  }
  __syncthreads();
  for (int kk = tid; kk < KC; kk += nthr) {
    float run = 0.f;
    for (int i = 0; i < CH; ++i) {
      run += sG[i * PG + kk];
      sG[i * PG + kk] = run * LOG2E;
    }
  }
  __syncthreads();
}

// Per sub-chunk J and feature: first-row value Gf, last-valid-row value Gl and
// the midpoint of the range (max + min) / 2.  sFlag[J] is set when a feature's
// range exceeds CENTRE_MAX_RANGE.  Arrays are [NSUB][KC]; sFlag must be zeroed.
template <int KC>
__device__ __forceinline__ void subchunk_stats(const float* sG, int PG, int n, float* sGf,
                                               float* sGl, float* sMid, int* sFlag, int tid,
                                               int nthr) {
  for (int idx = tid; idx < NSUB * KC; idx += nthr) {
    const int J = idx / KC, kk = idx - J * KC;
    const int r0 = J * SUB;
    float mid = 0.f, gf = 0.f, gl = 0.f;
    if (r0 < n) {
      const int r1 = min(r0 + SUB, n) - 1;
      float mx = -INFINITY, mn = INFINITY;
      for (int i = r0; i <= r1; ++i) {
        const float x = sG[i * PG + kk];
        mx = fmaxf(mx, x);
        mn = fminf(mn, x);
      }
      mid = 0.5f * (mx + mn);
      gf = sG[r0 * PG + kk];
      gl = sG[r1 * PG + kk];
      if (mx - mn > CENTRE_MAX_RANGE) sFlag[J] = 1;  // benign race: same value
    }
    if (sGf) sGf[idx] = gf;
    sGl[idx] = gl;
    sMid[idx] = mid;
  }
}

// Centred score tiles.  L (strict, fp32, pitch PL) gets beta_i <k_i, k_j>
// exp2(G_i - G_j) summed over features; with WITH_CQ, Cq (inclusive, type T,
// pitch PA) gets s <q_i, k_j> exp2(G_i - G_j).  A diagonal tile centres both
// factors on the sub-chunk midpoint; an off-diagonal tile (I > J) references
// the last row of sub-chunk J, so both factors are <= 1 for a decaying gate.
// A diagonal sub-chunk flagged in sFlag is evaluated pairwise.  L and Cq must
// be zero outside the tiles written here.  Called by all four waves.
template <typename T, int K, bool WITH_CQ>
__device__ __forceinline__ void score_tiles(const float* sG, int PG, const T* sK, const T* sQ,
                                            int PK, const float* sBeta, const float* sMid,
                                            const float* sGl, const int* sFlag, int n,
                                            float scale, float* sL, int PL, T* sCq, int PA) {
  constexpr bool BF = std::is_same_v<T, bf16>;
  const int w = wave_id(), l = lane_id();
  for (int p = w; p < 10; p += 4) {
    int I, J;
    pair_ij(p, I, J);
    if (I * SUB >= n) continue;
    const bool diag = (I == J);
    if (diag && sFlag[J]) {
      for (int e = l; e < SUB * SUB; e += 64) {
        const int ii = e / SUB, jj = e - ii * SUB;
        if (jj > ii) continue;
        const int ri = I * SUB + ii, rj = I * SUB + jj;
        float sl = 0.f, sc = 0.f;
        for (int kk = 0; kk < K; ++kk) {
          const float kj = tof(sK[rj * PK + kk]) * exp2f(sG[ri * PG + kk] - sG[rj * PG + kk]);
          sl += tof(sK[ri * PK + kk]) * kj;
          if constexpr (WITH_CQ) sc += tof(sQ[ri * PK + kk]) * kj;
        }
        if (jj < ii) sL[ri * PL + rj] = sBeta[ri] * sl;
        if constexpr (WITH_CQ) sCq[ri * PA + rj] = fromf<T>(scale * sc);
      }
      continue;
    }
    const float* ref = diag ? sMid + J * K : sGl + J * K;
    const int ri = I * SUB + (l & 15);
    const int rj = J * SUB + (l & 15);
    const float bi = sBeta[ri];
    f32x4 accL = zero4(), accC = zero4();
    for (int k0 = 0; k0 < K; k0 += MM<T>::KS) {
      typename MM<T>::frag ak, aq, bk;
      if constexpr (BF) {
        const int kb = k0 + (l >> 4) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kk = kb + e;
          const float r = ref[kk];
          const float fi = exp2f(sG[ri * PG + kk] - r);
          ak[e] = (bf16)(bi * tof(sK[ri * PK + kk]) * fi);
          if constexpr (WITH_CQ) aq[e] = (bf16)(scale * tof(sQ[ri * PK + kk]) * fi);
          bk[e] = (bf16)(tof(sK[rj * PK + kk]) * exp2f(r - sG[rj * PG + kk]));
        }
      } else {
        const int kk = k0 + (l >> 4);
        const float r = ref[kk];
        const float fi = exp2f(sG[ri * PG + kk] - r);
        ak = bi * tof(sK[ri * PK + kk]) * fi;
        if constexpr (WITH_CQ) aq = scale * tof(sQ[ri * PK + kk]) * fi;
        bk = tof(sK[rj * PK + kk]) * exp2f(r - sG[rj * PG + kk]);
      }
      accL = mma(ak, bk, accL);
      if constexpr (WITH_CQ) accC = mma(aq, bk, accC);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = I * SUB + crow(i), col = J * SUB + ccol();
      if (row > col) sL[row * PL + col] = accL[i];
      if constexpr (WITH_CQ)
        if (row >= col) sCq[row * PA + col] = fromf<T>(accC[i]);
    }
  }
}

// A = (I + L)^-1 for the strictly lower fp32 L (pitch PL); A must be zero on
// entry (its upper blocks stay zero).  Diagonal 16x16 blocks are inverted by
// forward substitution (one lane per column), then the off-diagonal blocks are
// merged in order of distance from the diagonal,
//   A_IJ = -A_II * sum_{m=J}^{I-1} L_Im A_mJ,
// with fp32 MFMA.  sT: 4 x 16 x 20 fp32 scratch.  Called by all four waves.
__device__ __forceinline__ void solve_unit_lower(const float* sL, float* sA, int PL, float* sT,
                                                 int n) {
  const int w = wave_id(), l = lane_id();
  if (w == 0) {
    const int b = l >> 4, cc = l & 15;
    const float* Lb = sL + (b * SUB) * PL + b * SUB;
    float x[SUB];
#pragma unroll
    for (int i = 0; i < SUB; ++i) x[i] = (i == cc) ? 1.f : 0.f;
#pragma unroll
    for (int i = 1; i < SUB; ++i) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s += Lb[i * PL + m] * x[m];
      if (i > cc) x[i] = -s;
    }
    float* Ab = sA + (b * SUB) * PL + b * SUB;
#pragma unroll
    for (int i = 0; i < SUB; ++i) Ab[i * PL + cc] = x[i];
  }
  __syncthreads();
  for (int d = 1; d < NSUB; ++d) {
    const int I = w + d, J = w;
    const bool act = (w < NSUB - d) && (I * SUB < n);
    float* Ts = sT + w * SUB * 20;
    if (act) {
      f32x4 t = zero4();
      mma_tile<float, false, false>(t, sL + (I * SUB) * PL + J * SUB, PL, 1,
                                    sA + (J * SUB) * PL + J * SUB, 1, PL, SUB * d);
      st_tile<float>(t, Ts, 20, 1);
    }
    __syncthreads();
    if (act) {
      f32x4 t = zero4();
      mma_tile<float, false, false>(t, sA + (I * SUB) * PL + I * SUB, PL, 1, Ts, 1, 20, SUB);
      st_tile<float>(-t, sA + (I * SUB) * PL + J * SUB, PL, 1);
    }
    __syncthreads();
  }
}

constexpr int cmax(int x, int y) { return x > y ? x : y; }

// Workgroups of a persistent chunk kernel: one per compute unit of the
// current device (queried once per device).
inline int persistent_grid() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
      cu = 256;
    cached[dev] = cu;
  }
  return cached[dev];
}

// Launch helper: the (T, K, V) instantiations this build provides.  fp32 keeps
// K, V <= 64 so that every kernel's LDS stays within one CU's 160 KB.
template <typename T, int K, int V>
constexpr bool kv_ok() {
  return std::is_same_v<T, bf16> || (K <= 64 && V <= 64);
}

#define REWY_KV_CASE(KERNEL, K_, V_)                                              \
  case K_ * 1000 + V_:                                                            \
    if constexpr (kv_ok<T, K_, V_>()) {                                           \
      hipLaunchKernelGGL((KERNEL<T, K_, V_>), grid, block, 0, s, a);              \
      return hipGetLastError();                                                   \
    } else {                                                                      \
      return hipErrorInvalidValue;                                                \
    }

#define REWY_KV_SWITCH(KERNEL)                                                    \
  switch (a.K * 1000 + a.V) {                                                     \
    REWY_KV_CASE(KERNEL, 32, 32)                                                  \
    REWY_KV_CASE(KERNEL, 32, 64)                                                  \
    REWY_KV_CASE(KERNEL, 32, 128)                                                 \
    REWY_KV_CASE(KERNEL, 64, 32)                                                  \
    REWY_KV_CASE(KERNEL, 64, 64)                                                  \
    REWY_KV_CASE(KERNEL, 64, 128)                                                 \
    REWY_KV_CASE(KERNEL, 128, 32)                                                 \
    REWY_KV_CASE(KERNEL, 128, 64)                                                 \
    REWY_KV_CASE(KERNEL, 128, 128)                                                \
    default:                                                                      \
      return hipErrorInvalidValue;                                                \
  }

}  // namespace rewy
