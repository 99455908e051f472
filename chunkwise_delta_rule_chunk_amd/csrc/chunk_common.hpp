// Per-chunk building blocks of the chunk-parallel kernels: the sub-chunk pair
// order, the blocked unit-lower-triangular inverse and the launch helpers.
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

// A = (I + L)^-1 for the strictly lower fp32 L (pitch PL); A must be zero on
// entry (its upper blocks stay zero).  Diagonal 16x16 blocks are inverted by
// forward substitution (one lane per column), then the off-diagonal blocks are
// merged in order of distance from the diagonal,
//   A_IJ = -A_II * sum_{m=J}^{I-1} L_Im A_mJ,
// with fp32 MFMA.  Called by every wave of the workgroup (waves 0 .. 2 do the
// merges).
__device__ __forceinline__ void solve_unit_lower(const float* sL, float* sA, int PL, int n) {
  const int w = wave_id(), l = lane_id();
  if (w == 0) {
    const int b = l >> 4, cc = l & 15;
    const float* Lb = sL + (b * SUB) * PL + b * SUB;
    float x[SUB];
#pragma unroll
    for (int i = 0; i < SUB; ++i) x[i] = (i == cc) ? 1.f : 0.f;
    // column-oriented substitution: once x[m] is final, its term leaves every
    // later row at once (15 dependent steps instead of a chain per row)
#pragma unroll
    for (int m = 0; m < SUB - 1; ++m)
#pragma unroll
      for (int i = m + 1; i < SUB; ++i) x[i] -= Lb[i * PL + m] * x[m];
    float* Ab = sA + (b * SUB) * PL + b * SUB;
#pragma unroll
    for (int i = 0; i < SUB; ++i) Ab[i * PL + cc] = x[i];
  }
  lds_barrier();
  // distance d is a compile-time constant, so each product's operand reads
  // are issued together ahead of its MFMA chain.  The inner sum stays in
  // registers: its C fragment (lane l: rows 4 (l >> 4) .. +3 of column l & 15)
  // is the B operand of the outer product with A_II.
  static_for<1, NSUB>([&](auto dd) {
    constexpr int d = decltype(dd)::value;
    const int I = w + d, J = w;
    if ((w < NSUB - d) && (I * SUB < n)) {
      f32x4 t = zero4();
      mma_tile<float, false, false>(t, sL + (I * SUB) * PL + J * SUB, PL, 1,
                                    sA + (J * SUB) * PL + J * SUB, 1, PL, SUB * d);
      const int l = lane_id();
      const f32x4 aII =
          *reinterpret_cast<const f32x4*>(sA + (I * SUB + (l & 15)) * PL + I * SUB + 4 * (l >> 4));
      f32x4 r = zero4();
      mm16(r, aII, t);
      st_tile<float>(-r, sA + (I * SUB) * PL + J * SUB, PL, 1);
    }
    lds_barrier();
  });
}

constexpr int cmax(int x, int y) { return x > y ? x : y; }
constexpr int cmin(int x, int y) { return x < y ? x : y; }

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

// Launch helper: the (T, K, V) instantiations the library provides.  fp32 keeps
// K, V <= 64 so that every kernel's LDS stays within one CU's 160 KB.
template <typename T, int K, int V>
constexpr bool kv_ok() {
  return std::is_same_v<T, bf16> || (K <= 64 && V <= 64);
}

#define REWY_KV_CASE(KERNEL, K_, V_)                                              \
  case K_ * 1000 + V_:                                                            \
    if constexpr (kv_ok<T, K_, V_>()) {                                           \
      REWY_LAUNCH((KERNEL<T, K_, V_>), grid, block, s, a);              \
      return hipGetLastError();                                                   \
    } else {                                                                      \
      return hipErrorInvalidValue;                                                \
    }

// The same with one more template argument after (T, K, V).
#define REWY_KV_CASE_X(KERNEL, X, K_, V_)                                         \
  case K_ * 1000 + V_:                                                            \
    if constexpr (kv_ok<T, K_, V_>()) {                                           \
      REWY_LAUNCH((KERNEL<T, K_, V_, X>), grid, block, s, a);           \
      return hipGetLastError();                                                   \
    } else {                                                                      \
      return hipErrorInvalidValue;                                                \
    }

#define REWY_KV_SWITCH_X(KERNEL, X)                                               \
  switch (a.K * 1000 + a.V) {                                                     \
    REWY_KV_CASE_X(KERNEL, X, 32, 32)                                             \
    REWY_KV_CASE_X(KERNEL, X, 32, 64)                                             \
    REWY_KV_CASE_X(KERNEL, X, 32, 128)                                            \
    REWY_KV_CASE_X(KERNEL, X, 64, 32)                                             \
    REWY_KV_CASE_X(KERNEL, X, 64, 64)                                             \
    REWY_KV_CASE_X(KERNEL, X, 64, 128)                                            \
    REWY_KV_CASE_X(KERNEL, X, 128, 32)                                            \
    REWY_KV_CASE_X(KERNEL, X, 128, 64)                                            \
    REWY_KV_CASE_X(KERNEL, X, 128, 128)                                           \
    default:                                                                      \
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
