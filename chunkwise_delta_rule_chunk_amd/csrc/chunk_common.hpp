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
// forward substitution (one lane per column), then the 32x32 halves and the
// whole 64x64 inverse follow from the 2 x 2 block formula
//   [M11 0; M21 M22]^-1 = [A11 0; -A22 M21 A11  A22]
// with fp32 MFMA: first A_10 and A_32 (two waves), then the four blocks of
// the lower-left 32x32 quarter (one wave each, forming the products
// T_kj = sum_m L_{2+k,m} A_mj it needs itself).  Every operand of a product is
// read from LDS before its MFMAs; a C fragment is used directly as the B
// operand of the next product.  Three barriers.  Called by every wave of the
// workgroup.
__device__ __forceinline__ void solve_unit_lower(const float* sL, float* sA, int PL, int n) {
  const int w = wave_id(), l = lane_id(), g = l >> 4, r16 = l & 15;
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
  // operands of a 16-long fp32 contraction: the A operand is four consecutive
  // columns of row r16, the B operand four consecutive rows of column r16
  auto arow = [&](const float* m, int I, int J) {
    return *reinterpret_cast<const f32x4*>(m + (I * SUB + r16) * PL + J * SUB + 4 * g);
  };
  auto bcol = [&](const float* m, int I, int J) {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = m[(I * SUB + 4 * g + e) * PL + J * SUB + r16];
    return v;
  };
  // A_{b+1,b} = -A_{b+1,b+1} L_{b+1,b} A_{b,b}, b = 0 (wave 0) and b = 2 (wave 1)
  if (w < 2 && (2 * w + 1) * SUB < n) {
    const int b = 2 * w;
    const f32x4 la = arow(sL, b + 1, b), ab = bcol(sA, b, b), aa = arow(sA, b + 1, b + 1);
    f32x4 t = zero4(), r = zero4();
    mm16(t, la, ab);
    mm16(r, aa, t);
    st_tile<float>(-r, sA + ((b + 1) * SUB) * PL + b * SUB, PL, 1);
  }
  lds_barrier();
  // block (2 + i, j) of A, wave 2 i + j: -sum_{k <= i} A_{2+i,2+k} T_kj
  {
    const int i = w >> 1, j = w & 1;
    if ((2 + i) * SUB < n) {
      f32x4 R = zero4();
      static_for<0, 2>([&](auto kk) {
        constexpr int k = decltype(kk)::value;
        if (k > i) return;
        const f32x4 l0 = arow(sL, 2 + k, 0), l1 = arow(sL, 2 + k, 1), a2 = arow(sA, 2 + i, 2 + k);
        const f32x4 b0 = bcol(sA, 0, j), b1 = bcol(sA, 1, j);
        f32x4 T = zero4();
        if (j == 0) mm16(T, l0, b0);  // m = 0 (A_0j is zero for j = 1)
        mm16(T, l1, b1);              // m = 1
        mm16(R, a2, T);
      });
      st_tile<float>(-R, sA + ((2 + i) * SUB) * PL + j * SUB, PL, 1);
    }
  }
  lds_barrier();
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
