// The two serial inter-chunk scans.  One workgroup per (sequence, head, value
// tile of BV columns) walks the sequence's chunks in order; the fp32 state
// tile [K x BV] stays in MFMA accumulator registers for the whole walk.
// Grid = (N*H, V/BV): consecutive workgroup ids, which the dispatcher spreads
// round-robin over the 8 XCDs, give the value tiles of one (sequence, head)
// the same XCD and L2 whenever N*H is a multiple of 8.
//
// Each step's operand tiles are prefetched one chunk ahead: the global reads
// for chunk c+1 are issued before chunk c's products and land in the other LDS
// buffer after them, so a step waits only on its two barriers.
//
// Forward (ReWY paper, "The chunk system": R = U - W S, S' = Lambda S + F^T R;
// KDA blog section 6.4 state fast-forward):
//   for each chunk c:  write S_c;  R_c = U_c - W_c S_c;  S_{c+1} = diag(exp2 G2_last) S_c + F_c^T R_c
// Reverse (ReWY paper Appendix 7.2 / Algorithm 1; the scan supplies the
// incoming-state term -E^T P = -W^T Rbar once):
//   for each chunk c from the last:  write dS_{c+1};
//     Rbar_c = F_c dS_{c+1} + Cq_c^T dO_c
//     dS_c   = diag(exp2 G2_last) dS_{c+1} + Qg_c^T dO_c - W_c^T Rbar_c
#include "chunk_common.hpp"

namespace rewy {

template <int K, int BV>
struct ScanShape {
  static constexpr int CT = BV / SUB;             // column tiles of the state
  static constexpr int TPW = (K / SUB) * CT / 4;  // state tiles per wave
  static constexpr int RPW = (CH / SUB) * CT / 4; // R tiles per wave
  static_assert(TPW >= 1 && RPW >= 1, "tile split");
};

template <typename T, int K, int V, int BV>
__global__ __launch_bounds__(256) void k_fwd_scan(Args a) {
  using S = ScanShape<K, BV>;
  constexpr int CT = S::CT, NTH = 256;
  constexpr int PK = pitch<T>(K), PU = pitch<T>(BV), PA = pitch<T>(CH);
  __shared__ __align__(16) T sW[2][CH * PK];
  __shared__ __align__(16) T sFt[2][K * PA];
  __shared__ __align__(16) T sU[2][CH * PU];
  __shared__ __align__(16) float sGl[2][K];
  __shared__ __align__(16) T sHt[BV * PK];  // state as operand, [v][k]
  __shared__ __align__(16) T sRt[BV * PA];  // R as operand, [v][i]

  const int H = a.H;
  const int u = blockIdx.x, vt = blockIdx.y;
  const int n = u / H, h = u - n * H;
  const int w = wave_id(), tid = threadIdx.x;
  const int64_t gsK = (int64_t)H * K, gsV = (int64_t)H * V;
  const int c0 = a.seqoff[n], c1 = a.seqoff[n + 1];
  const T* Wg = reinterpret_cast<const T*>(a.W);
  const T* Ftg = reinterpret_cast<const T*>(a.Ft);
  const T* Ug = reinterpret_cast<const T*>(a.U);

  Staged<T, CH, K, NTH> pW;
  Staged<T, K, CH, NTH> pF;
  Staged<T, CH, BV, NTH> pU;
  Staged<float, 1, K, NTH> pL;
  auto fetch = [&](int c) {
    const ChunkInfo ci = a.chunks[c];
    const int64_t t0 = ci.bos, cb = (int64_t)c * H + h;
    pW.load(Wg + (t0 * H + h) * K, gsK, ci.len, tid);
    pF.load(Ftg + cb * K * CH, CH, K, tid);
    pU.load(Ug + (t0 * H + h) * V + vt * BV, gsV, ci.len, tid);
    pL.load(a.glast + cb * K, K, 1, tid);
  };
  auto put = [&](int b) {
    pW.store(sW[b], PK, tid);
    pF.store(sFt[b], PA, tid);
    pU.store(sU[b], PU, tid);
    pL.store(sGl[b], K, tid);
  };

  f32x4 st[S::TPW];
#pragma unroll
  for (int s = 0; s < S::TPW; ++s) {
    const int t = w + 4 * s, tk = t / CT, tv = t - tk * CT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = tk * SUB + crow(i), vv = vt * BV + tv * SUB + ccol();
      st[s][i] = a.h0 ? a.h0[(((int64_t)n * H + h) * K + kk) * V + vv] : 0.f;
    }
  }
  if (c0 < c1) {
    fetch(c0);
    put(0);
  }
  for (int c = c0; c < c1; ++c) {
    const int b = (c - c0) & 1;
    const ChunkInfo ci = a.chunks[c];
    const int len = ci.len;
    const int64_t t0 = ci.bos;
    if (c + 1 < c1) fetch(c + 1);
    T* hb = reinterpret_cast<T*>(a.hbuf) + ((int64_t)c * H + h) * K * V + vt * BV;
#pragma unroll
    for (int s = 0; s < S::TPW; ++s) {
      const int t = w + 4 * s, tk = t / CT, tv = t - tk * CT;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = tk * SUB + crow(i), vv = tv * SUB + ccol();
        const T x = fromf<T>(st[s][i]);
        hb[(int64_t)kk * V + vv] = x;
        sHt[vv * PK + kk] = x;
      }
    }
    lds_barrier();
    // R = U - W S
    T* Rg = reinterpret_cast<T*>(a.R) + (t0 * H + h) * V + vt * BV;
#pragma unroll
    for (int r = 0; r < S::RPW; ++r) {
      const int t = w + 4 * r, ti = t / CT, tv = t - ti * CT;
      f32x4 p = zero4();
      mma_tile<T, true, true>(p, sW[b] + ti * SUB * PK, PK, 1, sHt + tv * SUB * PK, PK, 1, K);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = ti * SUB + crow(i), col = tv * SUB + ccol();
        const T rv = fromf<T>(tof(sU[b][row * PU + col]) - p[i]);
        if (row < len) Rg[row * gsV + col] = rv;
        sRt[col * PA + row] = rv;
      }
    }
    lds_barrier();
    // S = diag(exp2 G2_last) S + F^T R
#pragma unroll
    for (int s = 0; s < S::TPW; ++s) {
      const int t = w + 4 * s, tk = t / CT, tv = t - tk * CT;
#pragma unroll
      for (int i = 0; i < 4; ++i) st[s][i] *= fexp2(sGl[b][tk * SUB + crow(i)]);
      mma_tile<T, true, true>(st[s], sFt[b] + tk * SUB * PA, PA, 1, sRt + tv * SUB * PA, PA, 1, CH);
    }
    if (c + 1 < c1) put(b ^ 1);
  }
  if (a.ht) {
#pragma unroll
    for (int s = 0; s < S::TPW; ++s) {
      const int t = w + 4 * s, tk = t / CT, tv = t - tk * CT;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = tk * SUB + crow(i), vv = vt * BV + tv * SUB + ccol();
        a.ht[(((int64_t)n * H + h) * K + kk) * V + vv] = st[s][i];
      }
    }
  }
}

template <typename T, int K, int V, int BV>
__global__ __launch_bounds__(256) void k_bwd_scan(Args a) {
  using S = ScanShape<K, BV>;
  constexpr int CT = S::CT, NTH = 256;
  constexpr int PK = pitch<T>(K), PA = pitch<T>(CH);
  __shared__ __align__(16) T sF[2][CH * PK];
  __shared__ __align__(16) T sWt[2][K * PA];
  __shared__ __align__(16) T sQgt[2][K * PA];
  __shared__ __align__(16) T sCqt[2][CH * PA];
  __shared__ __align__(16) T sdOt[2][BV * PA];  // dO as operand, [v][j]
  __shared__ __align__(16) float sGl[2][K];
  __shared__ __align__(16) T sDt[BV * PK];      // dS_{c+1} as operand, [v][k]
  __shared__ __align__(16) T sRbt[BV * PA];     // -Rbar as operand, [v][i]

  const int H = a.H;
  const int u = blockIdx.x, vt = blockIdx.y;
  const int n = u / H, h = u - n * H;
  const int w = wave_id(), tid = threadIdx.x;
  const int64_t gsK = (int64_t)H * K, gsV = (int64_t)H * V;
  const int c0 = a.seqoff[n], c1 = a.seqoff[n + 1];

  Staged<T, CH, K, NTH> pF;
  Staged<T, K, CH, NTH> pW;
  Staged<T, K, CH, NTH> pQ;
  Staged<T, CH, CH, NTH> pC;
  Staged<T, CH, BV, NTH> pO;
  Staged<float, 1, K, NTH> pL;
  auto fetch = [&](int c) {
    const ChunkInfo ci = a.chunks[c];
    const int64_t t0 = ci.bos, cb = (int64_t)c * H + h;
    pF.load(reinterpret_cast<const T*>(a.F) + (t0 * H + h) * K, gsK, ci.len, tid);
    pW.load(reinterpret_cast<const T*>(a.Wt) + cb * K * CH, CH, K, tid);
    pQ.load(reinterpret_cast<const T*>(a.Qgt) + cb * K * CH, CH, K, tid);
    pC.load(reinterpret_cast<const T*>(a.Cqt) + cb * CH * CH, CH, CH, tid);
    pO.load(reinterpret_cast<const T*>(a.dO) + (t0 * H + h) * V + vt * BV, gsV, ci.len, tid);
    pL.load(a.glast + cb * K, K, 1, tid);
  };
  auto put = [&](int b) {
    pF.store(sF[b], PK, tid);
    pW.store(sWt[b], PA, tid);
    pQ.store(sQgt[b], PA, tid);
    pC.store(sCqt[b], PA, tid);
    pO.store_T(sdOt[b], PA, tid);
    pL.store(sGl[b], K, tid);
  };

  f32x4 st[S::TPW];
#pragma unroll
  for (int s = 0; s < S::TPW; ++s) {
    const int t = w + 4 * s, tk = t / CT, tv = t - tk * CT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = tk * SUB + crow(i), vv = vt * BV + tv * SUB + ccol();
      st[s][i] = a.dht ? a.dht[(((int64_t)n * H + h) * K + kk) * V + vv] : 0.f;
    }
  }
  if (c0 < c1) {
    fetch(c1 - 1);
    put(0);
  }
  for (int c = c1 - 1; c >= c0; --c) {
    const int b = (c1 - 1 - c) & 1;
    const ChunkInfo ci = a.chunks[c];
    const int len = ci.len;
    const int64_t t0 = ci.bos;
    if (c - 1 >= c0) fetch(c - 1);
    T* db = reinterpret_cast<T*>(a.dhbuf) + ((int64_t)c * H + h) * K * V + vt * BV;
#pragma unroll
    for (int s = 0; s < S::TPW; ++s) {
      const int t = w + 4 * s, tk = t / CT, tv = t - tk * CT;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = tk * SUB + crow(i), vv = tv * SUB + ccol();
        const T x = fromf<T>(st[s][i]);
        db[(int64_t)kk * V + vv] = x;
        sDt[vv * PK + kk] = x;
      }
    }
    lds_barrier();
    // Rbar = F dS+ + Cq^T dO
    T* Rbt = reinterpret_cast<T*>(a.Rbt) + ((int64_t)c * H + h) * V * CH + vt * BV * CH;
#pragma unroll
    for (int r = 0; r < S::RPW; ++r) {
      const int t = w + 4 * r, ti = t / CT, tv = t - ti * CT;
      f32x4 acc = zero4();
      mma_tile<T, true, true>(acc, sF[b] + ti * SUB * PK, PK, 1, sDt + tv * SUB * PK, PK, 1, K);
      mma_tile<T, true, true>(acc, sCqt[b] + ti * SUB * PA, PA, 1, sdOt[b] + tv * SUB * PA, PA, 1,
                              CH);
      // rows past the chunk's end are exact zeros (F and Cq vanish there)
      st_tile_T<T>(acc, Rbt + (tv * SUB) * CH + ti * SUB, CH);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = ti * SUB + crow(i), col = tv * SUB + ccol();
        sRbt[col * PA + row] = fromf<T>(-acc[i]);
      }
    }
    lds_barrier();
    // dS = diag(exp2 G2_last) dS+ + Qg^T dO - W^T Rbar
#pragma unroll
    for (int s = 0; s < S::TPW; ++s) {
      const int t = w + 4 * s, tk = t / CT, tv = t - tk * CT;
#pragma unroll
      for (int i = 0; i < 4; ++i) st[s][i] *= fexp2(sGl[b][tk * SUB + crow(i)]);
      mma_tile<T, true, true>(st[s], sQgt[b] + tk * SUB * PA, PA, 1, sdOt[b] + tv * SUB * PA, PA,
                              1, CH);
      mma_tile<T, true, true>(st[s], sWt[b] + tk * SUB * PA, PA, 1, sRbt + tv * SUB * PA, PA, 1,
                              CH);
    }
    if (c - 1 >= c0) put(b ^ 1);
  }
  if (a.dh0) {
#pragma unroll
    for (int s = 0; s < S::TPW; ++s) {
      const int t = w + 4 * s, tk = t / CT, tv = t - tk * CT;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = tk * SUB + crow(i), vv = vt * BV + tv * SUB + ccol();
        a.dh0[(((int64_t)n * H + h) * K + kk) * V + vv] = st[s][i];
      }
    }
  }
}

int scan_bv(const Args& a, int f32) {
  if (a.K == 32) return 32;  // four waves need K * BV >= 1024
  if (f32) return 16;        // keeps the fp32 double buffers within LDS
  // 32-wide tiles when they still give at least one workgroup per CU
  return (int64_t)a.N * a.H * (a.V / 32) >= 256 ? 32 : 16;
}

template <typename T, int BV>
static hipError_t fwd_scan_bv(const Args& a, hipStream_t s) {
  const dim3 grid(a.N * a.H, a.V / BV), block(256);
#define REWY_SCAN_CASE(K_, V_)                                                  \
  case K_ * 1000 + V_:                                                          \
    if constexpr (kv_ok<T, K_, V_>() && V_ >= BV && K_ * BV >= 1024 && \
                  (sizeof(T) == 2 || K_ == 32 || BV == 16)) {                             \
      hipLaunchKernelGGL((k_fwd_scan<T, K_, V_, BV>), grid, block, 0, s, a);    \
      return hipGetLastError();                                                 \
    } else {                                                                    \
      return hipErrorInvalidValue;                                              \
    }
  switch (a.K * 1000 + a.V) {
    REWY_SCAN_CASE(32, 32) REWY_SCAN_CASE(32, 64) REWY_SCAN_CASE(32, 128)
    REWY_SCAN_CASE(64, 32) REWY_SCAN_CASE(64, 64) REWY_SCAN_CASE(64, 128)
    REWY_SCAN_CASE(128, 32) REWY_SCAN_CASE(128, 64) REWY_SCAN_CASE(128, 128)
    default: return hipErrorInvalidValue;
  }
#undef REWY_SCAN_CASE
}

template <typename T, int BV>
static hipError_t bwd_scan_bv(const Args& a, hipStream_t s) {
  const dim3 grid(a.N * a.H, a.V / BV), block(256);
#define REWY_SCAN_CASE(K_, V_)                                                  \
  case K_ * 1000 + V_:                                                          \
    if constexpr (kv_ok<T, K_, V_>() && V_ >= BV && K_ * BV >= 1024 && \
                  (sizeof(T) == 2 || K_ == 32 || BV == 16)) {                             \
      hipLaunchKernelGGL((k_bwd_scan<T, K_, V_, BV>), grid, block, 0, s, a);    \
      return hipGetLastError();                                                 \
    } else {                                                                    \
      return hipErrorInvalidValue;                                              \
    }
  switch (a.K * 1000 + a.V) {
    REWY_SCAN_CASE(32, 32) REWY_SCAN_CASE(32, 64) REWY_SCAN_CASE(32, 128)
    REWY_SCAN_CASE(64, 32) REWY_SCAN_CASE(64, 64) REWY_SCAN_CASE(64, 128)
    REWY_SCAN_CASE(128, 32) REWY_SCAN_CASE(128, 64) REWY_SCAN_CASE(128, 128)
    default: return hipErrorInvalidValue;
  }
#undef REWY_SCAN_CASE
}

hipError_t launch_fwd_scan(const Args& a, int f32, hipStream_t s) {
  const bool w32 = scan_bv(a, f32) == 32;
  if (f32) return w32 ? fwd_scan_bv<float, 32>(a, s) : fwd_scan_bv<float, 16>(a, s);
  return w32 ? fwd_scan_bv<bf16, 32>(a, s) : fwd_scan_bv<bf16, 16>(a, s);
}
hipError_t launch_bwd_scan(const Args& a, int f32, hipStream_t s) {
  const bool w32 = scan_bv(a, f32) == 32;
  if (f32) return w32 ? bwd_scan_bv<float, 32>(a, s) : bwd_scan_bv<float, 16>(a, s);
  return w32 ? bwd_scan_bv<bf16, 32>(a, s) : bwd_scan_bv<bf16, 16>(a, s);
}

}  // namespace rewy
