// The two serial inter-chunk scans.  One workgroup per (sequence, head, value
// tile of SCAN_BV columns) walks the sequence's chunks in order; the fp32
// state tile [K x BV] stays in MFMA accumulator registers for the whole walk.
// Grid = (N*H, V/BV) so that consecutive workgroup ids, which the dispatcher
// spreads round-robin over the 8 XCDs, give the value tiles of one (sequence,
// head) the same XCD (and L2) whenever N*H is a multiple of 8.
//
// Forward (ReWY paper, "The chunk system": R = U - W S, S' = Lambda S + F^T R;
// KDA blog section 6.4 state fast-forward):
//   for each chunk c:  write S_c;  R_c = U_c - W_c S_c;  S_{c+1} = diag(exp2 G2_last) S_c + F_c^T R_c
// Reverse (ReWY paper Appendix 7.2 / Algorithm 1, the scan supplies -E^T P =
// -W^T Rbar once):
//   for each chunk c from the last:  write dS_{c+1};
//     Rbar_c = Cq_c^T dO_c + F_c dS_{c+1}
//     dS_c   = diag(exp2 G2_last) dS_{c+1} + Qg_c^T dO_c - W_c^T Rbar_c
#include "chunk_common.hpp"

namespace rewy {

template <int K, int V>
struct ScanShape {
  static constexpr int BV = V < SCAN_BV ? V : SCAN_BV;
  static constexpr int NVT = V / BV;
  static constexpr int CT = BV / SUB;          // column tiles of the state
  static constexpr int TPW = (K / SUB) * CT / 4; // state tiles per wave
  static constexpr int RPW = (CH / SUB) * CT / 4; // R tiles per wave
  static_assert(TPW >= 1 && RPW >= 1, "tile split");
};

template <typename T, int K, int V>
__global__ __launch_bounds__(256) void k_fwd_scan(Args a) {
  using S = ScanShape<K, V>;
  constexpr int BV = S::BV, CT = S::CT;
  constexpr int PK = pitch<T>(K), PU = pitch<T>(BV), PA = pitch<T>(CH);
  __shared__ __align__(16) T sW[CH * PK];
  __shared__ __align__(16) T sF[CH * PK];
  __shared__ __align__(16) T sU[CH * PU];
  __shared__ __align__(16) T sHt[BV * PK];  // state as operand, [v][k]
  __shared__ __align__(16) T sRt[BV * PA];  // R as operand, [v][i]
  __shared__ float sLam[K];

  const int H = a.H;
  const int u = blockIdx.x, vt = blockIdx.y;
  const int n = u / H, h = u - n * H;
  const int w = wave_id(), tid = threadIdx.x;
  const int64_t gsK = (int64_t)H * K, gsV = (int64_t)H * V;
  const int c0 = a.seqoff[n], c1 = a.seqoff[n + 1];

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
  for (int c = c0; c < c1; ++c) {
    const ChunkInfo ci = a.chunks[c];
    const int len = ci.len;
    const int64_t t0 = ci.bos;
    g2s<T, K>(sW, PK, reinterpret_cast<const T*>(a.W) + (t0 * H + h) * K, gsK, len, CH, tid, 256);
    g2s<T, K>(sF, PK, reinterpret_cast<const T*>(a.F) + (t0 * H + h) * K, gsK, len, CH, tid, 256);
    g2s<T, BV>(sU, PU, reinterpret_cast<const T*>(a.U) + (t0 * H + h) * V + vt * BV, gsV, len, CH,
               tid, 256);
    for (int kk = tid; kk < K; kk += 256) sLam[kk] = exp2f(a.glast[((int64_t)c * H + h) * K + kk]);
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
    __syncthreads();
    // R = U - W S
    T* Rg = reinterpret_cast<T*>(a.R) + (t0 * H + h) * V + vt * BV;
#pragma unroll
    for (int r = 0; r < S::RPW; ++r) {
      const int t = w + 4 * r, ti = t / CT, tv = t - ti * CT;
      f32x4 p = zero4();
      mma_tile<T, true, true>(p, sW + ti * SUB * PK, PK, 1, sHt + tv * SUB * PK, PK, 1, K);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = ti * SUB + crow(i), col = tv * SUB + ccol();
        const T rv = fromf<T>(tof(sU[row * PU + col]) - p[i]);
        if (row < len) Rg[row * gsV + col] = rv;
        sRt[col * PA + row] = rv;
      }
    }
    __syncthreads();
    // S = diag(exp2 G2_last) S + F^T R
#pragma unroll
    for (int s = 0; s < S::TPW; ++s) {
      const int t = w + 4 * s, tk = t / CT, tv = t - tk * CT;
#pragma unroll
      for (int i = 0; i < 4; ++i) st[s][i] *= sLam[tk * SUB + crow(i)];
      mma_tile<T, false, true>(st[s], sF + tk * SUB, 1, PK, sRt + tv * SUB * PA, PA, 1, CH);
    }
    __syncthreads();
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

template <typename T, int K, int V>
__global__ __launch_bounds__(256) void k_bwd_scan(Args a) {
  using S = ScanShape<K, V>;
  constexpr int BV = S::BV, CT = S::CT;
  constexpr int PK = pitch<T>(K), PU = pitch<T>(BV), PA = pitch<T>(CH);
  __shared__ __align__(16) T sW[CH * PK];
  __shared__ __align__(16) T sF[CH * PK];
  __shared__ __align__(16) T sQg[CH * PK];
  __shared__ __align__(16) T sCq[CH * PA];
  __shared__ __align__(16) T sdO[CH * PU];
  __shared__ __align__(16) T sDt[BV * PK];   // dS_{c+1} as operand, [v][k]
  __shared__ __align__(16) T sRbt[BV * PA];  // -Rbar as operand, [v][i]
  __shared__ float sLam[K];

  const int H = a.H;
  const int u = blockIdx.x, vt = blockIdx.y;
  const int n = u / H, h = u - n * H;
  const int w = wave_id(), tid = threadIdx.x;
  const int64_t gsK = (int64_t)H * K, gsV = (int64_t)H * V;
  const int c0 = a.seqoff[n], c1 = a.seqoff[n + 1];

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
  for (int c = c1 - 1; c >= c0; --c) {
    const ChunkInfo ci = a.chunks[c];
    const int len = ci.len;
    const int64_t t0 = ci.bos;
    g2s<T, K>(sW, PK, reinterpret_cast<const T*>(a.W) + (t0 * H + h) * K, gsK, len, CH, tid, 256);
    g2s<T, K>(sF, PK, reinterpret_cast<const T*>(a.F) + (t0 * H + h) * K, gsK, len, CH, tid, 256);
    g2s<T, K>(sQg, PK, reinterpret_cast<const T*>(a.Qg) + (t0 * H + h) * K, gsK, len, CH, tid,
              256);
    g2s<T, CH>(sCq, PA, reinterpret_cast<const T*>(a.Cq) + ((int64_t)c * H + h) * CH * CH, CH, CH,
               CH, tid, 256);
    g2s<T, BV>(sdO, PU, reinterpret_cast<const T*>(a.dO) + (t0 * H + h) * V + vt * BV, gsV, len,
               CH, tid, 256);
    for (int kk = tid; kk < K; kk += 256) sLam[kk] = exp2f(a.glast[((int64_t)c * H + h) * K + kk]);
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
    __syncthreads();
    // Rbar = F dS+ + Cq^T dO
    T* Rbg = reinterpret_cast<T*>(a.Rb) + (t0 * H + h) * V + vt * BV;
#pragma unroll
    for (int r = 0; r < S::RPW; ++r) {
      const int t = w + 4 * r, ti = t / CT, tv = t - ti * CT;
      f32x4 acc = zero4();
      mma_tile<T, true, true>(acc, sF + ti * SUB * PK, PK, 1, sDt + tv * SUB * PK, PK, 1, K);
      mma_tile<T, false, false>(acc, sCq + ti * SUB, 1, PA, sdO + tv * SUB, 1, PU, CH);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = ti * SUB + crow(i), col = tv * SUB + ccol();
        if (row < len) Rbg[row * gsV + col] = fromf<T>(acc[i]);
        sRbt[col * PA + row] = fromf<T>(-acc[i]);
      }
    }
    __syncthreads();
    // dS = diag(exp2 G2_last) dS+ + Qg^T dO - W^T Rbar
#pragma unroll
    for (int s = 0; s < S::TPW; ++s) {
      const int t = w + 4 * s, tk = t / CT, tv = t - tk * CT;
#pragma unroll
      for (int i = 0; i < 4; ++i) st[s][i] *= sLam[tk * SUB + crow(i)];
      mma_tile<T, false, false>(st[s], sQg + tk * SUB, 1, PK, sdO + tv * SUB, 1, PU, CH);
      mma_tile<T, false, true>(st[s], sW + tk * SUB, 1, PK, sRbt + tv * SUB * PA, PA, 1, CH);
    }
    __syncthreads();
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

template <typename T>
static hipError_t fwd_scan_t(const Args& a, hipStream_t s) {
  const int bv = a.V < SCAN_BV ? a.V : SCAN_BV;
  const dim3 grid(a.N * a.H, a.V / bv), block(256);
  REWY_KV_SWITCH(k_fwd_scan)
}
template <typename T>
static hipError_t bwd_scan_t(const Args& a, hipStream_t s) {
  const int bv = a.V < SCAN_BV ? a.V : SCAN_BV;
  const dim3 grid(a.N * a.H, a.V / bv), block(256);
  REWY_KV_SWITCH(k_bwd_scan)
}

hipError_t launch_fwd_scan(const Args& a, int f32, hipStream_t s) {
  return f32 ? fwd_scan_t<float>(a, s) : fwd_scan_t<bf16>(a, s);
}
hipError_t launch_bwd_scan(const Args& a, int f32, hipStream_t s) {
  return f32 ? bwd_scan_t<float>(a, s) : bwd_scan_t<bf16>(a, s);
}

}  // namespace rewy
