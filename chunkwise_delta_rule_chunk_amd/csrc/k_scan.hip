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

template <int V>
using ic = std::integral_constant<int, V>;

// exp2 of G2 at the chunk's last row, per key row: the chunk decay Lambda.
template <int K>
struct StagedDecay {
  f32x4 r;
  __device__ __forceinline__ void load(const float* g, int tid) {
    r = zero4();
    if (tid < K / 4) r = reinterpret_cast<const f32x4*>(g)[tid];
  }
  __device__ __forceinline__ void store(float* s, int tid) const {
    if (tid < K / 4) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = fexp2(r[e]);
      reinterpret_cast<f32x4*>(s)[tid] = x;
    }
  }
};

template <typename T, int K, int V, int BV>
__global__ __launch_bounds__(256) void k_fwd_scan(Args a) {
  using S = ScanShape<K, BV>;
  constexpr int CT = S::CT, NTH = 256;
  constexpr int PK = pitch<T>(K), PU = pitch<T>(BV), PA = pitch<T>(CH);
  __shared__ __align__(16) T sW[2][CH * PK];
  __shared__ __align__(16) T sFt[2][K * PA];
  __shared__ __align__(16) T sU[2][CH * PU];
  __shared__ __align__(16) float sLam[2][K];  // exp2(G2_last)
  // S_c and R_c as MFMA operands, [v][k] and [v][i]; two buffers, since the
  // transposed outputs are written from them during the next step
  __shared__ __align__(16) T sHt[2][BV * PK];
  __shared__ __align__(16) T sRt[2][BV * PA];
  // S_c and R_c in natural layout, written to global memory with 16-byte
  // stores during the next step (few memory instructions per step)
  __shared__ __align__(16) T sS[2][K * PU];
  __shared__ __align__(16) T sR[2][CH * PU];
  __shared__ int sLen[2];
  __shared__ int64_t sT0[2];

  const int H = a.H;
  const int u = blockIdx.x, vt = blockIdx.y;
  const int n = u / H, h = u - n * H;
  const int w = wave_id(), tid = threadIdx.x;
  const int64_t gsK = (int64_t)H * K, gsV = (int64_t)H * V;
  const int c0 = a.seqoff[n], c1 = a.seqoff[n + 1];
  const T* Wg = reinterpret_cast<const T*>(a.W);
  const T* Ftg = reinterpret_cast<const T*>(a.Ft);
  const T* Ug = reinterpret_cast<const T*>(a.U);

  // two register sets: chunk c + 2 is read while chunk c is processed
  Staged<T, CH, K, NTH> pW[2];
  Staged<T, K, CH, NTH> pF[2];
  Staged<T, CH, BV, NTH> pU[2];
  StagedDecay<K> pL[2];
  auto fetch = [&](auto set, int c) {
    const ChunkInfo ci = a.chunks[c];
    const int64_t t0 = ci.bos, cb = (int64_t)c * H + h;
    pW[set].load(Wg + (t0 * H + h) * K, gsK, ci.len, tid);
    pF[set].load(Ftg + cb * K * CH, CH, K, tid);
    pU[set].load(Ug + (t0 * H + h) * V + vt * BV, gsV, ci.len, tid);
    pL[set].load(a.glast + cb * K, tid);
  };
  auto put = [&](auto set) {
    pW[set].store(sW[set], PK, tid);
    pF[set].store(sFt[set], PA, tid);
    pU[set].store(sU[set], PU, tid);
    pL[set].store(sLam[set], tid);
  };
  // S and R staged in buffer b, to global memory (R rows past the end skipped):
  // natural layouts for the chunk backward, transposed ones for the output
  const bool natural = a.scan_out & SCAN_NATURAL, transposed = a.scan_out & SCAN_TRANSPOSED;
  auto flush = [&](auto b, int c) {
    constexpr int VE = 16 / (int)sizeof(T), PER = BV / VE;
    if (transposed) {
      T* ht = reinterpret_cast<T*>(a.hbufT) + (((int64_t)c * H + h) * V + vt * BV) * K;
      for (int idx = tid; idx < BV * (K / VE); idx += NTH) {
        const int r = idx / (K / VE), c8 = (idx - r * (K / VE)) * VE;
        *reinterpret_cast<uint4*>(ht + (int64_t)r * K + c8) =
            *reinterpret_cast<const uint4*>(sHt[b] + r * PK + c8);
      }
      T* rt = reinterpret_cast<T*>(a.RT) + (((int64_t)c * H + h) * V + vt * BV) * CH;
      for (int idx = tid; idx < BV * (CH / VE); idx += NTH) {
        const int r = idx / (CH / VE), c8 = (idx - r * (CH / VE)) * VE;
        *reinterpret_cast<uint4*>(rt + r * CH + c8) =
            *reinterpret_cast<const uint4*>(sRt[b] + r * PA + c8);
      }
    }
    if (!natural) return;
    T* hb = reinterpret_cast<T*>(a.hbuf) + ((int64_t)c * H + h) * K * V + vt * BV;
    for (int idx = tid; idx < K * PER; idx += NTH) {
      const int r = idx / PER, c8 = (idx - r * PER) * VE;
      *reinterpret_cast<uint4*>(hb + (int64_t)r * V + c8) =
          *reinterpret_cast<const uint4*>(sS[b] + r * PU + c8);
    }
    const int len = sLen[b];
    T* Rg = reinterpret_cast<T*>(a.R) + (sT0[b] * H + h) * V + vt * BV;
    for (int idx = tid; idx < CH * PER; idx += NTH) {
      const int r = idx / PER, c8 = (idx - r * PER) * VE;
      if (r < len)
        *reinterpret_cast<uint4*>(Rg + (int64_t)r * gsV + c8) =
            *reinterpret_cast<const uint4*>(sR[b] + r * PU + c8);
    }
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
    fetch(ic<0>{}, c0);
    if (c0 + 1 < c1) fetch(ic<1>{}, c0 + 1);
    put(ic<0>{});
  }
  lds_barrier();

  auto step = [&](auto buf, int c) {
    constexpr int B = decltype(buf)::value;
    if (c + 2 < c1) fetch(ic<B>{}, c + 2);
    if (c > c0) flush(ic<B ^ 1>{}, c - 1);
    // S_c: staged for global memory, and as the operand of W S
#pragma unroll
    for (int s = 0; s < S::TPW; ++s) {
      const int t = w + 4 * s, tk = t / CT, tv = t - tk * CT;
      f32x4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = tof(fromf<T>(st[s][i]));
        if (natural) sS[B][(tk * SUB + crow(i)) * PU + tv * SUB + ccol()] = fromf<T>(st[s][i]);
      }
      st_tile_T<T>(x, sHt[B] + (tv * SUB) * PK + tk * SUB, PK);
    }
    if (tid == 0) {
      const ChunkInfo ci = a.chunks[c];
      sLen[B] = ci.len;
      sT0[B] = ci.bos;
    }
    lds_barrier();
    // R = U - W S
#pragma unroll
    for (int r = 0; r < S::RPW; ++r) {
      const int t = w + 4 * r, ti = t / CT, tv = t - ti * CT;
      f32x4 p = zero4();
      mma_tile<T, true, true>(p, sW[B] + ti * SUB * PK, PK, 1, sHt[B] + tv * SUB * PK, PK, 1, K);
      f32x4 rv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = ti * SUB + crow(i), col = tv * SUB + ccol();
        const T x = fromf<T>(tof(sU[B][row * PU + col]) - p[i]);
        if (natural) sR[B][row * PU + col] = x;
        rv[i] = tof(x);
      }
      st_tile_T<T>(rv, sRt[B] + (tv * SUB) * PA + ti * SUB, PA);
    }
    lds_barrier();
    // S = diag(exp2 G2_last) S + F^T R
#pragma unroll
    for (int s = 0; s < S::TPW; ++s) {
      const int t = w + 4 * s, tk = t / CT, tv = t - tk * CT;
#pragma unroll
      for (int i = 0; i < 4; ++i) st[s][i] *= sLam[B][tk * SUB + crow(i)];
      mma_tile<T, true, true>(st[s], sFt[B] + tk * SUB * PA, PA, 1, sRt[B] + tv * SUB * PA, PA, 1, CH);
    }
    if (c + 1 < c1) put(ic<B ^ 1>{});  // chunk c + 1; its buffer was last read a step ago
  };
  for (int c = c0; c < c1; c += 2) {
    step(ic<0>{}, c);
    if (c + 1 < c1) step(ic<1>{}, c + 1);
  }
  lds_barrier();
  if (c1 > c0) {  // the last chunk's S and R
    if ((c1 - 1 - c0) & 1) flush(ic<1>{}, c1 - 1);
    else flush(ic<0>{}, c1 - 1);
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
  constexpr int PK = pitch<T>(K), PA = pitch<T>(CH), PS = pitch<T>(BV);
  // one buffer of chunk operands, refilled between two barriers
  __shared__ __align__(16) T sF[CH * PK];
  __shared__ __align__(16) T sWt[K * PA];
  __shared__ __align__(16) T sQgt[K * PA];
  __shared__ __align__(16) T sCqt[CH * PA];
  __shared__ __align__(16) T sdOt[BV * PA];   // dO as operand, [v][j]
  __shared__ __align__(16) float sLam[K];     // exp2(G2_last)
  __shared__ __align__(16) T sDt[BV * PK];    // dS_{c+1} as operand, [v][k]
  __shared__ __align__(16) T sRbt[BV * PA];   // -Rbar as operand, [v][i]
  // dS_{c+1} in natural layout, written to global memory during the next step
  __shared__ __align__(16) T sD[2][K * PS];

  const int H = a.H;
  const int u = blockIdx.x, vt = blockIdx.y;
  const int n = u / H, h = u - n * H;
  const int w = wave_id(), tid = threadIdx.x;
  const int64_t gsK = (int64_t)H * K, gsV = (int64_t)H * V;
  const int c0 = a.seqoff[n], c1 = a.seqoff[n + 1];

  // two register sets: chunk c - 2 is read while chunk c is processed
  Staged<T, CH, K, NTH> pF[2];
  Staged<T, K, CH, NTH> pW[2];
  Staged<T, K, CH, NTH> pQ[2];
  Staged<T, CH, CH, NTH> pC[2];
  Staged<T, CH, BV, NTH> pO[2];
  StagedDecay<K> pL[2];
  auto fetch = [&](auto set, int c) {
    const ChunkInfo ci = a.chunks[c];
    const int64_t t0 = ci.bos, cb = (int64_t)c * H + h;
    pF[set].load(reinterpret_cast<const T*>(a.F) + (t0 * H + h) * K, gsK, ci.len, tid);
    pW[set].load(reinterpret_cast<const T*>(a.Wt) + cb * K * CH, CH, K, tid);
    pQ[set].load(reinterpret_cast<const T*>(a.Qgt) + cb * K * CH, CH, K, tid);
    pC[set].load(reinterpret_cast<const T*>(a.Cqt) + cb * CH * CH, CH, CH, tid);
    pO[set].load(reinterpret_cast<const T*>(a.dO) + (t0 * H + h) * V + vt * BV, gsV, ci.len, tid);
    pL[set].load(a.glast + cb * K, tid);
  };
  auto put = [&](auto set) {
    pF[set].store(sF, PK, tid);
    pW[set].store(sWt, PA, tid);
    pQ[set].store(sQgt, PA, tid);
    pC[set].store(sCqt, PA, tid);
    pO[set].store_T(sdOt, PA, tid);
    pL[set].store(sLam, tid);
  };
  auto flush = [&](auto b, int c) {
    constexpr int VE = 16 / (int)sizeof(T), PER = BV / VE;
    T* db = reinterpret_cast<T*>(a.dhbuf) + ((int64_t)c * H + h) * K * V + vt * BV;
    for (int idx = tid; idx < K * PER; idx += NTH) {
      const int r = idx / PER, c8 = (idx - r * PER) * VE;
      *reinterpret_cast<uint4*>(db + (int64_t)r * V + c8) =
          *reinterpret_cast<const uint4*>(sD[b] + r * PS + c8);
    }
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
    fetch(ic<0>{}, c1 - 1);
    if (c1 - 2 >= c0) fetch(ic<1>{}, c1 - 2);
    put(ic<0>{});
  }

  auto step = [&](auto buf, int c) {
    constexpr int B = decltype(buf)::value;
    if (c - 2 >= c0) fetch(ic<B>{}, c - 2);
    if (c < c1 - 1) flush(ic<B ^ 1>{}, c + 1);  // dS_{c+2}, staged last step
    const ChunkInfo ci = a.chunks[c];
    const int64_t t0 = ci.bos;
    // dS_{c+1}: staged for global memory, and as the operand of F dS+
#pragma unroll
    for (int s = 0; s < S::TPW; ++s) {
      const int t = w + 4 * s, tk = t / CT, tv = t - tk * CT;
      f32x4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = tof(fromf<T>(st[s][i]));
        sD[B][(tk * SUB + crow(i)) * PS + tv * SUB + ccol()] = fromf<T>(st[s][i]);
      }
      st_tile_T<T>(x, sDt + (tv * SUB) * PK + tk * SUB, PK);
    }
    lds_barrier();  // operands of chunk c and dS_{c+1} visible
    // Rbar = F dS+ + Cq^T dO, stored token-contiguous
    T* Rbt = reinterpret_cast<T*>(a.Rbt) + ((int64_t)c * H + h) * V * CH + vt * BV * CH;
#pragma unroll
    for (int r = 0; r < S::RPW; ++r) {
      const int t = w + 4 * r, ti = t / CT, tv = t - ti * CT;
      f32x4 acc = zero4();
      mma_tile<T, true, true>(acc, sF + ti * SUB * PK, PK, 1, sDt + tv * SUB * PK, PK, 1, K);
      mma_tile<T, true, true>(acc, sCqt + ti * SUB * PA, PA, 1, sdOt + tv * SUB * PA, PA, 1, CH);
      // rows past the chunk's end are exact zeros (F and Cq vanish there)
      st_tile_T<T>(acc, Rbt + (tv * SUB) * CH + ti * SUB, CH);
      st_tile_T<T>(-acc, sRbt + (tv * SUB) * PA + ti * SUB, PA);
    }
    lds_barrier();
    // dS = diag(exp2 G2_last) dS+ + Qg^T dO - W^T Rbar
#pragma unroll
    for (int s = 0; s < S::TPW; ++s) {
      const int t = w + 4 * s, tk = t / CT, tv = t - tk * CT;
#pragma unroll
      for (int i = 0; i < 4; ++i) st[s][i] *= sLam[tk * SUB + crow(i)];
      mma_tile<T, true, true>(st[s], sQgt + tk * SUB * PA, PA, 1, sdOt + tv * SUB * PA, PA, 1, CH);
      mma_tile<T, true, true>(st[s], sWt + tk * SUB * PA, PA, 1, sRbt + tv * SUB * PA, PA, 1, CH);
    }
    (void)t0;
    if (c - 1 >= c0) {
      lds_barrier();  // every wave is done with chunk c's operands
      put(ic<B ^ 1>{});
    }
  };
  for (int c = c1 - 1; c >= c0; c -= 2) {
    step(ic<0>{}, c);
    if (c - 1 >= c0) step(ic<1>{}, c - 1);
  }
  lds_barrier();
  if (c1 > c0) {  // dS_{c0+1}, staged by the last step
    if ((c1 - 1 - c0) & 1) flush(ic<1>{}, c0);
    else flush(ic<0>{}, c0);
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
