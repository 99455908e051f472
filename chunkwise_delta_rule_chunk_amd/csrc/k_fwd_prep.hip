// Chunk index table and the chunk-parallel forward preparation.
//
// k_chunk_table: one record per 64-token chunk, restarting at every sequence
// start, the last chunk of a sequence partial (chunk length C = 64 as in the
// ReWY paper's experiments; KDA blog section 6.6 pipeline).
//
// k_fwd_prep, one workgroup per (chunk, head), for the chunk's n <= 64 rows
// (ReWY paper Appendix A; KDA blog sections 6.3-6.5):
//   G2 (base-2 in-chunk gate prefix sum), L = tril_strict(E Y^T),
//   Cq = tril_incl(Qg Y^T), A = (I + L)^-1 (fp32), W = A E, U = A Z (Z = beta V),
//   F = K exp2(G2_last - G2) (keys decayed to the chunk end), Qg = s Q exp2(G2),
//   and G2_last.  Score tiles are centred (see chunk_common.hpp).
#include "chunk_common.hpp"

namespace rewy {

__global__ void k_chunk_table(Args a) {
  __shared__ int s_total;
  if (threadIdx.x == 0) {
    int off = 0;
    for (int n = 0; n < a.N; ++n) {
      const int bos = a.cu ? a.cu[n] : n * a.T;
      const int eos = a.cu ? a.cu[n + 1] : (n + 1) * a.T;
      a.seqoff[n] = off;
      off += max(0, eos - bos + CH - 1) / CH;
    }
    a.seqoff[a.N] = off;
    s_total = min(off, a.nc_max);
  }
  __syncthreads();
  const int total = s_total;
  for (int c = threadIdx.x; c < a.nc_max; c += blockDim.x) {
    ChunkInfo ci = {0, 0, 0, 0};
    if (c < total) {
      // largest n with seqoff[n] <= c; it has seqoff[n+1] > c, so it is non-empty
      int lo = 0, hi = a.N - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.seqoff[mid] <= c) lo = mid;
        else hi = mid - 1;
      }
      const int bos = a.cu ? a.cu[lo] : lo * a.T;
      const int eos = a.cu ? a.cu[lo + 1] : (lo + 1) * a.T;
      const int pos = c - a.seqoff[lo];
      ci.seq = lo;
      ci.pos = pos;
      ci.bos = bos + pos * CH;
      ci.len = min(CH, eos - ci.bos);
    }
    a.chunks[c] = ci;
  }
}

hipError_t launch_chunk_table(const Args& a, hipStream_t s) {
  hipLaunchKernelGGL(k_chunk_table, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int K, int V>
__global__ __launch_bounds__(256) void k_fwd_prep(Args a) {
  constexpr int NTH = 256;
  constexpr bool BF = std::is_same_v<T, bf16>;
  constexpr int PK = pitch<T>(K);   // T rows of K
  constexpr int PG = K + 4;         // fp32 rows of K
  constexpr int PL = CH + 4;        // fp32 rows of 64
  constexpr int PA = pitch<T>(CH);  // T rows of 64
  constexpr int SZ_Q = CH * PK * (int)sizeof(T);
  constexpr int SZ_L = CH * PL * 4;
  constexpr int SZ_ET = K * PA * (int)sizeof(T);
  constexpr int SZ_ZT = V * PA * (int)sizeof(T);
  // phase 1: [sQ | sL | sA]; phase 2 (bf16): [E^T | Z^T] over the same bytes.
  // fp32 keeps sA alive during the WY products, so E^T / Z^T stay below sL.
  constexpr int OFF_L = BF ? SZ_Q : cmax(SZ_Q, cmax(SZ_ET, SZ_ZT));
  constexpr int REG = BF ? cmax(SZ_Q + 2 * SZ_L, SZ_ET + SZ_ZT) : OFF_L + 2 * SZ_L;

  __shared__ __align__(16) float sG[CH * PG];
  __shared__ __align__(16) T sK[CH * PK];
  __shared__ __align__(16) char sReg[REG];
  __shared__ __align__(16) T sCq[CH * PA];  // later: solve scratch
  __shared__ __align__(16) T sAb[BF ? CH * PA : 8];
  __shared__ float sBeta[CH];
  __shared__ float sMid[NSUB * K], sGl[NSUB * K];
  __shared__ int sFlag[NSUB];
  static_assert(CH * PA * sizeof(T) >= 4 * SUB * 20 * 4, "solve scratch");

  T* sQ = reinterpret_cast<T*>(sReg);
  float* sL = reinterpret_cast<float*>(sReg + OFF_L);
  float* sA = reinterpret_cast<float*>(sReg + OFF_L + SZ_L);
  T* sEt = reinterpret_cast<T*>(sReg);
  T* sZt = reinterpret_cast<T*>(sReg + (BF ? SZ_ET : 0));
  float* sT = reinterpret_cast<float*>(sCq);

  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const ChunkInfo ci = a.chunks[c];
  const int n = ci.len;
  if (n == 0) return;
  const int H = a.H;
  const int64_t t0 = ci.bos;
  const int64_t gsK = (int64_t)H * K, gsV = (int64_t)H * V;
  const T* qg = reinterpret_cast<const T*>(a.q) + (t0 * H + h) * K;
  const T* kg = reinterpret_cast<const T*>(a.k) + (t0 * H + h) * K;
  const T* vg = reinterpret_cast<const T*>(a.v) + (t0 * H + h) * V;

  // ---- 1. keys, queries, beta; zeroed score buffers; gate prefix sum -------
  g2s<T, K>(sK, PK, kg, gsK, n, CH, tid, NTH);
  g2s<T, K>(sQ, PK, qg, gsK, n, CH, tid, NTH);
  if (tid < CH) sBeta[tid] = tid < n ? ld_beta(a.beta, a.beta_f32, (t0 + tid) * H + h) : 0.f;
  if (tid < NSUB) sFlag[tid] = 0;
  for (int idx = tid; idx < CH * PL; idx += NTH) {
    sL[idx] = 0.f;
    sA[idx] = 0.f;
  }
  for (int idx = tid; idx < CH * PA; idx += NTH) sCq[idx] = fromf<T>(0.f);
  load_gate_cumsum<K>(sG, PG, a, t0, h, n, K, 0, tid, NTH);

  // ---- 2. sub-chunk statistics; element-wise outputs ----------------------
  subchunk_stats<K>(sG, PG, n, nullptr, sGl, sMid, sFlag, tid, NTH);
  const int mode = a.prep_mode;
  const int64_t cbase = (int64_t)c * H + h;  // chunk-tile index
  {
    const float* Gn = sG + (n - 1) * PG;
    if (mode & (PREP_FWD_OUT | PREP_BWD_SCAN)) {
      T* Qgo = reinterpret_cast<T*>(a.Qg) + (t0 * H + h) * K;
      T* Fo = reinterpret_cast<T*>(a.F) + (t0 * H + h) * K;
      for (int idx = tid; idx < n * K; idx += NTH) {
        const int i = idx / K, kk = idx - i * K;
        const float G = sG[i * PG + kk];
        if (mode & PREP_FWD_OUT) Qgo[i * gsK + kk] = fromf<T>(a.scale * tof(sQ[i * PK + kk]) * exp2f(G));
        if (mode & PREP_BWD_SCAN) Fo[i * gsK + kk] = fromf<T>(tof(sK[i * PK + kk]) * exp2f(Gn[kk] - G));
      }
    }
    if (mode & (PREP_FWD_SCAN | PREP_BWD_SCAN))
      for (int kk = tid; kk < K; kk += NTH) a.glast[cbase * K + kk] = Gn[kk];
    // token-contiguous tiles [K][64] (zeros past the chunk end: sK, sQ rows are zero there)
    if (mode & PREP_FWD_SCAN) {
      T* Fto = reinterpret_cast<T*>(a.Ft) + cbase * K * CH;
      for (int idx = tid; idx < K * CH; idx += NTH) {
        const int kk = idx / CH, i = idx - kk * CH;
        Fto[idx] = fromf<T>(tof(sK[i * PK + kk]) * exp2f(Gn[kk] - sG[i * PG + kk]));
      }
    }
    if (mode & PREP_BWD_SCAN) {
      T* Qgto = reinterpret_cast<T*>(a.Qgt) + cbase * K * CH;
      for (int idx = tid; idx < K * CH; idx += NTH) {
        const int kk = idx / CH, i = idx - kk * CH;
        Qgto[idx] = fromf<T>(a.scale * tof(sQ[i * PK + kk]) * exp2f(sG[i * PG + kk]));
      }
    }
  }
  __syncthreads();

  // ---- 3. centred score tiles: L (strict) and Cq (inclusive) ---------------
  score_tiles<T, K, true>(sG, PG, sK, sQ, PK, sBeta, sMid, sGl, sFlag, n, a.scale, sL, PL, sCq,
                          PA);
  __syncthreads();
  if (mode & PREP_FWD_OUT)
    s2g<T, CH>(reinterpret_cast<T*>(a.Cq) + cbase * CH * CH, CH, sCq, PA, CH, tid, NTH);
  if (mode & PREP_BWD_SCAN) {
    T* Cqto = reinterpret_cast<T*>(a.Cqt) + cbase * CH * CH;
    for (int idx = tid; idx < CH * CH; idx += NTH) {
      const int i = idx / CH, j = idx - i * CH;
      Cqto[idx] = sCq[j * PA + i];
    }
  }
  __syncthreads();  // sCq becomes solve scratch

  // ---- 4. A = (I + L)^-1 in fp32 --------------------------------------------
  solve_unit_lower(sL, sA, PL, sT, n);

  // ---- 5. operands of the WY products --------------------------------------
  if constexpr (BF) {
    for (int idx = tid; idx < CH * CH; idx += NTH) {
      const int i = idx / CH, j = idx - i * CH;
      sAb[i * PA + j] = (bf16)sA[i * PL + j];
    }
    __syncthreads();  // sA is overwritten by E^T / Z^T below
  }
  for (int idx = tid; idx < K * CH; idx += NTH) {
    const int kk = idx / CH, j = idx - kk * CH;
    sEt[kk * PA + j] = fromf<T>(sBeta[j] * tof(sK[j * PK + kk]) * exp2f(sG[j * PG + kk]));
  }
  const int w = wave_id();
  T* Wo = reinterpret_cast<T*>(a.W) + (t0 * H + h) * K;
  T* Uo = reinterpret_cast<T*>(a.U) + (t0 * H + h) * V;
  T* Wto = reinterpret_cast<T*>(a.Wt) + cbase * K * CH;
  const bool wantW = mode & PREP_FWD_SCAN, wantWt = mode & PREP_BWD_SCAN, wantU = wantW;
  // W^T needs every row block (rows past the chunk end are exact zeros)
  const int nblk = wantWt ? NSUB : (n + SUB - 1) / SUB;
  auto put_w = [&](const f32x4& acc, int I, int col) {
    if (wantW) st_tile<T>(acc, Wo + (I * SUB) * gsK + col, (int)gsK, 1, n - I * SUB);
    if (wantWt) st_tile_T<T>(acc, Wto + (int64_t)col * CH + I * SUB, CH);
  };
  if constexpr (BF) {
    constexpr int VEC = 8, PER = V / VEC;
    if (wantU) {
      for (int idx = tid; idx < CH * PER; idx += NTH) {
        const int r = idx / PER, c0 = (idx - r * PER) * VEC;
        union {
          uint4 u;
          T e[VEC];
        } val;
        val.u = uint4{0u, 0u, 0u, 0u};
        if (r < n) val.u = *reinterpret_cast<const uint4*>(vg + (int64_t)r * gsV + c0);
        const float b = sBeta[r];
#pragma unroll
        for (int e = 0; e < VEC; ++e) sZt[(c0 + e) * PA + r] = fromf<T>(b * tof(val.e[e]));
      }
    }
    __syncthreads();
    // ---- 6. W = A E, U = A Z ------------------------------------------------
    const int NCB = (K + (wantU ? V : 0)) / SUB;
    for (int cb = w; cb < NCB; cb += 4) {
      const bool isW = cb < K / SUB;
      if (isW && !wantW && !wantWt) continue;
      const int col = isW ? cb * SUB : (cb - K / SUB) * SUB;
      const T* Bop = (isW ? sEt : sZt) + col * PA;
      for (int I = 0; I < (isW ? nblk : (n + SUB - 1) / SUB); ++I) {
        f32x4 acc = zero4();
        const int kd = ((SUB * (I + 1) + 31) / 32) * 32;
        mma_tile<T, true, true>(acc, sAb + (I * SUB) * PA, PA, 1, Bop, PA, 1, kd);
        if (isW) put_w(acc, I, col);
        else st_tile<T>(acc, Uo + (I * SUB) * gsV + col, (int)gsV, 1, n - I * SUB);
      }
    }
  } else {
    __syncthreads();
    if (wantW || wantWt)
      for (int cb = w; cb < K / SUB; cb += 4)
        for (int I = 0; I < nblk; ++I) {
          f32x4 acc = zero4();
          mma_tile<float, false, false>(acc, sA + (I * SUB) * PL, PL, 1, sEt + cb * SUB * PA, PA,
                                        1, SUB * (I + 1));
          put_w(acc, I, cb * SUB);
        }
    __syncthreads();
    if (wantU) {
      for (int idx = tid; idx < V * CH; idx += NTH) {
        const int vv = idx / CH, j = idx - vv * CH;
        sZt[vv * PA + j] = fromf<T>(j < n ? sBeta[j] * tof(vg[(int64_t)j * gsV + vv]) : 0.f);
      }
      __syncthreads();
      for (int cb = w; cb < V / SUB; cb += 4)
        for (int I = 0; I < NSUB && I * SUB < n; ++I) {
          f32x4 acc = zero4();
          mma_tile<float, false, false>(acc, sA + (I * SUB) * PL, PL, 1, sZt + cb * SUB * PA, PA,
                                        1, SUB * (I + 1));
          st_tile<T>(acc, Uo + (I * SUB) * gsV + cb * SUB, (int)gsV, 1, n - I * SUB);
        }
    }
  }
}

template <typename T>
static hipError_t prep_t(const Args& a, hipStream_t s) {
  const dim3 grid(a.nc_max, a.H), block(256);
  REWY_KV_SWITCH(k_fwd_prep)
}

hipError_t launch_fwd_prep(const Args& a, int f32, hipStream_t s) {
  return f32 ? prep_t<float>(a, s) : prep_t<bf16>(a, s);
}

}  // namespace rewy
