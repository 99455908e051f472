// Chunk-parallel backward after the reverse scan: the ReWY producer and the
// gradient consumer.  One workgroup per (chunk, head) for each.
//
// Producer (ReWY paper Algorithm 1, steps 1-3; the value/write gradients of
// Appendix 7.3):
//   A = (I + L)^-1 recomputed from k, g, beta (same centred tiles as forward)
//   P = A^T Rbar                 shared sensitivity (no adjoint of A is formed)
//   dv = beta * P,   dbeta_write_i = <V_i, P_i>
//   D  = -tril_strict(P R^T),    Hq = tril_incl(dO R^T)   (output-path adjoint)
//
// Consumer (Algorithm 1 step 4, Appendix 7.2-7.3 chain rules, Appendix 10
// complete reverse order), per feature tile:
//   state products   dO S^T, P S^T, Fbar = R dS+^T             (S = S_c, dS+ = dS_{c+1})
//   matrix intra     gamma*(Hq Y), gamma*(D Y), (D^T E)/gamma, (Hq^T Qg)/gamma
//   chain rules      dq = s gamma Qgbar,  dk = beta gamma Ebar + Ybar/gamma,
//                    dbeta_erase = <gamma K, Ebar>,  Gbar = Qg Qgbar + E Ebar - Y Ybar
//   endpoints        Gbar_last += gamma_last * (rowsum(S * dS+) + colsum(Y * Fbar))
//   reverse sum      dg = reverse in-chunk cumulative sum of Gbar (feature sum for a
//                    scalar gate: the Gram-free reduction of paper section 3.4)
// The matrix-intra products are sub-chunk blocked.  For output block I and
// source block J < I the sending operand is K exp2(Gl_J - G) (reference: last
// row of J), the column factor exp2(Gf_I - Gl_J) and the receiving factor
// exp2(G - Gf_I) (first row of I): every factor is <= 1.  A diagonal block
// centres both sides on its midpoint (paper section 3.3 "Centered factors"), or
// is summed pairwise when its gate range exceeds CENTRE_MAX_RANGE.  The
// transposed products mirror this with the roles of I and J exchanged.
#include "chunk_common.hpp"

namespace rewy {

template <typename T, int K, int V>
__global__ __launch_bounds__(256) void k_bwd_prod(Args a) {
  constexpr int NTH = 256;
  constexpr int PK = pitch<T>(K), PG = K + 4, PL = CH + 4, PA = pitch<T>(CH), PV = pitch<T>(V);
  constexpr int SZ_G = CH * PG * 4, SZ_K = CH * PK * (int)sizeof(T), SZ_L = CH * PL * 4;
  constexpr int SZ_T = 4 * SUB * 20 * 4;
  constexpr int SZ_AT = CH * PA * (int)sizeof(T), SZ_RBT = V * PA * (int)sizeof(T);
  constexpr int SZ_PV = CH * PV * (int)sizeof(T);
  // phase A: L and A
  constexpr int A_G = 0, A_K = A_G + SZ_G, A_L = A_K + SZ_K, A_A = A_L + SZ_L, A_T = A_A + SZ_L;
  constexpr int END_A = A_T + SZ_T;
  // phase B: P = A^T Rbar (A^T is written while sA is still live)
  constexpr int B_AT = 0, B_RBT = SZ_AT, B_V = B_RBT + SZ_RBT, B_P = B_V + SZ_PV;
  constexpr int END_B = B_P + SZ_PV;
  static_assert(B_AT + SZ_AT <= A_A, "A^T must not overlap A");
  // phase C: D and Hq (P stays live)
  constexpr int C_D = 0, C_HQ = SZ_AT, C_R = END_B, C_DO = C_R + SZ_PV, END_C = C_DO + SZ_PV;
  static_assert(C_HQ + SZ_AT <= B_P, "D/Hq must not overlap P");
  constexpr int TOTAL = cmax(END_A, END_C);

  __shared__ __align__(16) char smem[TOTAL];
  __shared__ float sBeta[CH], sMid[NSUB * K], sGl[NSUB * K], sDbw[4 * CH];
  __shared__ int sFlag[NSUB];
  float* sG = reinterpret_cast<float*>(smem + A_G);
  T* sK = reinterpret_cast<T*>(smem + A_K);
  float* sL = reinterpret_cast<float*>(smem + A_L);
  float* sA = reinterpret_cast<float*>(smem + A_A);
  float* sT = reinterpret_cast<float*>(smem + A_T);
  T* sAT = reinterpret_cast<T*>(smem + B_AT);
  T* sRbT = reinterpret_cast<T*>(smem + B_RBT);
  T* sV = reinterpret_cast<T*>(smem + B_V);
  T* sP = reinterpret_cast<T*>(smem + B_P);
  T* sD = reinterpret_cast<T*>(smem + C_D);
  T* sHq = reinterpret_cast<T*>(smem + C_HQ);
  T* sR = reinterpret_cast<T*>(smem + C_R);
  T* sdO = reinterpret_cast<T*>(smem + C_DO);

  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const ChunkInfo ci = a.chunks[c];
  const int n = ci.len;
  if (n == 0) return;
  const int H = a.H;
  const int64_t t0 = ci.bos;
  const int64_t gsK = (int64_t)H * K, gsV = (int64_t)H * V;
  const int w = wave_id(), l = lane_id();

  // ---- A: recompute L and A -------------------------------------------------
  g2s<T, K>(sK, PK, reinterpret_cast<const T*>(a.k) + (t0 * H + h) * K, gsK, n, CH, tid, NTH);
  if (tid < CH) sBeta[tid] = tid < n ? ld_beta(a.beta, a.beta_f32, (t0 + tid) * H + h) : 0.f;
  if (tid < NSUB) sFlag[tid] = 0;
  for (int idx = tid; idx < CH * PL; idx += NTH) {
    sL[idx] = 0.f;
    sA[idx] = 0.f;
  }
  for (int idx = tid; idx < 4 * CH; idx += NTH) sDbw[idx] = 0.f;
  load_gate_cumsum<K>(sG, PG, a, t0, h, n, K, 0, tid, NTH);
  subchunk_stats<K>(sG, PG, n, nullptr, sGl, sMid, sFlag, tid, NTH);
  __syncthreads();
  score_tiles<T, K, false>(sG, PG, sK, nullptr, PK, sBeta, sMid, sGl, sFlag, n, 0.f, sL, PL,
                           nullptr, PA);
  __syncthreads();
  solve_unit_lower(sL, sA, PL, sT, n);

  // ---- B: P = A^T Rbar, dv, write part of dbeta ----------------------------
  for (int idx = tid; idx < CH * CH; idx += NTH) {
    const int i = idx / CH, j = idx - i * CH;
    sAT[i * PA + j] = fromf<T>(sA[j * PL + i]);
  }
  __syncthreads();
  g2s_T<T, V>(sRbT, PA, reinterpret_cast<const T*>(a.Rb) + (t0 * H + h) * V, gsV, n, CH, tid, NTH);
  g2s<T, V>(sV, PV, reinterpret_cast<const T*>(a.v) + (t0 * H + h) * V, gsV, n, CH, tid, NTH);
  __syncthreads();
  {
    T* dvg = reinterpret_cast<T*>(a.dv) + (t0 * H + h) * V;
    float part[NSUB][4];
#pragma unroll
    for (int I = 0; I < NSUB; ++I)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[I][i] = 0.f;
    for (int cb = w; cb < V / SUB; cb += 4) {
#pragma unroll
      for (int I = 0; I < NSUB; ++I) {
        if (I * SUB >= n) break;
        const int j0 = (I * SUB / MM<T>::KS) * MM<T>::KS;  // A^T is upper triangular
        f32x4 acc = zero4();
        mma_tile<T, true, true>(acc, sAT + I * SUB * PA + j0, PA, 1, sRbT + cb * SUB * PA + j0,
                                PA, 1, CH - j0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = I * SUB + crow(i), col = cb * SUB + ccol();
          if (row < n) dvg[row * gsV + col] = fromf<T>(sBeta[row] * acc[i]);
          sP[row * PV + col] = fromf<T>(acc[i]);
          part[I][i] += acc[i] * tof(sV[row * PV + col]);
        }
      }
    }
#pragma unroll
    for (int I = 0; I < NSUB; ++I)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = part[I][i];
        x += __shfl_xor(x, 1);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 8);
        if ((l & 15) == 0) sDbw[w * CH + I * SUB + crow(i)] = x;
      }
  }
  __syncthreads();
  if (tid < n)
    a.dbw[(t0 + tid) * H + h] = sDbw[tid] + sDbw[CH + tid] + sDbw[2 * CH + tid] + sDbw[3 * CH + tid];
  s2g<T, V>(reinterpret_cast<T*>(a.P) + (t0 * H + h) * V, gsV, sP, PV, n, tid, NTH);
  // ---- C: D = -tril_strict(P R^T), Hq = tril_incl(dO R^T) -------------------
  g2s<T, V>(sR, PV, reinterpret_cast<const T*>(a.R) + (t0 * H + h) * V, gsV, n, CH, tid, NTH);
  g2s<T, V>(sdO, PV, reinterpret_cast<const T*>(a.dO) + (t0 * H + h) * V, gsV, n, CH, tid, NTH);
  __syncthreads();  // sAT / sRbT are dead: D / Hq take their place
  for (int idx = tid; idx < CH * PA; idx += NTH) {
    sD[idx] = fromf<T>(0.f);
    sHq[idx] = fromf<T>(0.f);
  }
  __syncthreads();
  for (int p = w; p < 10; p += 4) {
    int I, J;
    pair_ij(p, I, J);
    if (I * SUB >= n) continue;
    f32x4 accD = zero4(), accH = zero4();
    mma_tile<T, true, true>(accD, sP + I * SUB * PV, PV, 1, sR + J * SUB * PV, PV, 1, V);
    mma_tile<T, true, true>(accH, sdO + I * SUB * PV, PV, 1, sR + J * SUB * PV, PV, 1, V);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = I * SUB + crow(i), col = J * SUB + ccol();
      if (row > col) sD[row * PA + col] = fromf<T>(-accD[i]);
      if (row >= col) sHq[row * PA + col] = fromf<T>(accH[i]);
    }
  }
  __syncthreads();
  s2g<T, CH>(reinterpret_cast<T*>(a.D) + ((int64_t)c * H + h) * CH * CH, CH, sD, PA, CH, tid, NTH);
  s2g<T, CH>(reinterpret_cast<T*>(a.Hq) + ((int64_t)c * H + h) * CH * CH, CH, sHq, PA, CH, tid,
             NTH);
}

template <typename T, int K, int V>
__global__ __launch_bounds__(256) void k_bwd_cons(Args a) {
  constexpr int NTH = 256;
  constexpr bool BF = std::is_same_v<T, bf16>;
  constexpr int KT = K < (BF ? 32 : 16) ? K : (BF ? 32 : 16);  // feature tile
  constexpr int NKT = K / KT, CTK = KT / SUB;
  constexpr int PA = pitch<T>(CH), PV = pitch<T>(V), PKT = pitch<T>(KT), PGT = KT + 4;

  __shared__ __align__(16) T sD[CH * PA];
  __shared__ __align__(16) T sHq[CH * PA];
  __shared__ __align__(16) T sdO[CH * PV];
  __shared__ __align__(16) T sP[CH * PV];
  __shared__ __align__(16) T sR[CH * PV];
  __shared__ __align__(16) float sG[CH * PGT];
  __shared__ __align__(16) T sK[CH * PKT];
  __shared__ __align__(16) T sQ[CH * PKT];
  // scaled sending operands, [feature][token]; for bf16 each is held as a
  // high part and a low part (x ~ hi + lo) so that the matrix-intra products
  // keep about 16 mantissa bits of the sending side: the log-gate gradient is a
  // difference of nearly equal receiving and sending sums, which amplifies the
  // rounding of these operands.
  constexpr int NPART = BF ? 2 : 1;
  __shared__ __align__(16) T sSc[6 * NPART][KT * PA];
  enum { KC_E = 0, KC_M = 1, KA_F = 2, KA_M = 3, QA_F = 4, QA_M = 5 };
  __shared__ __align__(16) float sGb[CH * PGT];
  __shared__ float sBeta[CH], sDbe[CH], sGs[CH];
  __shared__ float sGf[NSUB * KT], sGl[NSUB * KT], sMid[NSUB * KT];
  __shared__ float sLamW[4 * KT], sLam0[KT];
  __shared__ int sFlag[NSUB];

  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const ChunkInfo ci = a.chunks[c];
  const int n = ci.len;
  if (n == 0) return;
  const int H = a.H;
  const int64_t t0 = ci.bos;
  const int64_t gsK = (int64_t)H * K, gsV = (int64_t)H * V;
  const int w = wave_id(), l = lane_id();
  const float scale = a.scale;

  {
    const T* Dg = reinterpret_cast<const T*>(a.D) + ((int64_t)c * H + h) * CH * CH;
    const T* Hg = reinterpret_cast<const T*>(a.Hq) + ((int64_t)c * H + h) * CH * CH;
    g2s<T, CH>(sD, PA, Dg, CH, CH, CH, tid, NTH);
    g2s<T, CH>(sHq, PA, Hg, CH, CH, CH, tid, NTH);
  }
  g2s<T, V>(sdO, PV, reinterpret_cast<const T*>(a.dO) + (t0 * H + h) * V, gsV, n, CH, tid, NTH);
  g2s<T, V>(sP, PV, reinterpret_cast<const T*>(a.P) + (t0 * H + h) * V, gsV, n, CH, tid, NTH);
  g2s<T, V>(sR, PV, reinterpret_cast<const T*>(a.R) + (t0 * H + h) * V, gsV, n, CH, tid, NTH);
  if (tid < CH) {
    sBeta[tid] = tid < n ? ld_beta(a.beta, a.beta_f32, (t0 + tid) * H + h) : 0.f;
    sDbe[tid] = 0.f;
    sGs[tid] = 0.f;
  }
  const T* hb = reinterpret_cast<const T*>(a.hbuf) + ((int64_t)c * H + h) * K * V;
  const T* dhb = reinterpret_cast<const T*>(a.dhbuf) + ((int64_t)c * H + h) * K * V;
  T* dqg = reinterpret_cast<T*>(a.dq) + (t0 * H + h) * K;
  T* dkg = reinterpret_cast<T*>(a.dk) + (t0 * H + h) * K;

  const int I = w;  // this wave owns token rows [16 I, 16 I + 16) of every output
  const bool rows_ok = I * SUB < n;
  float dbe[4] = {0.f, 0.f, 0.f, 0.f};

  for (int kt = 0; kt < NKT; ++kt) {
    const int kf0 = kt * KT;
    g2s<T, KT>(sK, PKT, reinterpret_cast<const T*>(a.k) + (t0 * H + h) * K + kf0, gsK, n, CH, tid,
               NTH);
    g2s<T, KT>(sQ, PKT, reinterpret_cast<const T*>(a.q) + (t0 * H + h) * K + kf0, gsK, n, CH, tid,
               NTH);
    if (tid < NSUB) sFlag[tid] = 0;
    load_gate_cumsum<KT>(sG, PGT, a, t0, h, n, K, kf0, tid, NTH);
    subchunk_stats<KT>(sG, PGT, n, sGf, sGl, sMid, sFlag, tid, NTH);
    // state endpoint part of lambda-bar: rowsum over V of S * dS+
    for (int idx = tid; idx < KT * 8; idx += NTH) {
      const int kk = idx >> 3, seg = idx & 7;
      float acc = 0.f;
      const T* hr = hb + (int64_t)(kf0 + kk) * V;
      const T* dr = dhb + (int64_t)(kf0 + kk) * V;
      for (int vv = seg; vv < V; vv += 8) acc += tof(hr[vv]) * tof(dr[vv]);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      acc += __shfl_xor(acc, 4);
      if (seg == 0) sLam0[kk] = acc;
    }
    __syncthreads();
    // scaled sending operands
    for (int idx = tid; idx < KT * CH; idx += NTH) {
      const int kk = idx / CH, j = idx - kk * CH, J = j / SUB;
      const float G = sG[j * PGT + kk];
      const float kv = tof(sK[j * PKT + kk]), qv = tof(sQ[j * PKT + kk]), b = sBeta[j];
      const float gl = sGl[J * KT + kk], gf = sGf[J * KT + kk], md = sMid[J * KT + kk];
      const bool cen = !sFlag[J];
      const float em = cen ? exp2f(md - G) : 0.f, ep = cen ? exp2f(G - md) : 0.f;
      const float val[6] = {kv * exp2f(gl - G), kv * em, b * kv * exp2f(G - gf), b * kv * ep,
                            scale * qv * exp2f(G - gf), scale * qv * ep};
#pragma unroll
      for (int o = 0; o < 6; ++o) {
        const T hi = fromf<T>(val[o]);
        sSc[o * NPART][kk * PA + j] = hi;
        if constexpr (BF) sSc[o * NPART + 1][kk * PA + j] = fromf<T>(val[o] - tof(hi));
      }
    }
    __syncthreads();

    for (int ct = 0; ct < CTK; ++ct) {
      const int kl = ct * SUB;     // feature offset inside the tile
      const int kf = kf0 + kl;     // feature offset in K
      const int kc = kl + ccol();  // this lane's feature inside the tile
      float lamw = 0.f;
      if (rows_ok) {
        // -- state products: contraction over V ------------------------------
        f32x4 SQ = zero4(), SE = zero4(), SF = zero4();
        mma_tile<T, true, true>(SQ, sdO + I * SUB * PV, PV, 1, hb + (int64_t)kf * V, V, 1, V);
        mma_tile<T, true, true>(SE, sP + I * SUB * PV, PV, 1, hb + (int64_t)kf * V, V, 1, V);
        mma_tile<T, true, true>(SF, sR + I * SUB * PV, PV, 1, dhb + (int64_t)kf * V, V, 1, V);
        // -- matrix intra, receiving block I ----------------------------------
        f32x4 XHY = zero4(), XDY = zero4(), XDE = zero4(), XHQ = zero4();
        const float gfI = sGf[I * KT + kc], glI = sGl[I * KT + kc], mdI = sMid[I * KT + kc];
        // acc += M-block (rows of this wave's block) x sending operand op (all parts)
        auto mm = [&](f32x4& acc, const T* m, int m_rs, int m_ks, int op, int src) {
#pragma unroll
          for (int pt = 0; pt < NPART; ++pt) {
            const T* B = sSc[op * NPART + pt] + kl * PA + src * SUB;
            if (m_ks == 1) mma_k16<T, true, true>(acc, m, m_rs, 1, B, PA, 1);
            else mma_k16<T, false, true>(acc, m, 1, m_ks, B, PA, 1);
          }
        };
        for (int J = 0; J < I; ++J) {  // sources before I: gamma (H Y), gamma (D Y)
          f32x4 tH = zero4(), tD = zero4();
          mm(tH, sHq + I * SUB * PA + J * SUB, PA, 1, KC_E, J);
          mm(tD, sD + I * SUB * PA + J * SUB, PA, 1, KC_E, J);
          const float cf = exp2f(gfI - sGl[J * KT + kc]);
          XHY += cf * tH;
          XDY += cf * tD;
        }
        for (int J2 = I + 1; J2 < NSUB && J2 * SUB < n; ++J2) {  // sources after I: transposed
          f32x4 tE = zero4(), tQ = zero4();
          mm(tE, sD + J2 * SUB * PA + I * SUB, 1, PA, KA_F, J2);   // D^T block, read strided
          mm(tQ, sHq + J2 * SUB * PA + I * SUB, 1, PA, QA_F, J2);
          const float cf = exp2f(sGf[J2 * KT + kc] - glI);
          XDE += cf * tE;
          XHQ += cf * tQ;
        }
        f32x4 Gv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = I * SUB + crow(i);
          Gv[i] = sG[row * PGT + kc];
          const float fr = exp2f(Gv[i] - gfI), fc = exp2f(glI - Gv[i]);
          XHY[i] *= fr;
          XDY[i] *= fr;
          XDE[i] *= fc;
          XHQ[i] *= fc;
        }
        // diagonal block I
        if (!sFlag[I]) {
          f32x4 tH = zero4(), tD = zero4(), tE = zero4(), tQ = zero4();
          mm(tH, sHq + I * SUB * PA + I * SUB, PA, 1, KC_M, I);
          mm(tD, sD + I * SUB * PA + I * SUB, PA, 1, KC_M, I);
          mm(tE, sD + I * SUB * PA + I * SUB, 1, PA, KA_M, I);
          mm(tQ, sHq + I * SUB * PA + I * SUB, 1, PA, QA_M, I);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float fr = exp2f(Gv[i] - mdI), fc = exp2f(mdI - Gv[i]);
            XHY[i] += fr * tH[i];
            XDY[i] += fr * tD[i];
            XDE[i] += fc * tE[i];
            XHQ[i] += fc * tQ[i];
          }
        } else {
          // pairwise exp2(G_i - G_j) inside the sub-chunk (all factors <= 1)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = I * SUB + crow(i);
            float sH = 0.f, sDv = 0.f, sE = 0.f, sQv = 0.f;
            for (int jj = 0; jj < SUB; ++jj) {
              const int r2 = I * SUB + jj;
              const float G2 = sG[r2 * PGT + kc];
              if (r2 <= row) {  // sending r2 -> receiving row
                const float f = exp2f(Gv[i] - G2) * tof(sK[r2 * PKT + kc]);
                sH += tof(sHq[row * PA + r2]) * f;
                sDv += tof(sD[row * PA + r2]) * f;
              }
              if (r2 >= row) {  // sending row -> receiving r2, transposed
                const float f = exp2f(G2 - Gv[i]);
                sE += tof(sD[r2 * PA + row]) * sBeta[r2] * tof(sK[r2 * PKT + kc]) * f;
                sQv += tof(sHq[r2 * PA + row]) * scale * tof(sQ[r2 * PKT + kc]) * f;
              }
            }
            XHY[i] += sH;
            XDY[i] += sDv;
            XDE[i] += sE;
            XHQ[i] += sQv;
          }
        }
        // -- chain rules --------------------------------------------------------
        const float Gn = sG[(n - 1) * PGT + kc];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = I * SUB + crow(i);
          float gb = 0.f;
          if (row < n) {
            const float gam = exp2f(Gv[i]), tail = exp2f(Gn - Gv[i]);
            const float XQ = gam * SQ[i] + XHY[i];
            const float XE = -gam * SE[i] + XDY[i];
            const float XY = XDE[i] + XHQ[i] + SF[i] * tail;
            const float qv = tof(sQ[row * PKT + kc]), kv = tof(sK[row * PKT + kc]);
            const float b = sBeta[row];
            dqg[row * gsK + kf + ccol()] = fromf<T>(scale * XQ);
            dkg[row * gsK + kf + ccol()] = fromf<T>(b * XE + XY);
            gb = scale * qv * XQ + b * kv * XE - kv * XY;
            dbe[i] += kv * XE;
            lamw += kv * SF[i] * tail;
          }
          sGb[row * PGT + kc] = gb;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) sGb[(I * SUB + crow(i)) * PGT + kc] = 0.f;
      }
      // key endpoint: column sum over this wave's rows of K * Fbar * exp2(Gn - G)
      lamw += __shfl_xor(lamw, 16);
      lamw += __shfl_xor(lamw, 32);
      if (l < 16) sLamW[w * KT + kc] = lamw;
    }
    __syncthreads();
    for (int kk = tid; kk < KT; kk += NTH) {
      const float Gn = sG[(n - 1) * PGT + kk];
      sGb[(n - 1) * PGT + kk] += exp2f(Gn) * sLam0[kk] + sLamW[kk] + sLamW[KT + kk] +
                                 sLamW[2 * KT + kk] + sLamW[3 * KT + kk];
    }
    __syncthreads();
    if (a.gate == 2) {
      for (int kk = tid; kk < KT; kk += NTH) {
        float run = 0.f;
        for (int i = n - 1; i >= 0; --i) {
          run += sGb[i * PGT + kk];
          a.dg[((t0 + i) * H + h) * K + kf0 + kk] = run;
        }
      }
    } else if (a.gate == 1) {
      for (int i = tid; i < n; i += NTH) {
        float s = 0.f;
        for (int kk = 0; kk < KT; ++kk) s += sGb[i * PGT + kk];
        sGs[i] += s;
      }
    }
    __syncthreads();
  }
  // erase part of dbeta: reduce over this wave's 16 feature lanes, rows are wave-owned
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x = dbe[i];
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    if ((l & 15) == 0 && rows_ok) sDbe[I * SUB + crow(i)] = x;
  }
  __syncthreads();
  if (tid < n) {
    const int64_t idx = (t0 + tid) * H + h;
    st_beta(a.dbeta, a.beta_f32, idx, a.dbw[idx] + sDbe[tid]);
  }
  if (a.gate == 1 && tid == 0) {
    float run = 0.f;
    for (int i = n - 1; i >= 0; --i) {
      run += sGs[i];
      a.dg[(t0 + i) * H + h] = run;
    }
  }
}

template <typename T>
static hipError_t prod_t(const Args& a, hipStream_t s) {
  const dim3 grid(a.nc_max, a.H), block(256);
  REWY_KV_SWITCH(k_bwd_prod)
}
template <typename T>
static hipError_t cons_t(const Args& a, hipStream_t s) {
  const dim3 grid(a.nc_max, a.H), block(256);
  REWY_KV_SWITCH(k_bwd_cons)
}

hipError_t launch_bwd_prod(const Args& a, int f32, hipStream_t s) {
  return f32 ? prod_t<float>(a, s) : prod_t<bf16>(a, s);
}
hipError_t launch_bwd_cons(const Args& a, int f32, hipStream_t s) {
  return f32 ? cons_t<float>(a, s) : cons_t<bf16>(a, s);
}

}  // namespace rewy
