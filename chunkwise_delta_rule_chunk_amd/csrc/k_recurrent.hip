// Token-serial (fused recurrent) forward, the form used to decode: the
// recurrence of the ReWY paper (Background / Delta-rule operators) and the KDA
// blog (section 4), one token at a time,
//   S~ = diag(exp g_t) S;   r_t = beta_t (v_t - S~^T k_t);   S = S~ + k_t r_t^T;   o_t = S^T (s q_t).
// The state never leaves the chip between tokens: one wave per (sequence,
// head, 64 value columns) holds its [K x 64] fp32 tile in registers, one
// state column per lane, from h0 to ht.  Per token the wave stages k, s q and
// the decay factors in LDS (two rows per lane, one exp2 each) and every lane
// then reads them as broadcasts; predict, correct, write and read are lane-
// local sums over K (four partial sums each for instruction-level
// parallelism).  Lanes past V work on a valid column and store nothing.
//
// EW: the erase/write form (ReWY paper Table 1, GDN2 row; GDN2 spec section 3,
// the recurrent kernel): r_t = w_t * v_t - S~^T (b_t * k_t) with an erase gate
// b per key feature (staged as b * k) and a write gate w per value column.
#include "chunk_common.hpp"

namespace rewy {

template <typename T, int K, int GATE, bool EW>
__global__ __launch_bounds__(64) void k_recurrent(Args a) {
  __shared__ __align__(16) float sk[K];  // k_t
  __shared__ __align__(16) float sq[K];  // s q_t
  __shared__ __align__(16) float sa[K];  // exp(g_t) per key row (vector gate)
  __shared__ __align__(16) float se[EW ? K : 4];  // erase/write form: b_t * k_t
  const int H = a.H, V = a.V;
  const int u = blockIdx.x, n = u / H, h = u - n * H;
  const int l = threadIdx.x, v = blockIdx.y * 64 + l;
  const bool on = v < V;
  const int vc = min(v, V - 1);
  // device cu_seqlens clamped to the packed token axis (never a token outside the inputs)
  const int BT = a.B * a.T;
  const int bos = a.cu ? min(max(a.cu[n], 0), BT) : n * a.T;
  const int eos = a.cu ? min(max(a.cu[n + 1], bos), BT) : (n + 1) * a.T;
  const int64_t sb = ((int64_t)n * H + h) * K * V + vc;  // state element (0, vc)
  const T* qg = reinterpret_cast<const T*>(a.q);
  const T* kg = reinterpret_cast<const T*>(a.k);
  const T* vg = reinterpret_cast<const T*>(a.v);
  const T* bg = reinterpret_cast<const T*>(a.beta);  // erase/write form: b [.., K]
  const T* wg = reinterpret_cast<const T*>(a.wg);    // erase/write form: w [.., V]
  T* og = reinterpret_cast<T*>(a.o);

  float S[K];
#pragma unroll
  for (int k = 0; k < K; ++k) S[k] = a.h0 ? a.h0[sb + (int64_t)k * V] : 0.f;

  for (int t = bos; t < eos; ++t) {
    const int64_t th = (int64_t)t * H + h;
#pragma unroll
    for (int r0 = 0; r0 < K; r0 += 64) {
      const int r = r0 + l;
      if (r < K) {
        const float kr = tof(kg[th * K + r]);
        sk[r] = kr;
        if constexpr (EW) se[r] = tof(bg[th * K + r]) * kr;
        sq[r] = a.scale * tof(qg[th * K + r]);
        if constexpr (GATE == 2) sa[r] = fexp2(a.g[th * K + r] * LOG2E);
      }
    }
    float decay = 1.f;
    if constexpr (GATE == 1) decay = fexp2(a.g[th] * LOG2E);
    const float b = EW ? 0.f : ld_beta(a.beta, a.beta_f32, th);
    const float wv = EW ? tof(wg[th * V + vc]) : 0.f;
    const float vt = tof(vg[th * V + vc]);
    __syncthreads();  // k, s q, exp(g) staged
    // decay and predict: p = (diag(exp g) S)^T k  (erase/write form: b * k)
    float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < K; k += 4) {
      const f32x4 kk = *reinterpret_cast<const f32x4*>((EW ? se : sk) + k);
      f32x4 dd;
      if constexpr (GATE == 2) dd = *reinterpret_cast<const f32x4*>(sa + k);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (GATE == 2) S[k + e] *= dd[e];
        else if constexpr (GATE == 1) S[k + e] *= decay;
        p[e] += S[k + e] * kk[e];
      }
    }
    // correct, write, read
    const float pr = (p[0] + p[1]) + (p[2] + p[3]);
    const float r = EW ? wv * vt - pr : b * (vt - pr);
    float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < K; k += 4) {
      const f32x4 kk = *reinterpret_cast<const f32x4*>(sk + k);
      const f32x4 qq = *reinterpret_cast<const f32x4*>(sq + k);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S[k + e] += kk[e] * r;
        o[e] += S[k + e] * qq[e];
      }
    }
    if (on) og[th * V + v] = fromf<T>((o[0] + o[1]) + (o[2] + o[3]));
    __syncthreads();  // the next token's staging overwrites k, s q, exp(g)
  }
  if (a.ht && on) {
#pragma unroll
    for (int k = 0; k < K; ++k) a.ht[sb + (int64_t)k * V] = S[k];
  }
}

template <typename T, int K, bool EW>
static hipError_t recurrent_e(const Args& a, hipStream_t s) {
  const dim3 grid(a.N * a.H, (a.V + 63) / 64), block(64);
  switch (a.gate) {
    case 0: REWY_LAUNCH((k_recurrent<T, K, 0, EW>), grid, block, s, a); break;
    case 1: REWY_LAUNCH((k_recurrent<T, K, 1, EW>), grid, block, s, a); break;
    case 2: REWY_LAUNCH((k_recurrent<T, K, 2, EW>), grid, block, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template <typename T, int K>
static hipError_t recurrent_k(const Args& a, hipStream_t s) {
  return a.ew ? recurrent_e<T, K, true>(a, s) : recurrent_e<T, K, false>(a, s);
}

template <typename T>
static hipError_t recurrent_t(const Args& a, hipStream_t s) {
  switch (a.K) {
    case 32: return recurrent_k<T, 32>(a, s);
    case 64: return recurrent_k<T, 64>(a, s);
    case 128: return recurrent_k<T, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_recurrent(const Args& a, int f32, hipStream_t s) {
  return f32 ? recurrent_t<float>(a, s) : recurrent_t<bf16>(a, s);
}

}  // namespace rewy
