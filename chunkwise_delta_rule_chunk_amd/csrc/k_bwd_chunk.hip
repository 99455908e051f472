// Chunk-parallel backward after the reverse scan: the ReWY shared-sensitivity
// producer, the gradient consumers and the gate reverse sum, fused into one
// workgroup per (chunk, head).  ReWY paper Algorithm 1 steps 1-4 and
// Appendices 7 and 10; KDA blog sections 6.3-6.5 for the gated operands.
//
//   P  = A^T Rbar                       shared sensitivity (no adjoint of A)
//   dv = beta * P,  dbeta_write_i = <V_i, P_i>
//   D  = -tril_strict(P R^T),  Hq = tril_incl(dO R^T)
//   Qgbar = dO S^T + Hq Y,  Ebar = -P S^T + D Y,  Ybar = D^T E + Hq^T Qg + Fbar Lambda,
//   Fbar = R dS+^T        (S = state entering the chunk, dS+ = adjoint of the state leaving it)
//   dq = s gamma Qgbar,  dk = beta gamma Ebar + Ybar / gamma,  dbeta_erase = <gamma K, Ebar>
//   Gbar = Qg Qgbar + E Ebar - Y Ybar,  plus at the last row
//          lambda = gamma_last * (rowsum(S * dS+) + colsum(Y * Fbar))
//   dg = reverse in-chunk cumulative sum of Gbar (summed over features for a scalar gate)
//
// Work split.  Wave I (of four) owns the token rows [16 I, 16 I + 16) of every
// output.  Its left operands D[I, :], Hq[I, :] and the transposed D[:, I]^T,
// Hq[:, I]^T are computed straight into MFMA operand registers: the C tile of
// M^T holds, lane by lane, exactly the A-operand fragment of M (lane l gets row
// l & 15 and four consecutive columns), so none of them goes through LDS.  The
// gated right operands (keys and queries times exp2 factors) are formed in
// registers from token-contiguous tiles, one 16-feature block at a time; a lane
// holds four consecutive tokens of one feature, which is the B-operand fragment
// of a 16-token contraction.
//
// Gate factors (ReWY paper section 3.3 and Appendix 8).  For receiving block I
// and an earlier sending block J the sending operand is K exp2(Gl_J - G), the
// column factor exp2(Gf_I - Gl_J) and the receiving factor exp2(G - Gf_I), where
// Gf and Gl are G2 at the block's first and last valid row: every factor is at
// most 1.  The transposed products mirror this with I and J exchanged.  A
// diagonal block is centred on its midpoint (max + min) / 2, and when some
// feature of the 16-feature block spans more than CENTRE_MAX_RANGE it is summed
// pairwise instead.  Sending operands are split into a high and a low bf16 part
// (x ~ hi + lo): the log-gate gradient is a difference of nearly equal
// receiving and sending sums, which amplifies operand rounding.
#include "chunk_common.hpp"

namespace rewy {

// GX = GATE + 4 EW + 8 GIN.  GATE: 0 none, 1 scalar, 2 vector (a template
// parameter: no gate tests in the loops).  EW: the erase/write form, with an
// erase gate b per (token, feature) in place of beta in E = b gamma K and a
// write gate w per (token, value) in Z = w V; it returns db = (gamma K) Ebar
// and dw = V P per element (ReWY paper Table 1, GDN2 row) and runs one
// workgroup per CU.  GIN (vector gate only): the gate was formed from its
// pre-activation, z = x + dt_bias, as g = -exp(A_log) softplus(z) (GDN2 spec
// section 4.4) or as the bounded g = lb sigmoid(exp(A_log) z) (section 3), and
// the chain rule is taken here: dx = (dg/dz) dg is written in place of dg, and
// each wave writes its partial sums of dA_log (sum of dg g for the softplus
// form, of dx z for the bounded form) and of ddt_bias = sum over tokens of dx,
// for a later reduction over chunks.
//
// GX & 16 (PROD) and GX & 32 (CONS) split the kernel for the separate
// schedule of the ReWY paper ("Execution and numerical precision", joint and
// separate consumers): PROD runs the producer only (P, dv, the write part of
// dbeta and D, written to the workspace; it needs no gate), CONS the
// consumers only (P, D and the write part of dbeta read back, Hq formed as
// in the joint kernel).  Every value is rounded at the same point in both
// schedules, so their results are bitwise equal.
// One workgroup per CU for the erase/write form and for fp32 (both need more
// than half of a SIMD's registers), two otherwise.
template <typename T, int V, int GX>
constexpr int bwd_chunk_wgs() {
  return ((GX & 4) || std::is_same_v<T, float>) ? 1 : 2;
}
template <typename T, int K, int V, int GX>
__global__ __launch_bounds__(256, (bwd_chunk_wgs<T, V, GX>())) void k_bwd_chunk(Args a) {
  constexpr int GATE = GX & 3;
  constexpr bool EW = GX & 4;
  constexpr bool GIN = GX & 8;
  constexpr bool PROD = GX & 16, CONS = GX & 32;
  static_assert(!GIN || (GATE == 2 && !EW), "the gate is formed in the kernel for the vector gate");
  static_assert(!(PROD && CONS) && (!(PROD || CONS) || (!EW && !GIN)),
                "the separate schedule serves the shared-beta forms");
  static_assert(!PROD || GATE == 0, "the producer does not depend on the gate");
  constexpr int NTH = 256;
  constexpr int PV = pitch<T>(V), PA = pitch<T>(CH);
  constexpr int NFB = K / SUB, NVB = V / SUB;
  static_assert(NFB % 2 == 0, "feature blocks are written in pairs");
  constexpr int KS = MM<T>::KS;
  constexpr int PD = SUB + 1;  // fp32 diagonal blocks for the pairwise path
  constexpr int SZ_AT = CH * PA * (int)sizeof(T), SZ_DG = NSUB * 2 * SUB * PD * 4;
  using FR = typename Frag4<T>::type;

  __shared__ __align__(16) T sO[CH * PV];  // dO
  __shared__ __align__(16) T sP[CH * PV];  // P
  __shared__ __align__(16) T sR[CH * PV];  // R
  __shared__ __align__(16) char sX[cmax(SZ_AT, SZ_DG)];  // A^T, then the diagonal blocks
  __shared__ __align__(16) T sBs[EW ? SUB * pitch<T>(CH) : 8];  // erase gate, [feature][token]
  __shared__ __align__(16) float sBeta[CH];
  __shared__ float sDbw[CH];
  __shared__ float sTot[2][NSUB * SUB], sLam[2][NSUB * SUB];  // per feature block, two buffers
  // One 16-feature block of per-feature operands, loaded once per workgroup
  // (every wave needs all of it): G2 [feature][token] (row 0 for a scalar
  // gate), K^T and Q^T [feature][token], the sub-chunk statistics [J][feature],
  // the state and state-adjoint rows [feature][v], and G2 at the last row.
  constexpr int PGS = CH + 4, PKS = pitch<T>(CH), PSS = pitch<T>(V);
  __shared__ __align__(16) float sG2[SUB * PGS];
  __shared__ __align__(16) T sKs[SUB * PKS];
  __shared__ __align__(16) T sQs[SUB * PKS];
  __shared__ __align__(16) float sSt[NSUB * SUB * 4];
  __shared__ __align__(16) T sSs[SUB * PSS];
  __shared__ __align__(16) T sDs[SUB * PSS];
  __shared__ __align__(16) float sGn[SUB];

  const int H = a.H;
  const int c = blockIdx.x / H, h = blockIdx.x - c * H;
  const ChunkInfo ci = load_chunk(a.chunks, c);
  const int n = ci.len;
  if (n == 0) {
    // gate in the kernel: an empty slot adds zero to the parameter gradients
    if constexpr (GIN) {
      float* gp = a.gpart + ((int64_t)c * H + h) * NSUB * K;
      for (int i = threadIdx.x; i < NSUB * K; i += 256) gp[i] = 0.f;
      if (threadIdx.x < NSUB) a.gpart[(int64_t)a.nc_max * H * NSUB * K + ((int64_t)c * H + h) * NSUB + threadIdx.x] = 0.f;
    }
    return;
  }
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int q4 = l >> 4, f = l & 15;
  const int I = w;  // row block of this wave
  const bool live = I * SUB < n;
  const int64_t t0 = ci.bos, cb = (int64_t)c * H + h;
  const int64_t gsK = (int64_t)H * K, gsV = (int64_t)H * V;
  const float scale = a.scale;
  T* sAt = reinterpret_cast<T*>(sX);
  float* sDiag = reinterpret_cast<float*>(sX) + w * 2 * SUB * PD;  // [D_II | Hq_II], this wave

  // ---- loads: every read of the first phase is issued before the first wait.
  // Rows past the chunk's end read as zero (bounds-checked buffer loads).
  const GBuf bv = gbuf(reinterpret_cast<const T*>(a.v) + (t0 * H + h) * V, tile_bytes<T>(n, gsV, V));
  const int k0a = (I * SUB / KS) * KS;  // A^T is upper triangular: tokens j >= 16 I
  {
    // the producer reads no dO; the consumers read P (and the write part of
    // dbeta) in place of A^T and Rbar
    TileRegs<T, CH, V, NTH> pO, pR, pP;
    TileRegs<T, CH, CH, NTH> pA;
    if constexpr (!PROD)
      pO.load(gbuf(reinterpret_cast<const T*>(a.dO) + (t0 * H + h) * V, tile_bytes<T>(n, gsV, V)), gsV, tid);
    // R per chunk-head, column-blocked [V/16][64][16], zero past the chunk's end
    pR.load_cb(gbuf(reinterpret_cast<const T*>(a.R) + cb * V * CH, V * CH * sizeof(T)), CH, 0, tid);
    if constexpr (!CONS)
      pA.load(gbuf(reinterpret_cast<const T*>(a.At) + cb * CH * CH, CH * CH * sizeof(T)), CH, tid);
    else
      pP.load(gbuf(reinterpret_cast<const T*>(a.Pbuf) + cb * CH * V, CH * V * sizeof(T)), V, tid);
    const uint32_t braw = EW ? 0u : ld_beta_raw(a.beta, a.beta_f32, (t0 + min(tid, n - 1)) * H + h);
    const float dbwr = CONS ? a.dbw[cb * CH + (tid & (CH - 1))] : 0.f;
    if constexpr (!PROD) pO.store(sO, PV, tid);
    pR.store_cb(sR, PV, tid);
    if constexpr (!CONS) pA.store(sAt, PA, tid);
    else pP.store(sP, PV, tid);
    if (tid < CH) sBeta[tid] = (tid < n && !EW) ? beta_val(braw, a.beta_f32) : 0.f;
    if (CONS && tid < CH) sDbw[tid] = dbwr;
  }

  // ---- P = A^T Rbar, rows of block I; dv and the write part of dbeta --------
  // The tile computed is P^T (rows v, columns i): its C fragment gives lane l
  // row i = 16 I + (l & 15) and the four columns v0 .. v0 + 3, v0 = 16 vb + 4 (l >> 4).
  // All value blocks are computed first, then each row of dv is written in one
  // sweep (whole rows reach the cache together and leave it as full lines).
  // The producer of the separate schedule also writes P (rounded as the
  // consumers read it) and the write part of dbeta to the workspace.
  if constexpr (!CONS) {
    const T* Rbt = reinterpret_cast<const T*>(a.Rbt) + cb * V * CH;
    const GBuf bdv = gbuf(reinterpret_cast<T*>(a.dv) + (t0 * H + h) * V, tile_bytes<T>(n, gsV, V));
    const int k0 = k0a;
    const int i = I * SUB + f;
    // this lane's four values of v in each value block (zero past the end)
    using VR = std::conditional_t<std::is_same_v<T, bf16>, uint2, uint4>;
    VR vr[NVB], wr[EW ? NVB : 1];  // v and (erase/write form) the write gate
    const GBuf bw = gbuf(reinterpret_cast<const T*>(a.wg) + (t0 * H + h) * V, EW ? tile_bytes<T>(n, gsV, V) : 0u);
    static_for<0, NVB>([&](auto vb) {
      const uint32_t off = (uint32_t)(((int64_t)i * gsV + vb * SUB + 4 * q4) * (int64_t)sizeof(T));
      if constexpr (std::is_same_v<T, bf16>) vr[vb] = gld8(bv, off);
      else vr[vb] = gld16(bv, off);
      if constexpr (EW) {
        if constexpr (std::is_same_v<T, bf16>) wr[vb] = gld8(bw, off);
        else wr[vb] = gld16(bw, off);
      }
    });
    // Rbar is stored in the C-fragment order of its 16 x 16 tiles [token block
    // T][v block]: lane l's piece of tile (vb, T) holds Rbar[16 T + 4 (l >> 4) + e]
    // [16 vb + (l & 15)], e < 4, which is the 16-long A fragment of Rbar^T.
    const GBuf brb = gbuf(Rbt, V * CH * sizeof(T));
    auto rb_off = [&](int vb, int tb, bool use) {
      return use ? (uint32_t)((((vb * NSUB + tb) * 64 + l) * 4) * (int)sizeof(T)) : OOB;
    };
    f32x4 acc[NVB];
    if constexpr (std::is_same_v<T, bf16>) {
      // bf16: at most two 32-token steps, every Rbar fragment requested up
      // front (unused steps read as zero).  A step joins token blocks 2 st and
      // 2 st + 1: slots 8 q4 + e take token 32 st + 4 q4 + e and slots
      // 8 q4 + 4 + e token 32 st + 16 + 4 q4 + e, in both operands.
      bf16x8 rb[NVB][2];
      static_for<0, NVB>([&](auto vb) {
        static_for<0, 2>([&](auto st) {
          const bool use = live && st * 32 >= k0;
          const uint2 x0 = gld8(brb, rb_off(vb, 2 * st, use)), x1 = gld8(brb, rb_off(vb, 2 * st + 1, use));
          rb[vb][st] = __builtin_bit_cast(bf16x8, uint4{x0.x, x0.y, x1.x, x1.y});
        });
      });
      lds_barrier();
      auto atf = [&](int st) {
        const T* p = sAt + (I * SUB + f) * PA + 32 * st + 4 * q4;
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p), hi = *reinterpret_cast<const bf16x4*>(p + SUB);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      const bf16x8 at0 = atf(0), at1 = atf(1);
      static_for<0, NVB>([&](auto vb) {
        acc[vb] = mma(rb[vb][1], at1, zero4());
        if (k0 == 0) acc[vb] = mma(rb[vb][0], at0, acc[vb]);
      });
    } else {
      // fp32: one 16-token product per token block T >= I (A^T is upper
      // triangular), the others read as zero
      lds_barrier();
      static_for<0, NVB>([&](auto vb) {
        f32x4 rb[NSUB];
        static_for<0, NSUB>([&](auto tb) {
          rb[tb] = __builtin_bit_cast(f32x4, gld16(brb, rb_off(vb, tb, live && tb >= I)));
        });
        acc[vb] = zero4();
        static_for<0, NSUB>([&](auto tb) {
          mm16(acc[vb], rb[tb], *reinterpret_cast<const f32x4*>(sAt + (I * SUB + f) * PA + SUB * tb + 4 * q4));
        });
      });
    }
    const float b = sBeta[i];
    float dbw = 0.f;
    const GBuf bpo = gbuf(reinterpret_cast<T*>(a.Pbuf) + cb * CH * V, PROD ? CH * V * sizeof(T) : 0u);
    static_for<0, NVB>([&](auto vb) {
      const int v0 = vb * SUB + 4 * q4;
      *reinterpret_cast<FR*>(sP + i * PV + v0) = to_frag<T>(acc[vb]);
      if constexpr (PROD) {
        const uint32_t off = (uint32_t)((i * V + v0) * (int)sizeof(T));
        if constexpr (std::is_same_v<T, bf16>) gst8(bpo, off, __builtin_bit_cast(uint2, to_frag<T>(acc[vb])));
        else gst16(bpo, off, __builtin_bit_cast(uint4, acc[vb]));
      }
      const FR x = __builtin_bit_cast(FR, vr[vb]);
#pragma unroll
      for (int e = 0; e < 4; ++e) dbw += tof(x[e]) * acc[vb][e];
    });
    // rows past the chunk's end fall outside the buffer and are dropped.
    // Erase/write form: dv = w P and dw = v P, element by element.
    const GBuf bdw = gbuf(reinterpret_cast<T*>(a.dw) + (t0 * H + h) * V, EW ? tile_bytes<T>(n, gsV, V) : 0u);
    static_for<0, NVB>([&](auto vb) {
      const uint32_t off = (uint32_t)(((int64_t)i * gsV + vb * SUB + 4 * q4) * (int64_t)sizeof(T));
      f32x4 dvv = b * acc[vb], dww = zero4();
      if constexpr (EW) {
        const FR wx = __builtin_bit_cast(FR, wr[vb]), vx = __builtin_bit_cast(FR, vr[vb]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dvv[e] = tof(wx[e]) * acc[vb][e];
          dww[e] = tof(vx[e]) * acc[vb][e];
        }
      }
      const FR y = to_frag<T>(dvv);
      if constexpr (std::is_same_v<T, bf16>) gst8(bdv, off, __builtin_bit_cast(uint2, y));
      else gst16(bdv, off, __builtin_bit_cast(uint4, y));
      if constexpr (EW) {
        const FR z = to_frag<T>(dww);
        if constexpr (std::is_same_v<T, bf16>) gst8(bdw, off, __builtin_bit_cast(uint2, z));
        else gst16(bdw, off, __builtin_bit_cast(uint4, z));
      }
    });
    dbw = rows_sum(dbw);
    if (q4 == 0) {
      if constexpr (PROD) a.dbw[cb * CH + i] = dbw;
      else sDbw[i] = dbw;
    }
  }
  lds_barrier();  // P complete (loaded, for the consumers); A^T is dead

  // ---- the first feature block's operands --------------------------------------
  // requested here in the joint schedule, so that their latency overlaps the
  // D and H_q products (the consumers of the separate schedule read D first)
  const T* hb = reinterpret_cast<const T*>(a.hbuf) + cb * K * V;
  const T* dhb = reinterpret_cast<const T*>(a.dhbuf) + cb * K * V;
  // raw k and q rows of the chunk (rows past the end read as zero)
  const GBuf bk = gbuf(reinterpret_cast<const T*>(a.k) + (t0 * H + h) * K, tile_bytes<T>(n, gsK, K));
  const GBuf bq = gbuf(reinterpret_cast<const T*>(a.q) + (t0 * H + h) * K, tile_bytes<T>(n, gsK, K));
  const float* Gstg = a.Gst + cb * NSUB * K * 4;  // float4 records, [J][K]
  const GBuf bgx = gbuf(reinterpret_cast<const T*>(a.gx) + (t0 * H + h) * K, GIN ? tile_bytes<T>(n, gsK, K) : 0u);
  const GBuf bdt = gbuf(a.dt_bias + (int64_t)h * K, GIN ? K * 4 : 0u);
  // registers of the next block's operands (loaded during this block's
  // products).  Every load is unconditional: a scalar gate has one G2 row
  // (the others read as zero) and no gate reads none.
  TileRegs<float, SUB, CH, NTH> pG;
  // A vector gate: G2 of the feature block is rebuilt here (the prep keeps
  // only its sub-chunk statistics).  Wave w takes rows [16 w, 16 w + 16):
  // lane (q4, f) reads g at rows 16 w + 4 q4 + e of feature 16 fb + f (the
  // gate formed in the kernels: x there and dt_bias of the feature, g formed
  // as in the prep) and G2 at the block's first row (its statistics record;
  // zero for a block past the chunk's end, whose G2 is never used).  The
  // scalar gate reads the prep's G2 row.
  constexpr bool GRAW = GATE == 2;
  uint32_t graw[GRAW ? 4 : 1], gfw = 0u, gdw = 0u;
  const GBuf bgr = gbuf(a.g + (t0 * H + h) * K, GRAW && !GIN ? tile_bytes<float>(n, gsK, K) : 0u);
  const GBuf bgf = gbuf(Gstg, GRAW ? (uint32_t)(((n + SUB - 1) / SUB) * K * 16) : 0u);
  // k and q of a feature block from their natural rows: a piece is KQV
  // features of one token; the first half of the pieces is k, the second q
  // (uniform per wave), transposed into [feature][token] when stored
  constexpr int KQV = 16 / (int)sizeof(T), KQR = SUB / KQV;  // features per piece, pieces per row
  constexpr int KQP = 2 * CH * KQR, KQN = KQP / NTH;         // pieces, per thread
  static_assert(KQP % NTH == 0 && (CH * KQR) % 64 == 0, "k/q pieces");
  uint4 pkq[KQN];
  // erase/write form: the erase gate of the feature block, like k (a piece
  // is KQV features of one token; only the first CH KQR pieces exist)
  constexpr int BQN = EW ? (CH * KQR + NTH - 1) / NTH : 1;
  static_assert((CH * KQR) % 64 == 0, "erase-gate pieces");
  uint4 pbq[BQN];
  const GBuf bbk = gbuf(reinterpret_cast<const T*>(a.beta) + (t0 * H + h) * K, EW ? tile_bytes<T>(n, gsK, K) : 0u);
  TileRegs<float, NSUB, SUB * 4, NTH> pX;
  TileRegs<T, SUB, V, NTH> pS, pD;
  TileRegs<float, 1, SUB, NTH> pN;
  // the scalar gate's G2 row [64] (rows 1 .. 15 of the tile read as zero and
  // are not used)
  const float* gp = a.G2t + cb * CH;
  const uint32_t gbytes = GATE == 1 ? CH * 4 : 0;
  auto fetch_fb = [&](int fb) {
    if constexpr (GRAW) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t el = (int64_t)(w * SUB + 4 * q4 + e) * gsK + fb * SUB + f;
        if constexpr (!GIN) graw[e] = gld4(bgr, (uint32_t)(el * 4));
        else if constexpr (sizeof(T) == 2) graw[e] = gld2(bgx, (uint32_t)(el * 2));
        else graw[e] = gld4(bgx, (uint32_t)(el * 4));
      }
      if constexpr (GIN) gdw = gld4(bdt, (uint32_t)((fb * SUB + f) * 4));
      gfw = gld4(bgf, (uint32_t)(((w * K + fb * SUB + f) * 4) * 4));
    } else {
      pG.load_cb(gbuf(gp, gbytes), 1, 0, tid);
    }
#pragma unroll
    for (int j = 0; j < KQN; ++j) {
      const int pc = tid + j * NTH, rem = pc % (CH * KQR);
      const int t = rem / KQR, f0 = (rem % KQR) * KQV;
      const uint32_t off = (uint32_t)(((int64_t)t * gsK + fb * SUB + f0) * (int64_t)sizeof(T));
      // k or q is the same for the whole wave (64 consecutive pieces)
      const bool isk = __builtin_amdgcn_readfirstlane(pc) < CH * KQR;
      pkq[j] = gld16(isk ? bk : bq, off);
    }
    if constexpr (EW) {
#pragma unroll
      for (int j = 0; j < BQN; ++j) {
        const int pc = tid + j * NTH, t = pc / KQR, f0 = (pc % KQR) * KQV;
        pbq[j] = gld16(bbk, pc < CH * KQR ? (uint32_t)(((int64_t)t * gsK + fb * SUB + f0) * (int64_t)sizeof(T)) : OOB);
      }
    }
    pX.load(gbuf(Gstg + fb * SUB * 4, tile_bytes<float>(NSUB, K * 4, SUB * 4)), K * 4, tid);
    pS.load_cb(gbuf(hb, K * V * sizeof(T)), K, fb * SUB, tid);
    pD.load_cb(gbuf(dhb, K * V * sizeof(T)), K, fb * SUB, tid);
    pN.load(gbuf(a.glast + cb * K + fb * SUB, SUB * sizeof(float)), SUB, tid);
  };
  if constexpr (!PROD && !CONS) fetch_fb(0);

  // ---- left operands of block I, straight into fragments ---------------------
  //   Dm[J]  = D[I, J]      (J <= I)    Hm[J]  = Hq[I, J]      (J <= I)
  //   Dtm[J] = D[J, I]^T    (J >= I)    Htm[J] = Hq[J, I]^T    (J >= I)
  // The fragment of M is the C tile of M^T; lane l holds M(l & 15, 4 (l >> 4) + e).
  FR Dm[NSUB], Hm[NSUB], Dtm[NSUB], Htm[NSUB];
  f32x4 ddiag = zero4();  // this lane's four values of the diagonal block D_II (fp32)
  static_for<0, NSUB>([&](auto J) {
    Dm[J] = Hm[J] = Dtm[J] = Htm[J] = to_frag<T>(zero4());
    if (!live || J * SUB >= n) return;
    if (J <= I) {
      f32x4 yd = zero4(), yh = zero4();
      if constexpr (!CONS) mma_tile<T, true, true>(yd, sR + J * SUB * PV, PV, 1, sP + I * SUB * PV, PV, 1, V);
      if constexpr (!PROD) mma_tile<T, true, true>(yh, sR + J * SUB * PV, PV, 1, sO + I * SUB * PV, PV, 1, V);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jj = 4 * q4 + e;  // column of M inside block J; row is f
        yd[e] = (J < I || jj < f) ? -yd[e] : 0.f;
        yh[e] = (J < I || jj <= f) ? yh[e] : 0.f;
        if (J == I) {
          if constexpr (!CONS) sDiag[f * PD + jj] = ddiag[e] = yd[e];
          if constexpr (!PROD) sDiag[SUB * PD + f * PD + jj] = yh[e];
        }
      }
      Dm[J] = to_frag<T>(yd);
      Hm[J] = to_frag<T>(yh);
    }
    if (J >= I) {
      f32x4 yd = zero4(), yh = zero4();
      if constexpr (!CONS) mma_tile<T, true, true>(yd, sP + J * SUB * PV, PV, 1, sR + I * SUB * PV, PV, 1, V);
      if constexpr (!PROD) mma_tile<T, true, true>(yh, sO + J * SUB * PV, PV, 1, sR + I * SUB * PV, PV, 1, V);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int jj = 4 * q4 + e;
        yd[e] = (J > I || jj > f) ? -yd[e] : 0.f;
        yh[e] = (J > I || jj >= f) ? yh[e] : 0.f;
      }
      Dtm[J] = to_frag<T>(yd);
      Htm[J] = to_frag<T>(yh);
    }
  });
  // Separate schedule: D leaves the producer as the operand fragments the
  // consumers use, [wave I][J][D[I, J] | D[J, I]^T][lane][4] in the feature
  // dtype, and its diagonal blocks in fp32, [I][16 rows][16]; the consumers
  // read them back in place of computing D.
  if constexpr (PROD || CONS) {
    constexpr int FB = 4 * (int)sizeof(T);  // bytes of one lane's fragment
    const GBuf bdf = gbuf(reinterpret_cast<T*>(a.Dfrag) + cb * NSUB * NSUB * 2 * 64 * 4,
                          NSUB * NSUB * 2 * 64 * FB);
    const GBuf bdd = gbuf(a.Ddiag + cb * NSUB * SUB * SUB, NSUB * SUB * SUB * 4);
    auto foff = [&](int J, int kind) { return (uint32_t)((((I * NSUB + J) * 2 + kind) * 64 + l) * FB); };
    const uint32_t doff = (uint32_t)((I * SUB * SUB + f * SUB + 4 * q4) * 4);
    if constexpr (PROD) {
      static_for<0, NSUB>([&](auto J) {
        if constexpr (std::is_same_v<T, bf16>) {
          gst8(bdf, foff(J, 0), __builtin_bit_cast(uint2, Dm[J]));
          gst8(bdf, foff(J, 1), __builtin_bit_cast(uint2, Dtm[J]));
        } else {
          gst16(bdf, foff(J, 0), __builtin_bit_cast(uint4, Dm[J]));
          gst16(bdf, foff(J, 1), __builtin_bit_cast(uint4, Dtm[J]));
        }
      });
      gst16(bdd, doff, __builtin_bit_cast(uint4, ddiag));
      return;  // every wave of the producer ends here
    } else {
      static_for<0, NSUB>([&](auto J) {
        if constexpr (std::is_same_v<T, bf16>) {
          Dm[J] = __builtin_bit_cast(FR, gld8(bdf, foff(J, 0)));
          Dtm[J] = __builtin_bit_cast(FR, gld8(bdf, foff(J, 1)));
        } else {
          Dm[J] = __builtin_bit_cast(FR, gld16(bdf, foff(J, 0)));
          Dtm[J] = __builtin_bit_cast(FR, gld16(bdf, foff(J, 1)));
        }
      });
      ddiag = __builtin_bit_cast(f32x4, gld16(bdd, doff));
#pragma unroll
      for (int e = 0; e < 4; ++e) sDiag[f * PD + 4 * q4 + e] = ddiag[e];
    }
  }
  lds_barrier();  // diagonal blocks in sDiag visible to every lane of the wave

  // ---- per 16-feature block: state products, matrix intra, chain rules -------
  // The gate reverse sum needs the block totals of the later row blocks: they
  // are exchanged through LDS once per feature block (all waves take part).
  // outputs through bounds-checked buffers: rows past the chunk's end are dropped
  const GBuf bdq = gbuf(reinterpret_cast<T*>(a.dq) + (t0 * H + h) * K, tile_bytes<T>(n, gsK, K));
  const GBuf bdk = gbuf(reinterpret_cast<T*>(a.dk) + (t0 * H + h) * K, tile_bytes<T>(n, gsK, K));
  const GBuf bdg = gbuf(a.dg + (t0 * H + h) * K, GATE == 2 && !GIN ? tile_bytes<float>(n, gsK, K) : 0u);
  // gate in the kernel: dx (like dq), the pre-activation and dt_bias of this
  // lane's row and four features, the wave's partial sums
  const GBuf bdx = gbuf(reinterpret_cast<T*>(a.dgx) + (t0 * H + h) * K, GIN ? tile_bytes<T>(n, gsK, K) : 0u);
  const GBuf bgp = gbuf(a.gpart + cb * NSUB * K, GIN ? NSUB * K * 4 : 0u);
  const float nea = GIN ? -fexp2(__uint_as_float(gld4(gbuf(a.a_log, H * 4), h * 4)) * LOG2E) : 0.f;
  const float lb = GIN ? a.gate_lb : 0.f, lbea = -lb * nea;  // bounded form: lb exp(A_log)
  float dal = 0.f;                 // gate in the kernel: this lane's part of the dA_log sum
  FR pdx = to_frag<T>(zero4());    // dx of the previous (even) feature block
  const int jl = n - 1;  // last valid row
  const FR DmI = pick(Dm, I), HmI = pick(Hm, I), DtmI = pick(Dtm, I), HtmI = pick(Htm, I);
  const f32x4 bIb = *reinterpret_cast<const f32x4*>(sBeta + I * SUB + 4 * q4);  // beta, rows of block I
  f32x4 sufs = zero4();  // scalar gate: Gbar summed over features, this lane's rows
  float dbe[4] = {0.f, 0.f, 0.f, 0.f};
  // dq, dk of the previous feature blocks of this group, transposed (see
  // below): a group is the blocks that fill whole 128-byte lines of a row,
  // four in bf16 and two in fp32
  constexpr int QG = cmin(128 / (SUB * (int)sizeof(T)), NFB);
  static_assert(NFB % QG == 0, "whole groups of feature blocks");
  FR pdq[QG - 1], pdk[QG - 1];
#pragma unroll
  for (int j = 0; j < QG - 1; ++j) pdq[j] = pdk[j] = to_frag<T>(zero4());
  FR pdb = to_frag<T>(zero4());
  f32x4 pdg = zero4();  // dg of the previous (even) feature block
  // erase/write form: db of this lane's rows, stored like dk
  const GBuf bdb = gbuf(reinterpret_cast<T*>(a.dbeta) + (t0 * H + h) * K, EW ? tile_bytes<T>(n, gsK, K) : 0u);
  // identity as the B operand of a 16-long product: C = X^T I turns this
  // lane's C-tile values (rows 4 q4 + e, feature f) into the transposed
  // layout (row f, features 4 q4 .. + 3), exactly (one term per output)
  f32x4 idf;
#pragma unroll
  for (int e = 0; e < 4; ++e) idf[e] = (4 * q4 + e == f) ? 1.f : 0.f;
  const FR idt = to_frag<T>(idf);
  float lam0s = 0.f, lamws = 0.f;

  auto put_fb = [&]() {
    if constexpr (GRAW) {
      // G2 = G2 at the first row + log2(e) times the sum of g over the later
      // rows up to this one (in-lane over four rows, then the lane rows before)
      f32x4 gv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (GIN) {  // g = -ea softplus(z) or lb sigmoid(ea z), z = x + dt_bias; zero past the end
          const float z = (sizeof(T) == 2 ? __uint_as_float(graw[e] << 16) : __uint_as_float(graw[e])) +
                          __uint_as_float(gdw);
          const float gg = lb == 0.f ? nea * softplus(z) : lb * sigmoid_f(-nea * z);
          gv[e] = w * SUB + 4 * q4 + e < n ? gg : 0.f;
        } else {
          gv[e] = __uint_as_float(graw[e]);
        }
      }
      f32x4 x;
      x[0] = q4 == 0 ? 0.f : gv[0];
#pragma unroll
      for (int e = 1; e < 4; ++e) x[e] = x[e - 1] + gv[e];
      const float off = rows_prefix_excl(x[3], q4), gf = __uint_as_float(gfw);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = gf + LOG2E * (off + x[e]);
      *reinterpret_cast<f32x4*>(sG2 + f * PGS + w * SUB + 4 * q4) = x;
    } else if constexpr (GATE != 0) {
      pG.store_cb(sG2, PGS, tid);
    }
#pragma unroll
    for (int j = 0; j < KQN; ++j) {
      const int pc = tid + j * NTH, rem = pc % (CH * KQR);
      const int t = rem / KQR, f0 = (rem % KQR) * KQV;
      union {
        uint4 u;
        T e[KQV];
      } x;
      x.u = pkq[j];
      T* dst = (pc < CH * KQR ? sKs : sQs) + f0 * PKS + t;
#pragma unroll
      for (int e = 0; e < KQV; ++e) dst[e * PKS] = x.e[e];
    }
    if constexpr (EW) {
#pragma unroll
      for (int j = 0; j < BQN; ++j) {
        const int pc = tid + j * NTH, t = pc / KQR, f0 = (pc % KQR) * KQV;
        if (pc < CH * KQR) {  // whole waves
          union {
            uint4 u;
            T e[KQV];
          } x;
          x.u = pbq[j];
#pragma unroll
          for (int e = 0; e < KQV; ++e) sBs[(f0 + e) * PKS + t] = x.e[e];
        }
      }
    }
    pX.store(sSt, SUB * 4, tid);
    pS.store_cb(sSs, PSS, tid);
    pD.store_cb(sDs, PSS, tid);
    pN.store(sGn, SUB, tid);
  };
  if constexpr (PROD || CONS) fetch_fb(0);  // the joint schedule issued it before D and H_q
  put_fb();
  lds_barrier();

#pragma unroll 1
  for (int fb = 0; fb < NFB; ++fb) {
    const int kc = fb * SUB + f;  // this lane's feature
    const int buf = fb & 1;
    fetch_fb(min(fb + 1, NFB - 1));  // the last block reads itself again, unused
    // gate in the kernel: x at (row 16 I + f, features 16 fb + 4 q4 .. + 3)
    // and dt_bias of those features, used after the block's reverse sum
    uint4 xr = {0u, 0u, 0u, 0u}, dtr = {0u, 0u, 0u, 0u};
    if constexpr (GIN) {
      const uint32_t xo = (uint32_t)(((int64_t)(I * SUB + f) * gsK + fb * SUB + 4 * q4) * (int64_t)sizeof(T));
      if constexpr (sizeof(T) == 2) {
        const uint2 x2 = gld8(bgx, xo);
        xr.x = x2.x;
        xr.y = x2.y;
      } else {
        xr = gld16(bgx, xo);
      }
      dtr = gld16(bdt, (uint32_t)((fb * SUB + 4 * q4) * 4));
    }
    // first row of this lane, opaque per iteration: the output addresses derived
    // from it are recomputed rather than kept live (and spilled) across blocks
    int lrow = I * SUB + 4 * q4;
    asm volatile("" : "+v"(lrow));
    f32x4 gbar = zero4();
    float lamw = 0.f, l0 = 0.f;
    float oq[4] = {0.f, 0.f, 0.f, 0.f}, ok_[4] = {0.f, 0.f, 0.f, 0.f};  // dq, dk of this block
    float ob[4] = {0.f, 0.f, 0.f, 0.f};  // erase/write form: db of this block
    if (live) {
      // gated operands of all four blocks at this lane's rows 16 J + 4 q4 + e
      // (k and q stay packed in their storage type until used)
      f32x4 G[NSUB];
      FR kp[NSUB], qp[NSUB], bp[NSUB];
      static_for<0, NSUB>([&](auto J) {
        const int r0 = J * SUB + 4 * q4;
        if constexpr (GATE == 2)
          G[J] = *reinterpret_cast<const f32x4*>(sG2 + f * PGS + r0);
        else if constexpr (GATE == 1)
          G[J] = *reinterpret_cast<const f32x4*>(sG2 + r0);
        else
          G[J] = zero4();
        kp[J] = *reinterpret_cast<const FR*>(sKs + f * PKS + r0);
        qp[J] = *reinterpret_cast<const FR*>(sQs + f * PKS + r0);
        if constexpr (EW) bp[J] = *reinterpret_cast<const FR*>(sBs + f * PKS + r0);
      });
      auto unpack = [](const FR& x) {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = tof(x[e]);
        return r;
      };
      // sub-chunk statistics of this feature (written by the forward prep):
      // G2 at the first and last valid row, midpoint, range; only blocks with
      // valid rows are used
      float Gf[NSUB], Gl[NSUB];
      f32x4 stJ[NSUB];
      static_for<0, NSUB>([&](auto J) {
        stJ[J] = zero4();
        if (J * SUB < n) stJ[J] = *reinterpret_cast<const f32x4*>(sSt + (J * SUB + f) * 4);
        Gf[J] = stJ[J][0];
        Gl[J] = stJ[J][1];
      });
      const float Gn = sGn[f];
      // Block I's own operands and statistics.  Read again at the wave's own
      // (uniform) offsets, which costs fewer instructions than selecting them
      // from the arrays above; the gate formed in the kernel keeps the
      // selection (its extra registers would not fit beside the re-reads).
      const int rI = I * SUB + 4 * q4;
      f32x4 GI, kI, qI, stI, bI = bIb;
      if constexpr (GIN) {
        GI = pick(G, I);
        kI = unpack(pick(kp, I));
        qI = unpack(pick(qp, I));
        stI = pick(stJ, I);
      } else {
        GI = zero4();
        if constexpr (GATE == 2) GI = *reinterpret_cast<const f32x4*>(sG2 + f * PGS + rI);
        else if constexpr (GATE == 1) GI = *reinterpret_cast<const f32x4*>(sG2 + rI);
        kI = unpack(*reinterpret_cast<const FR*>(sKs + f * PKS + rI));
        qI = unpack(*reinterpret_cast<const FR*>(sQs + f * PKS + rI));
        // erase factor of this lane's rows: beta per row, or b per (row, feature)
        if constexpr (EW) bI = unpack(*reinterpret_cast<const FR*>(sBs + f * PKS + rI));
        stI = *reinterpret_cast<const f32x4*>(sSt + (I * SUB + f) * 4);  // live: I * SUB < n
      }
      const float GfI = stI[0], GlI = stI[1], MdI = stI[2];
      const bool wideI = __any(stI[3] > CENTRE_MAX_RANGE);
      // Row factors of block I.  Centred block: xp = exp2(G - Md), xm = exp2(Md - G)
      // (each at most 2^(range/2)), and the receiving factors follow by per-lane
      // constants, fr = exp2(G - Gf) = xp exp2(Md - Gf), fc = exp2(Gl - G) =
      // xm exp2(Gl - Md), tail = exp2(Gn - G) = xm exp2(Gn - Md).  A wide block
      // forms fr, fc and tail directly (xp and xm are not used there).
      f32x4 xp, xm, fr, fc, tail;
      if (!wideI) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xp[e] = fexp2(GI[e] - MdI);
          xm[e] = fexp2(MdI - GI[e]);
        }
        fr = xp * fexp2(MdI - GfI);
        fc = xm * fexp2(GlI - MdI);
        tail = xm * fexp2(Gn - MdI);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xp[e] = xm[e] = 0.f;
          fr[e] = fexp2(GI[e] - GfI);
          fc[e] = fexp2(GlI - GI[e]);
          tail[e] = fexp2(Gn - GI[e]);
        }
      }
      // state products (contraction over V); rowsum(S * dS+) for this feature is
      // the diagonal of S_fb dS+_fb^T, one more MFMA on the same fragments
      f32x4 SQ = zero4(), SE = zero4(), SF = zero4(), SS = zero4();
      {
#pragma unroll
        for (int k0 = 0; k0 < V; k0 += KS) {
          const auto sf = ldfrag<T, true>(sSs, PSS, 1, k0);
          const auto df = ldfrag<T, true>(sDs, PSS, 1, k0);
          SS = mma(sf, df, SS);
          SQ = mma(ldfrag<T, true>(sO + I * SUB * PV, PV, 1, k0), sf, SQ);
          SE = mma(ldfrag<T, true>(sP + I * SUB * PV, PV, 1, k0), sf, SE);
          SF = mma(ldfrag<T, true>(sR + I * SUB * PV, PV, 1, k0), df, SF);
        }
        // diagonal element (f, f) sits in lane 16 (f >> 2) + f, component f & 3
        l0 = __shfl(comp(SS, f & 3), ((f >> 2) << 4) | f) * fexp2(Gn);
      }
      // -- sources before I: gamma (Hq Y), gamma (D Y) ----------------------------
      // The sending factor of an earlier block J carries the column factor as
      // well, exp2(Gf_I - G) = exp2(Gf_I - Gl_J) exp2(Gl_J - G) <= 1, so the
      // products of every J accumulate in the MFMA accumulators directly.  XHQ
      // is formed without the query scale, applied once in the chain rules.
      f32x4 XHY = zero4(), XDY = zero4(), XDE = zero4(), XHQ = zero4();
      static_for<0, NSUB - 1>([&](auto J) {
        if (J >= I) return;
        f32x4 ks;
        const f32x4 kJ = unpack(kp[J]);
#pragma unroll
        for (int e = 0; e < 4; ++e) ks[e] = kJ[e] * fexp2(GfI - G[J][e]);
        mm16_split<T>(XHY, Hm[J], ks);
        mm16_split<T>(XDY, Dm[J], ks);
      });
      // -- sources after I: (D^T E) / gamma, (Hq^T Qg) / gamma -------------------
      // (the mirror: exp2(G - Gl_I) = exp2(Gf_J - Gl_I) exp2(G - Gf_J) <= 1)
      static_for<1, NSUB>([&](auto J) {
        if (J <= I || J * SUB >= n) return;
        f32x4 es, qs;
        const f32x4 kJ = unpack(kp[J]), qJ = unpack(qp[J]);
        f32x4 bJ;
        if constexpr (EW) bJ = unpack(bp[J]);
        else bJ = *reinterpret_cast<const f32x4*>(sBeta + J * SUB + 4 * q4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = fexp2(G[J][e] - GlI);
          es[e] = bJ[e] * kJ[e] * x;
          qs[e] = qJ[e] * x;
        }
        mm16_split<T>(XDE, Dtm[J], es);
        mm16_split<T>(XHQ, Htm[J], qs);
      });
      XHY *= fr;
      XDY *= fr;
      XDE *= fc;
      XHQ *= fc;
      // -- diagonal block ------------------------------------------------------------
      if (!wideI) {
        const f32x4 ks = kI * xm, es = bI * kI * xp, qs = qI * xp;
        f32x4 tH = zero4(), tD = zero4(), tE = zero4(), tQ = zero4();
        mm16_split<T>(tH, HmI, ks);
        mm16_split<T>(tD, DmI, ks);
        mm16_split<T>(tE, DtmI, es);
        mm16_split<T>(tQ, HtmI, qs);
        XHY += xp * tH;
        XDY += xp * tD;
        XDE += xm * tE;
        XHQ += xm * tQ;
      } else {
        // pairwise inside the block: exp2(G_r - G_j) formed per pair, never above 1
        const float* Dd = sDiag;
        const float* Hd = sDiag + SUB * PD;
        // this lane's first row, opaque here (bf16): the row comparisons below
        // are formed on this (rare) path instead of being hoisted out of the
        // feature-block loop, where their lane masks stayed live and spilled
        // (measured on the bf16 kernels; the fp32 ones are left as they were)
        int r0 = 4 * q4;
        if constexpr (std::is_same_v<T, bf16>) asm volatile("" : "+v"(r0));
#pragma unroll
        for (int j = 0; j < SUB; ++j) {
          const int src = ((j >> 2) << 4) | f;
          const float Gj = __shfl(GI[j & 3], src);
          const float kj = __shfl(kI[j & 3], src);
          const float qj = __shfl(qI[j & 3], src);
          const float bj = EW ? tof(sBs[f * PKS + I * SUB + j]) : sBeta[I * SUB + j];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = r0 + e;
            if (j <= r) {
              const float x = fexp2(GI[e] - Gj) * kj;
              XHY[e] += Hd[r * PD + j] * x;
              XDY[e] += Dd[r * PD + j] * x;
            }
            if (j >= r) {
              const float x = fexp2(Gj - GI[e]);
              XDE[e] += Dd[j * PD + r] * bj * kj * x;
              XHQ[e] += Hd[j * PD + r] * qj * x;
            }
          }
        }
      }
      // -- chain rules ---------------------------------------------------------------
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = lrow + e;
        if (row < n) {
          const float gam = fexp2(GI[e]);
          const float XQ = gam * SQ[e] + XHY[e];
          const float XE = -gam * SE[e] + XDY[e];
          const float XY = XDE[e] + scale * XHQ[e] + SF[e] * tail[e];
          const float kv = kI[e], qv = qI[e], b = bI[e];
          oq[e] = scale * XQ;
          ok_[e] = b * XE + XY;
          gbar[e] = scale * qv * XQ + b * kv * XE - kv * XY;
          dbe[e] += kv * XE;
          ob[e] = kv * XE;
          lamw += kv * SF[e] * tail[e];
        }
      }
      lamw = rows_sum(lamw);
    }
    // dq, dk of this block, transposed by one product with the identity: lane
    // (q4, f) then holds row 16 I + f, features 16 fb + 4 q4 .. + 3, one 8-byte
    // piece (16 bytes in fp32).  The blocks of a group wait for its last one,
    // so each 128-byte line of a row is written whole in one burst (a line
    // completed across iterations can leave the cache half written and cost
    // a second write); the stores are issued in every block (other blocks and
    // rows past the end fall outside the buffers and are dropped), which
    // keeps the loop's memory operations the same on every path.
    {
      f32x4 tq = zero4(), tk = zero4();
      mm16(tq, to_frag<T>(f32x4{oq[0], oq[1], oq[2], oq[3]}), idt);
      mm16(tk, to_frag<T>(f32x4{ok_[0], ok_[1], ok_[2], ok_[3]}), idt);
      const FR yq = to_frag<T>(tq), yk = to_frag<T>(tk);
      FR yb = to_frag<T>(zero4());
      if constexpr (EW) {
        f32x4 tbb = zero4();
        mm16(tbb, to_frag<T>(f32x4{ob[0], ob[1], ob[2], ob[3]}), idt);
        yb = to_frag<T>(tbb);
      }
      const int64_t tb = (int64_t)(I * SUB + f) * gsK + fb * SUB + 4 * q4;
      const bool last = (fb % QG) == QG - 1;
      // block fb - d of the group, d = QG - 1 .. 0 (d = 0: this block)
      auto qoff = [&](int d) { return last ? (uint32_t)((tb - d * SUB) * (int64_t)sizeof(T)) : OOB; };
      auto st = [&](const GBuf& b, uint32_t off, const FR& x) {
        if constexpr (std::is_same_v<T, bf16>) gst8(b, off, __builtin_bit_cast(uint2, x));
        else gst16(b, off, __builtin_bit_cast(uint4, x));
      };
#pragma unroll
      for (int j = QG - 2; j >= 0; --j) {  // pdq[j] is block fb - 1 - j
        st(bdq, qoff(j + 1), pdq[j]);
        st(bdk, qoff(j + 1), pdk[j]);
      }
      st(bdq, qoff(0), yq);
      st(bdk, qoff(0), yk);
#pragma unroll
      for (int j = QG - 2; j > 0; --j) {
        pdq[j] = pdq[j - 1];
        pdk[j] = pdk[j - 1];
      }
      pdq[0] = yq;
      pdk[0] = yk;
      if constexpr (EW) {  // db in pairs of blocks
        const bool odd = fb & 1;
        const uint32_t o1 = odd ? (uint32_t)((tb - SUB) * (int64_t)sizeof(T)) : OOB;
        const uint32_t o2 = odd ? (uint32_t)(tb * (int64_t)sizeof(T)) : OOB;
        st(bdb, o1, pdb);
        st(bdb, o2, yb);
        pdb = yb;
      }
    }
    if constexpr (GATE == 2) {
      // in-block reverse sum: own rows, then the lane groups after this one
      const float s = gbar[0] + gbar[1] + gbar[2] + gbar[3];
      const float x = rows_suffix_sum(s, q4);  // sum over lane groups >= q4
      float run = x - s;
      f32x4 suf;
      suf[3] = run += gbar[3];
      suf[2] = run += gbar[2];
      suf[1] = run += gbar[1];
      suf[0] = run + gbar[0];
      if (q4 == 0) {
        sTot[buf][I * SUB + f] = x;
        sLam[buf][I * SUB + f] = lamw;
      }
      lds_barrier();  // block totals visible; this block's operands are no longer read
      float add = l0;  // endpoint term, added to every row
#pragma unroll
      for (int J = 0; J < NSUB; ++J) {
        add += sLam[buf][J * SUB + f];
        if (J > I) add += sTot[buf][J * SUB + f];
      }
      // transposed like dq (in fp32, exactly): one 16-byte piece per lane;
      // rows past the end (all rows of a wave past the end) are dropped
      f32x4 tg = zero4();
      mm16(tg, f32x4{suf[0] + add, suf[1] + add, suf[2] + add, suf[3] + add}, idf);
      if constexpr (GIN) {
        // dx = (dg/dz) dg, z = x + dt_bias: softplus form -ea sigmoid(z),
        // bounded form lb s (1 - s) ea with s = sigmoid(ea z).  The wave's sums
        // over its valid rows of dg softplus(z) (times -ea at the end: dg g)
        // or of dx z, and, per feature, of dx.  dg is zeroed on rows past the
        // end (their dx is not stored), so no other mask is needed.
        const float rm = I * SUB + f < n ? 1.f : 0.f;
        f32x4 xv, dx, px;
        if constexpr (sizeof(T) == 2) {
          xv[0] = __uint_as_float(xr.x << 16);
          xv[1] = __uint_as_float(xr.x & 0xffff0000u);
          xv[2] = __uint_as_float(xr.y << 16);
          xv[3] = __uint_as_float(xr.y & 0xffff0000u);
        } else {
          xv = __builtin_bit_cast(f32x4, xr);
        }
        const f32x4 dt = __builtin_bit_cast(f32x4, dtr);
        if (lb == 0.f) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float sp, sg;
            softplus_sigmoid(xv[e] + dt[e], sp, sg);
            const float dgm = tg[e] * rm;
            dx[e] = nea * sg * dgm;
            dal += dgm * sp;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // s (1 - s) = e / (1 + e)^2 with e = exp(-|u|), u = ea z: no
            // cancellation where s is close to 1
            const float z = xv[e] + dt[e];
            const float ex = fexp2(nea * fabsf(z) * LOG2E), rr = __builtin_amdgcn_rcpf(1.f + ex);
            dx[e] = lbea * (ex * rr * rr) * (tg[e] * rm);
            dal += dx[e] * z;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) px[e] = row16_sum(dx[e]);  // over the wave's 16 rows
        gst16(bgp, f == 0 ? (uint32_t)((I * K + fb * SUB + 4 * q4) * 4) : OOB, __builtin_bit_cast(uint4, px));
        // stored in pairs of feature blocks, like dq
        const FR yx = to_frag<T>(dx);
        const bool odd = fb & 1;
        const int64_t tb = (int64_t)(I * SUB + f) * gsK + fb * SUB + 4 * q4;
        const uint32_t o1 = odd ? (uint32_t)((tb - SUB) * (int64_t)sizeof(T)) : OOB;
        const uint32_t o2 = odd ? (uint32_t)(tb * (int64_t)sizeof(T)) : OOB;
        if constexpr (std::is_same_v<T, bf16>) {
          gst8(bdx, o1, __builtin_bit_cast(uint2, pdx));
          gst8(bdx, o2, __builtin_bit_cast(uint2, yx));
        } else {
          gst16(bdx, o1, __builtin_bit_cast(uint4, pdx));
          gst16(bdx, o2, __builtin_bit_cast(uint4, yx));
        }
        pdx = yx;
      } else {  // in pairs of blocks: each 128-byte line of a row in one burst
        const bool odd = fb & 1;
        const int64_t tb = (int64_t)(I * SUB + f) * gsK + fb * SUB + 4 * q4;
        gst16(bdg, odd ? (uint32_t)((tb - SUB) * 4) : OOB, __builtin_bit_cast(uint4, pdg));
        gst16(bdg, odd ? (uint32_t)(tb * 4) : OOB, __builtin_bit_cast(uint4, tg));
        pdg = tg;
      }
    } else if (GATE == 1 && live) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sufs[e] += row16_sum(gbar[e]);  // over the block's 16 features
      lamws += row16_sum(lamw);
      lam0s += row16_sum(l0);
    }
    if constexpr (GATE != 2) lds_barrier();  // this block's operands are no longer read
    put_fb();                        // after the last block: unused
    lds_barrier();                   // the next block's operands are visible
  }

  // ---- gate in the kernel: the wave's partial sum of dg g ---------------------
  if constexpr (GIN) {
    const float x = rows_sum(row16_sum(dal) * (lb == 0.f ? nea : 1.f));
    const GBuf bga = gbuf(a.gpart + (int64_t)a.nc_max * H * NSUB * K + cb * NSUB, NSUB * 4);
    gst4(bga, l == 0 ? (uint32_t)(I * 4) : OOB, __float_as_uint(x));
  }

  // ---- dbeta = write part + erase part (rows of block I) ---------------------
  // (the erase/write form wrote db and dw element by element instead)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (EW) break;
    const float x = row16_sum(dbe[e]);
    const int row = I * SUB + 4 * q4 + e;
    if (f == 0 && row < n)
      st_beta(a.dbeta, a.beta_f32, (t0 + row) * H + h, sDbw[row] + x);
  }

  // ---- scalar gate: reverse sum over the chunk's rows ---------------------------
  if constexpr (GATE == 1) {
    const float s = sufs[0] + sufs[1] + sufs[2] + sufs[3];
    const float x = rows_suffix_sum(s, q4);
    float run = x - s;
    sufs[3] = run += sufs[3];
    sufs[2] = run += sufs[2];
    sufs[1] = run += sufs[1];
    sufs[0] = run + sufs[0];
    const int buf = NFB & 1;  // not used by the last feature block
    if (l == 0) {
      sTot[buf][I] = live ? x : 0.f;
      sLam[buf][I] = live ? lamws : 0.f;
    }
    lds_barrier();
    if (live) {
      float add = lam0s;
      for (int J = 0; J < NSUB; ++J) {
        add += sLam[buf][J];
        if (J > I) add += sTot[buf][J];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = I * SUB + 4 * q4 + e;
        if (f == 0 && row < n) a.dg[(t0 + row) * H + h] = sufs[e] + add;
      }
    }
  }
}

template <typename T, int GX>
static hipError_t bwd_chunk_g(const Args& a, hipStream_t s) {
  const dim3 grid(a.nc_max * a.H), block(256);
  REWY_KV_SWITCH_X(k_bwd_chunk, GX)
}

template <typename T>
static hipError_t bwd_chunk_t(const Args& a, hipStream_t s) {
  switch (a.gate) {
    case 0: return a.ew ? bwd_chunk_g<T, 4>(a, s) : bwd_chunk_g<T, 0>(a, s);
    case 1: return a.ew ? bwd_chunk_g<T, 5>(a, s) : bwd_chunk_g<T, 1>(a, s);
    case 2: return a.ew ? bwd_chunk_g<T, 6>(a, s) : a.gin ? bwd_chunk_g<T, 10>(a, s) : bwd_chunk_g<T, 2>(a, s);
    default: return hipErrorInvalidValue;
  }
}
template <typename T>
static hipError_t bwd_consumers_t(const Args& a, hipStream_t s) {
  switch (a.gate) {
    case 0: return bwd_chunk_g<T, 32>(a, s);
    case 1: return bwd_chunk_g<T, 33>(a, s);
    case 2: return bwd_chunk_g<T, 34>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_chunk(const Args& a, int f32, hipStream_t s) {
  return f32 ? bwd_chunk_t<float>(a, s) : bwd_chunk_t<bf16>(a, s);
}
hipError_t launch_bwd_producer(const Args& a, int f32, hipStream_t s) {
  if (a.ew || a.gin) return hipErrorInvalidValue;
  return f32 ? bwd_chunk_g<float, 16>(a, s) : bwd_chunk_g<bf16, 16>(a, s);
}
hipError_t launch_bwd_consumers(const Args& a, int f32, hipStream_t s) {
  if (a.ew || a.gin) return hipErrorInvalidValue;
  return f32 ? bwd_consumers_t<float>(a, s) : bwd_consumers_t<bf16>(a, s);
}

// Parameter gradients of the gate formed in the kernel, from the chunk
// backward's per-wave partial sums (GDN2 spec section 4.4: dA_log = sum of
// dg g over tokens and features, ddt_bias = sum of dx over tokens).  Block
// (h, y): y < ceil(K/64) sums ddt_bias of 64 features, sixteen slices of the
// chunk slots per feature; the last y sums dA_log of the head.  Every chunk
// slot holds partials (zeros for a slot without tokens), so the loads are
// independent of each other.  A fixed order of summation: the result does not
// depend on timing.
__global__ __launch_bounds__(1024) void k_gate_reduce(Args a) {
  constexpr int NS = 16;
  __shared__ float sp[NS][64];
  const int h = blockIdx.x, H = a.H, K = a.K;
  const int tid = threadIdx.x, tx = tid & 63, sl = tid >> 6;
  const int nkb = (K + 63) / 64;
  float acc = 0.f;
  if ((int)blockIdx.y == nkb) {
    const float* p = a.gpart + (int64_t)a.nc_max * H * NSUB * K;
#pragma unroll 4
    for (int i = tid; i < a.nc_max * NSUB; i += 1024) {
      const int c = i / NSUB;
      acc += p[((int64_t)c * H + h) * NSUB + (i - c * NSUB)];
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) acc += __shfl_xor(acc, m);
    if (tx == 0) sp[sl][0] = acc;
    __syncthreads();
    if (tid == 0) {
      float t = 0.f;
      for (int j = 0; j < NS; ++j) t += sp[j][0];
      a.da_log[h] = t;
    }
    return;
  }
  const int k = blockIdx.y * 64 + tx;
  if (k < K) {
#pragma unroll 4
    for (int c = sl; c < a.nc_max; c += NS) {
      const float* p = a.gpart + ((int64_t)c * H + h) * NSUB * K + k;
      acc += (p[0] + p[K]) + (p[2 * K] + p[3 * K]);
    }
  }
  sp[sl][tx] = acc;
  __syncthreads();
  if (sl == 0 && k < K) {
    float t = 0.f;
    for (int j = 0; j < NS; ++j) t += sp[j][tx];
    a.ddt_bias[(int64_t)h * K + k] = t;
  }
}

hipError_t launch_gate_reduce(const Args& a, hipStream_t s) {
  REWY_LAUNCH(k_gate_reduce, dim3(a.H, (a.K + 63) / 64 + 1), dim3(1024), s, a);
  return hipGetLastError();
}

}  // namespace rewy
