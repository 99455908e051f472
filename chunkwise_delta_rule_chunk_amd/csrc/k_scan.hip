// The two serial inter-chunk scans.  One workgroup of four waves per
// (sequence, head, value tile of BV columns) walks the sequence's chunks in
// order; the fp32 state tile [K x BV] stays in MFMA accumulator registers for
// the whole walk.  A 1D grid dispatches eight (sequence, head) units at a
// time with all their value tiles, longest sequences first, and keeps each
// unit on one XCD (workgroup ids go round-robin over the eight XCDs), so the
// tiles of a unit share that XCD's L2 (scan_unit below).
//
// Wave w owns token tile w of the per-chunk product (R or Rbar) and a set of
// key tiles of the state.  The chunk operands it contracts (rows of W, F^T,
// F, Cq^T, Qg^T, W^T) go straight from global memory into MFMA operand
// registers, 16 bytes per lane, two chunks ahead; only the state and the
// per-chunk product pass through LDS, with two barriers per step.  Every
// global load and store inside the chunk loop is unconditional (clamped
// indices, rows past a chunk's end masked where they are used), so the
// compiler's memory counters let each use wait for exactly its own load and
// the prefetches stay in flight across steps.
//
// Forward (ReWY paper, "The chunk system": R = U - W S, S' = Lambda S + F^T R,
// O = Qg S + Cq R; KDA blog sections 6.4-6.5, state fast-forward and output):
//   for each chunk c:  [write S_c];  R_c = U_c - W_c S_c;  [write R_c];
//                      S_{c+1} = diag(exp2 G2_last) S_c + F_c^T R_c;
//                      o_c = Qg_c S_c + Cq_c R_c   (the forward pass; the
//                      recompute in the backward writes S_c and R_c instead)
// Reverse (ReWY paper Appendix 7.2 / Algorithm 1; the scan supplies the
// incoming-state term -E^T P = -W^T Rbar once):
//   for each chunk c from the last:  write dS_{c+1};
//     Rbar_c = F_c dS_{c+1} + Cq_c^T dO_c
//     dS_c   = diag(exp2 G2_last) dS_{c+1} + Qg_c^T dO_c - W_c^T Rbar_c
#include "chunk_common.hpp"

namespace rewy {

template <int V>
using ic = std::integral_constant<int, V>;

// Forward scan.  Wave w owns token tile w of R (all value columns of the
// workgroup) and a set of key tiles of the state; it reads the W rows and F^T
// rows it contracts straight from global memory into MFMA operand registers
// (16 bytes per lane, DEPTH chunks ahead), so only S_c and R_c pass through
// LDS.  Every global load and store in the chunk loop is unconditional
// (clamped indices, selects): the compiler then counts exactly which loads a
// use has to wait for, and the prefetches stay in flight across steps.
template <typename T, int K, int V, int BV, int OUT>
__device__ __forceinline__ void fwd_scan_wg(const Args& a, const int u, const int vt) {
  constexpr int NTH = 256, DEPTH = 2;
  constexpr bool NAT = OUT & SCAN_NATURAL, OUTP = OUT & SCAN_OUTPUT;
  constexpr int VE = 16 / (int)sizeof(T), KG = 4 * VE;  // elements per lane piece, per group
  constexpr int CT = BV / SUB, NKT = K / SUB;
  constexpr int NGK = K / KG, NGT = CH / KG;
  // state tiles: wave w takes key tiles w, w + 4, ... with all CT column tiles,
  // or, for K = 32, key tile w % 2 and column tile w / 2
  constexpr bool WIDE = NKT >= 4;
  constexpr int KW = WIDE ? NKT / 4 : 1, CW = WIDE ? CT : CT * NKT / 4;
  static_assert(WIDE || (NKT == 2 && CT == 2), "state tile split");
  constexpr int PK = pitch<T>(K), PA = pitch<T>(CH);
  __shared__ __align__(16) T sHt[BV * PK];        // S_c as operand, [v][k]
  __shared__ __align__(16) T sRt[BV * PA];        // R_c as operand, [v][i]

  const int H = a.H;
  const int rk = u / H, h = u - rk * H;
  const int n = a.seqord[rk];  // the rk-th longest sequence
  const int w = wave_id(), tid = threadIdx.x, l = lane_id();
  const int r16 = l & 15, g = l >> 4;
  const int c0 = a.seqoff[n], c1 = a.seqoff[n + 1];
  // token range of the sequence from its chunk records (clamped to the inputs)
  const ChunkInfo cfirst = load_chunk(a.chunks, c0 < c1 ? c0 : 0);
  const ChunkInfo clast = load_chunk(a.chunks, c0 < c1 ? c1 - 1 : 0);
  const int seq_bos = cfirst.bos, seq_eos = clast.bos + clast.len;
  const int64_t gsV = (int64_t)H * V;
  const T* Wg = reinterpret_cast<const T*>(a.W);
  const T* Ftg = reinterpret_cast<const T*>(a.Ft);
  const T* Ug = reinterpret_cast<const T*>(a.U);
  auto ktile = [&](int j) { return WIDE ? w + 4 * j : w % NKT; };
  auto vtile = [&](int m) { return WIDE ? m : (w / NKT) * CW + m; };

  // DEPTH register sets: chunk c + DEPTH is read while chunk c is processed.
  // W, F^T and U are stored in operand-fragment order (kernels.hpp), rows past
  // a chunk's end as exact zeros: every read below is one contiguous piece.
  using FR = typename Frag4<T>::type;
  constexpr int GPP = 16 / (int)sizeof(FR);  // 16-long key groups per W piece
  // identity as the B operand of a 16-long product: C = X^T I turns a C tile
  // (rows 4 g + e, column r16) into row r16, columns 4 g .. + 3, exactly; the
  // natural-layout S_c and R_c leave the registers that way, 8 (bf16) or 16
  // (fp32) bytes of one row per lane
  f32x4 idf;
#pragma unroll
  for (int e = 0; e < 4; ++e) idf[e] = (4 * g + e == r16) ? 1.f : 0.f;
  const FR idt = to_frag<T>(idf);
  static_assert(NGK * GPP == K / SUB, "W pieces");
  uint4 wf[DEPTH][NGK];      // W rows 16 w + r16, GPP 16-long key groups per piece
  FR uf[DEPTH][CT];          // U in the C layout of R's tiles
  // output product O = Qg S + Cq R for token tile w: Qg rows in the order of
  // W (contracted with the same S operand), Cq row block w in C-fragment
  // order (two 16-token blocks joined per lane group, R read to match)
  uint4 qf[DEPTH][OUTP ? NGK : 1], cqf[DEPTH][OUTP ? NGT : 1];
  uint4 ff[DEPTH][KW][NGT];  // F^T rows 16 ktile + r16, lane piece of every token group
  f32x4 lam[DEPTH][KW];      // G2_last of the state rows this lane holds
  // past the last chunk the last one is read again (valid memory, never used)
  auto fetch_wu = [&](auto set, int c) {
    constexpr int B = decltype(set)::value;
    const int64_t cb = (int64_t)min(c, c1 - 1) * H + h;
    const T* wp = Wg + cb * CH * K + (int64_t)(w * NGK * 64 + l) * VE;
#pragma unroll
    for (int q = 0; q < NGK; ++q) wf[B][q] = *reinterpret_cast<const uint4*>(wp + q * 64 * VE);
    const T* up = Ug + cb * CH * V + (int64_t)((vt * CT * NSUB + w) * 64 + l) * 4;
#pragma unroll
    for (int m = 0; m < CT; ++m) uf[B][m] = *reinterpret_cast<const FR*>(up + m * NSUB * 64 * 4);
    if constexpr (OUTP) {  // used with W, before this set is refilled
      const T* qp = reinterpret_cast<const T*>(a.Qg) + cb * CH * K + (int64_t)(w * NGK * 64 + l) * VE;
#pragma unroll
      for (int q = 0; q < NGK; ++q) qf[B][q] = *reinterpret_cast<const uint4*>(qp + q * 64 * VE);
    }
  };
  auto fetch_fl = [&](auto set, int c) {
    constexpr int B = decltype(set)::value;
    const int64_t cb = (int64_t)min(c, c1 - 1) * H + h;
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      const int kr = SUB * ktile(j);
      const T* fp = Ftg + cb * K * CH + (int64_t)(ktile(j) * NGT * 64 + l) * VE;
#pragma unroll
      for (int q = 0; q < NGT; ++q) ff[B][j][q] = *reinterpret_cast<const uint4*>(fp + q * 64 * VE);
      lam[B][j] = *reinterpret_cast<const f32x4*>(a.glast + cb * K + kr + 4 * g);
    }
    if constexpr (OUTP) {  // used after the state update, with F^T's set
      const T* cp = reinterpret_cast<const T*>(a.Cq) + cb * CH * CH + (int64_t)(w * NSUB * 64 + l) * 4;
#pragma unroll
      for (int q = 0; q < NGT; ++q) cqf[B][q] = cfrag_op<T>(cp, q);
    }
  };

  f32x4 st[KW][CW];
#pragma unroll
  for (int j = 0; j < KW; ++j)
#pragma unroll
    for (int m = 0; m < CW; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = SUB * ktile(j) + 4 * g + i, vv = vt * BV + SUB * vtile(m) + r16;
        st[j][m][i] = a.h0 ? a.h0[(((int64_t)n * H + h) * K + kk) * V + vv] : 0.f;
      }
  if (c0 >= c1) {  // empty sequence: the final state is the initial one
    if (a.ht)
#pragma unroll
      for (int j = 0; j < KW; ++j)
#pragma unroll
        for (int m = 0; m < CW; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kk = SUB * ktile(j) + 4 * g + i, vv = vt * BV + SUB * vtile(m) + r16;
            a.ht[(((int64_t)n * H + h) * K + kk) * V + vv] = st[j][m][i];
          }
    return;
  }
  static_for<0, DEPTH>([&](auto B) {
    fetch_wu(B, c0 + B);
    fetch_fl(B, c0 + B);
  });

  // The output of a chunk is stored one step late: its C_q R product is issued
  // at the end of the chunk's step, and its transpose and store come in the
  // next step, so their latency overlaps that step's work instead of holding
  // the wave (instructions issue in order).  pbos / plen are the rows of the
  // pending chunk; plen = 0 drops the stores (nothing pending yet).
  f32x4 pend[OUTP ? CT : 1], ptr[OUTP ? CT : 1];
  int pbos = 0, plen = 0;
  auto out_transpose = [&]() {
    if constexpr (OUTP) {
#pragma unroll
      for (int m = 0; m < CT; ++m) {
        ptr[m] = zero4();
        mm16(ptr[m], to_frag<T>(pend[m]), idt);
      }
    }
  };
  auto out_store = [&]() {
    if constexpr (OUTP) {
      const GBuf bo = gbuf(reinterpret_cast<T*>(a.o) + ((int64_t)pbos * H + h) * V, tile_bytes<T>(plen, gsV, V));
#pragma unroll
      for (int m = 0; m < CT; ++m) {
        const uint32_t off = (uint32_t)(((int64_t)(SUB * w + r16) * gsV + vt * BV + SUB * m + 4 * g) * (int64_t)sizeof(T));
        if constexpr (std::is_same_v<T, bf16>) gst8(bo, off, __builtin_bit_cast(uint2, to_frag<T>(ptr[m])));
        else gst16(bo, off, __builtin_bit_cast(uint4, ptr[m]));
      }
    }
  };
  if constexpr (OUTP) {
#pragma unroll
    for (int m = 0; m < CT; ++m) pend[m] = zero4();
  }

  auto step = [&](auto buf, int c) {
    constexpr int B = decltype(buf)::value;
    const int64_t cb = (int64_t)c * H + h;
    const int bos = seq_bos + (c - c0) * CH, len = min(CH, seq_eos - bos);
    out_transpose();  // the previous chunk's output rows
    // S_c: operand [v][k] in LDS and, for global memory, natural [k][v] (its
    // transposes are issued here and stored after the barrier, whose wait
    // covers their latency)
    f32x4 trh[NAT ? KW : 1][NAT ? CW : 1];
#pragma unroll
    for (int j = 0; j < KW; ++j)
#pragma unroll
      for (int m = 0; m < CW; ++m) {
        const int kr = SUB * ktile(j), vc = SUB * vtile(m);
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = tof(fromf<T>(st[j][m][i]));
        st_tile_T<T>(x, sHt + vc * PK + kr, PK);
        if constexpr (NAT) {  // column-blocked [V/16][K][16]: a wave writes 16 whole block rows
          trh[j][m] = zero4();
          mm16(trh[j][m], to_frag<T>(x), idt);
        }
      }
    lds_barrier();
    if constexpr (NAT)
#pragma unroll
      for (int j = 0; j < KW; ++j)
#pragma unroll
        for (int m = 0; m < CW; ++m)
          *reinterpret_cast<FR*>(reinterpret_cast<T*>(a.hbuf) + cb * K * V +
                                 ((int64_t)(vt * CT + vtile(m)) * K + SUB * ktile(j) + r16) * SUB + 4 * g) =
              to_frag<T>(trh[j][m]);
    // R = U - W S for token tile w (rows past the chunk's end are zero: W and
    // U are zero there).  A W piece holds, for lane l (row l & 15), the keys
    // 16 kb + 4 (l >> 4) + e of GPP consecutive 16-key groups kb.  bf16 takes
    // both groups as one 32-slot fragment (slot 8 (l >> 4) + 4 hh + e is key
    // 32 q + 16 hh + 4 (l >> 4) + e) and reads S^T with the same assignment;
    // fp32 runs each group as four 16x16x4 steps.
    // (Qg S for the output goes with it, on the same S operand; its Cq R
    // part follows the state update, when R_c is in LDS.)
    f32x4 po[OUTP ? CT : 1];
    f32x4 trr[NAT ? CT : 1];
#pragma unroll
    for (int m = 0; m < CT; ++m) {
      f32x4 p = zero4();
      if constexpr (OUTP) po[m] = zero4();
      const T* hb = sHt + (SUB * m + r16) * PK + 4 * g;
#pragma unroll
      for (int q = 0; q < NGK; ++q) {
        if constexpr (std::is_same_v<T, bf16>) {
          const bf16x4 s0 = *reinterpret_cast<const bf16x4*>(hb + 32 * q);
          const bf16x4 s1 = *reinterpret_cast<const bf16x4*>(hb + 32 * q + SUB);
          const bf16x8 sb = __builtin_shufflevector(s0, s1, 0, 1, 2, 3, 4, 5, 6, 7);
          p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[B][q]), sb, p, 0, 0, 0);
          if constexpr (OUTP)
            po[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qf[B][q]), sb, po[m], 0, 0, 0);
        } else {
          const f32x4 sv = *reinterpret_cast<const f32x4*>(hb + SUB * q);
          mm16(p, __builtin_bit_cast(f32x4, wf[B][q]), sv);
          if constexpr (OUTP) mm16(po[m], __builtin_bit_cast(f32x4, qf[B][q]), sv);
        }
      }
      f32x4 rv;
#pragma unroll
      for (int i = 0; i < 4; ++i) rv[i] = tof(fromf<T>(tof(uf[B][m][i]) - p[i]));
      st_tile_T<T>(rv, sRt + (SUB * m) * PA + SUB * w, PA);
      if constexpr (NAT) {  // column-blocked [V/16][64][16], all 64 rows (zero past the end); stored after the barrier
        trr[m] = zero4();
        mm16(trr[m], to_frag<T>(rv), idt);
      }
    }
    out_store();
    fetch_wu(ic<B>{}, c + DEPTH);
    lds_barrier();
    if constexpr (NAT)
#pragma unroll
      for (int m = 0; m < CT; ++m)
        *reinterpret_cast<FR*>(reinterpret_cast<T*>(a.R) + cb * V * CH +
                               ((int64_t)(vt * CT + m) * CH + SUB * w + r16) * SUB + 4 * g) = to_frag<T>(trr[m]);
    // S = diag(exp2 G2_last) S + F^T R
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      f32x4 d;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = fexp2(lam[B][j][i]);
#pragma unroll
      for (int m = 0; m < CW; ++m) {
        const T* rb = sRt + (SUB * vtile(m) + r16) * PA + VE * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) st[j][m][i] *= d[i];
#pragma unroll
        for (int q = 0; q < NGT; ++q) mma16B<T>(st[j][m], ff[B][j][q], *reinterpret_cast<const uint4*>(rb + KG * q));
      }
    }
    // o rows of token tile w: O += Cq R, left pending; the next step (or the
    // end of the walk) transposes it by the identity product into 8-byte
    // (16-byte fp32) row pieces and stores them; rows past the chunk's end
    // fall outside the buffer and are dropped
    if constexpr (OUTP) {
#pragma unroll
      for (int m = 0; m < CT; ++m) {
        const T* rb = sRt + (SUB * m + r16) * PA + 4 * g;
#pragma unroll
        for (int q = 0; q < NGT; ++q) mma16B<T>(po[m], cqf[B][q], perm_row<T>(rb, q));
        pend[m] = po[m];
      }
      pbos = bos;
      plen = len;
    }
    fetch_fl(ic<B>{}, c + DEPTH);
  };
  // the back edge always follows both steps, so the loop body's memory
  // operations are the same on every path
  for (int c = c0;;) {
    step(ic<0>{}, c);
    if (++c >= c1) break;
    step(ic<1>{}, c);
    if (++c >= c1) break;
  }
  out_transpose();  // the last chunk's output rows
  out_store();
  if (a.ht) {
#pragma unroll
    for (int j = 0; j < KW; ++j)
#pragma unroll
      for (int m = 0; m < CW; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = SUB * ktile(j) + 4 * g + i, vv = vt * BV + SUB * vtile(m) + r16;
          a.ht[(((int64_t)n * H + h) * K + kk) * V + vv] = st[j][m][i];
        }
  }
}

// Reverse scan, organised like the forward one: wave w owns token tile w of
// Rbar and a set of key tiles of dS; F rows, Cq^T rows, Qg^T rows and W^T rows
// go straight from global memory into operand registers; dS_{c+1}, dO_c
// (transposed) and Rbar_c pass through LDS.
template <typename T, int K, int V, int BV>
__device__ __forceinline__ void bwd_scan_wg(const Args& a, const int u, const int vt) {
  constexpr int NTH = 256, DEPTH = 2;
  constexpr int VE = 16 / (int)sizeof(T), KG = 4 * VE;
  constexpr int CT = BV / SUB, NKT = K / SUB;
  constexpr int NGK = K / KG, NGT = CH / KG;
  constexpr bool WIDE = NKT >= 4;
  constexpr int KW = WIDE ? NKT / 4 : 1, CW = WIDE ? CT : CT * NKT / 4;
  static_assert(WIDE || (NKT == 2 && CT == 2), "state tile split");
  constexpr int PK = pitch<T>(K), PA = pitch<T>(CH);
  // dO rows as staged by the threads: 8-byte pieces (4 elements)
  constexpr int OE = 8 / (int)sizeof(T), OPER = BV / OE;
  constexpr int ON = CH * BV * (int)sizeof(T) / (NTH * 8);  // dO pieces per thread
  static_assert(ON >= 1 && CH * BV * (int)sizeof(T) == NTH * 8 * ON, "dO staging split");
  __shared__ __align__(16) T sDt[BV * PK];      // dS_{c+1} as operand, [v][k]
  __shared__ __align__(16) T sOt[2][BV * PA];   // dO_c as operand, [v][j]
  __shared__ __align__(16) T sRbt[BV * PA];     // Rbar_c as operand, [v][i]

  const int H = a.H;
  const int rk = u / H, h = u - rk * H;
  const int n = a.seqord[rk];  // the rk-th longest sequence
  const int w = wave_id(), tid = threadIdx.x, l = lane_id();
  const int r16 = l & 15, g = l >> 4;
  const int c0 = a.seqoff[n], c1 = a.seqoff[n + 1];
  // token range of the sequence from its chunk records (clamped to the inputs)
  const ChunkInfo cfirst = load_chunk(a.chunks, c0 < c1 ? c0 : 0);
  const ChunkInfo clast = load_chunk(a.chunks, c0 < c1 ? c1 - 1 : 0);
  const int seq_bos = cfirst.bos, seq_eos = clast.bos + clast.len;
  const int64_t gsV = (int64_t)H * V;
  auto ktile = [&](int j) { return WIDE ? w + 4 * j : w % NKT; };
  auto vtile = [&](int m) { return WIDE ? m : (w / NKT) * CW + m; };

  uint4 ff[DEPTH][NGK];      // F row 16 w + r16 (keys)
  uint4 cf[DEPTH][NGT];      // Cq^T row 16 w + r16 (tokens j)
  uint4 qf[DEPTH][KW][NGT];  // Qg^T row 16 ktile + r16 (tokens)
  uint4 wf[DEPTH][KW][NGT];  // W^T row 16 ktile + r16 (tokens)
  f32x4 lam[DEPTH][KW];
  uint2 of[DEPTH][ON];       // dO pieces
  using FR = typename Frag4<T>::type;
  // identity as the B operand of a 16-long product (C = X^T I, exact): the
  // natural-layout dS_{c+1} leaves the registers as pieces of one row
  f32x4 idf;
#pragma unroll
  for (int e = 0; e < 4; ++e) idf[e] = (4 * g + e == r16) ? 1.f : 0.f;
  const FR idt = to_frag<T>(idf);
  // chunks are walked from the last; before the first one the first is read
  // again (valid memory, never used)
  auto chunk_of = [&](int c) { return max(c, c0); };
  // F, Cq^T, Qg^T and W^T are stored in operand-fragment order (kernels.hpp),
  // rows past a chunk's end as exact zeros: each read is one contiguous piece
  auto fetch = [&](auto set, int c) {
    constexpr int B = decltype(set)::value;
    const int cc = chunk_of(c);
    const int bos = seq_bos + (cc - c0) * CH, len = min(CH, seq_eos - bos);
    const int64_t cb = (int64_t)cc * H + h;
    const T* fp = reinterpret_cast<const T*>(a.F) + cb * CH * K + (int64_t)(w * NGK * 64 + l) * VE;
#pragma unroll
    for (int q = 0; q < NGK; ++q) ff[B][q] = *reinterpret_cast<const uint4*>(fp + q * 64 * VE);
    const T* cp = reinterpret_cast<const T*>(a.Cqt) + cb * CH * CH + (int64_t)(w * NGT * 64 + l) * VE;
#pragma unroll
    for (int q = 0; q < NGT; ++q) cf[B][q] = *reinterpret_cast<const uint4*>(cp + q * 64 * VE);
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      const int kr = SUB * ktile(j);
      const int64_t po = (int64_t)(ktile(j) * NGT * 64 + l) * VE;
      const T* qp = reinterpret_cast<const T*>(a.Qgt) + cb * K * CH + po;
      const T* wp = reinterpret_cast<const T*>(a.Wt) + cb * K * CH + po;
#pragma unroll
      for (int q = 0; q < NGT; ++q) {
        qf[B][j][q] = *reinterpret_cast<const uint4*>(qp + q * 64 * VE);
        wf[B][j][q] = *reinterpret_cast<const uint4*>(wp + q * 64 * VE);
      }
      lam[B][j] = *reinterpret_cast<const f32x4*>(a.glast + cb * K + kr + 4 * g);
    }
    const T* op = reinterpret_cast<const T*>(a.dO) + ((int64_t)bos * H + h) * V + vt * BV;
#pragma unroll
    for (int e = 0; e < ON; ++e) {
      const int idx = tid + e * NTH, r = idx / OPER, c8 = (idx % OPER) * OE;
      of[B][e] = *reinterpret_cast<const uint2*>(op + (int64_t)min(r, len - 1) * gsV + c8);
    }
  };

  f32x4 st[KW][CW];
#pragma unroll
  for (int j = 0; j < KW; ++j)
#pragma unroll
    for (int m = 0; m < CW; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = SUB * ktile(j) + 4 * g + i, vv = vt * BV + SUB * vtile(m) + r16;
        st[j][m][i] = a.dht ? a.dht[(((int64_t)n * H + h) * K + kk) * V + vv] : 0.f;
      }
  auto final_out = [&]() {
    if (a.dh0)
#pragma unroll
      for (int j = 0; j < KW; ++j)
#pragma unroll
        for (int m = 0; m < CW; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kk = SUB * ktile(j) + 4 * g + i, vv = vt * BV + SUB * vtile(m) + r16;
            a.dh0[(((int64_t)n * H + h) * K + kk) * V + vv] = st[j][m][i];
          }
  };
  if (c0 >= c1) {
    final_out();
    return;
  }
  static_for<0, DEPTH>([&](auto B) { fetch(B, c1 - 1 - B); });

  auto step = [&](auto buf, int c) {
    constexpr int B = decltype(buf)::value;
    const int bos = seq_bos + (c - c0) * CH, len = min(CH, seq_eos - bos);
    const int64_t cb = (int64_t)c * H + h;
    // dS_{c+1}: operand [v][k] and natural [k][v]; dO_c transposed (rows past
    // the chunk's end zero).  The natural copy's transposes are issued here and
    // stored after the barrier, whose wait covers their latency.
    f32x4 trd[KW][CW];
#pragma unroll
    for (int j = 0; j < KW; ++j)
#pragma unroll
      for (int m = 0; m < CW; ++m) {
        const int kr = SUB * ktile(j), vc = SUB * vtile(m);
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = tof(fromf<T>(st[j][m][i]));
        st_tile_T<T>(x, sDt + vc * PK + kr, PK);
        trd[j][m] = zero4();  // column-blocked [V/16][K][16]
        mm16(trd[j][m], to_frag<T>(x), idt);
      }
#pragma unroll
    for (int e = 0; e < ON; ++e) {
      const int idx = tid + e * NTH, r = idx / OPER, c8 = (idx % OPER) * OE;
      union {
        uint2 u;
        T v[OE];
      } x;
      x.u = of[B][e];
#pragma unroll
      for (int k = 0; k < OE; ++k) sOt[B][(c8 + k) * PA + r] = r < len ? x.v[k] : fromf<T>(0.f);
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < KW; ++j)
#pragma unroll
      for (int m = 0; m < CW; ++m)
        *reinterpret_cast<FR*>(reinterpret_cast<T*>(a.dhbuf) + cb * K * V +
                               ((int64_t)(vt * CT + vtile(m)) * K + SUB * ktile(j) + r16) * SUB + 4 * g) =
            to_frag<T>(trd[j][m]);
    // Rbar = F dS+ + Cq^T dO for token tile w (rows past the end are zero: F
    // and Cq vanish there)
#pragma unroll
    for (int m = 0; m < CT; ++m) {
      f32x4 acc = zero4();
      const T* db = sDt + (SUB * m + r16) * PK + VE * g;
      const T* ob = sOt[B] + (SUB * m + r16) * PA + VE * g;
#pragma unroll
      for (int q = 0; q < NGK; ++q) mma16B<T>(acc, ff[B][q], *reinterpret_cast<const uint4*>(db + KG * q));
#pragma unroll
      for (int q = 0; q < NGT; ++q) mma16B<T>(acc, cf[B][q], *reinterpret_cast<const uint4*>(ob + KG * q));
      st_tile_T<T>(acc, sRbt + (SUB * m) * PA + SUB * w, PA);
      // Rbar in the C-fragment order of its 16 x 16 tiles: a wave writes one
      // contiguous tile
      *reinterpret_cast<FR*>(reinterpret_cast<T*>(a.Rbt) + cb * V * CH +
                             (((int64_t)(vt * CT + m) * NSUB + w) * 64 + l) * 4) = to_frag<T>(acc);
    }
    lds_barrier();
    // dS = diag(exp2 G2_last) dS+ + Qg^T dO - W^T Rbar (W^T negated by its sign bits)
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      f32x4 d;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = fexp2(lam[B][j][i]);
      uint4 wn[NGT];
      constexpr unsigned SGN = sizeof(T) == 2 ? 0x80008000u : 0x80000000u;
#pragma unroll
      for (int q = 0; q < NGT; ++q) {
        const uint4 x = wf[B][j][q];
        wn[q] = uint4{x.x ^ SGN, x.y ^ SGN, x.z ^ SGN, x.w ^ SGN};
      }
#pragma unroll
      for (int m = 0; m < CW; ++m) {
        const T* ob = sOt[B] + (SUB * vtile(m) + r16) * PA + VE * g;
        const T* rb = sRbt + (SUB * vtile(m) + r16) * PA + VE * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) st[j][m][i] *= d[i];
#pragma unroll
        for (int q = 0; q < NGT; ++q) mma16B<T>(st[j][m], qf[B][j][q], *reinterpret_cast<const uint4*>(ob + KG * q));
#pragma unroll
        for (int q = 0; q < NGT; ++q) mma16B<T>(st[j][m], wn[q], *reinterpret_cast<const uint4*>(rb + KG * q));
      }
    }
    fetch(ic<B>{}, c - DEPTH);
  };
  for (int c = c1 - 1;;) {
    step(ic<0>{}, c);
    if (--c < c0) break;
    step(ic<1>{}, c);
    if (--c < c0) break;
  }
  final_out();
}

// Workgroup id -> (unit, value tile), units u = rank * H + head in the scan
// order (longest sequences first, Args::seqord).  Eight consecutive units form
// a group whose NSC scans x NT value tiles are dispatched together, and unit u
// runs on XCD u % 8 (workgroup ids go round-robin over the eight XCDs), so the
// tiles of one (sequence, head) share that XCD's L2.  Ids past the last unit
// exit at once.
template <int NT, int NSC>
__device__ __forceinline__ bool scan_unit(const Args& a, int& u, int& vt, int& sc) {
  const int id = blockIdx.x, grp = id / (8 * NT * NSC), rem = id - grp * 8 * NT * NSC;
  sc = rem / (8 * NT);
  vt = (rem / 8) % NT;
  u = grp * 8 + (rem & 7);
  return u < a.N * a.H;
}
inline dim3 scan_grid(const Args& a, int nt, int nsc) {
  return dim3(((a.N * a.H + 7) / 8) * 8 * nt * nsc);
}

template <typename T, int K, int V, int BV, int OUT>
__global__ __launch_bounds__(256) void k_fwd_scan(Args a) {
  int u, vt, sc;
  if (scan_unit<V / BV, 1>(a, u, vt, sc)) fwd_scan_wg<T, K, V, BV, OUT>(a, u, vt);
}
template <typename T, int K, int V, int BV>
__global__ __launch_bounds__(256) void k_bwd_scan(Args a) {
  int u, vt, sc;
  if (scan_unit<V / BV, 1>(a, u, vt, sc)) bwd_scan_wg<T, K, V, BV>(a, u, vt);
}
// Both scans of the backward under recompute in one launch: they read
// disjoint operands and write disjoint outputs, so the reverse scan (the
// longer one, dispatched first within each group of units) and the forward
// recompute scan run side by side, each on its own share of the CUs.  Wider
// value tiles halve the operand reads of each scan.
template <typename T, int K, int V, int BV>
__global__ __launch_bounds__(256) void k_scans(Args a) {
  int u, vt, sc;
  if (!scan_unit<V / BV, 2>(a, u, vt, sc)) return;
  if (sc == 0)
    bwd_scan_wg<T, K, V, BV>(a, u, vt);
  else
    fwd_scan_wg<T, K, V, BV, SCAN_NATURAL>(a, u, vt);
}

int scan_bv(const Args& a, int f32) {
  if (a.K == 32) return 32;  // four waves need K * BV >= 1024
  if (f32) return 16;        // keeps the fp32 double buffers within LDS
  // 32-wide tiles when they still give at least one workgroup per CU
  return (int64_t)a.N * a.H * (a.V / 32) >= 256 ? 32 : 16;
}

template <typename T, int BV>
static hipError_t fwd_scan_bv(const Args& a, hipStream_t s) {
  const dim3 grid = scan_grid(a, a.V / BV, 1), block(256);
#define REWY_SCAN_CASE(K_, V_)                                                  \
  case K_ * 1000 + V_:                                                          \
    if constexpr (kv_ok<T, K_, V_>() && V_ >= BV && K_ * BV >= 1024 && \
                  (sizeof(T) == 2 || K_ == 32 || BV == 16)) {                             \
      if (a.scan_out == SCAN_OUTPUT)                                            \
        REWY_LAUNCH((k_fwd_scan<T, K_, V_, BV, SCAN_OUTPUT>), grid, block, s, a); \
      else if (a.scan_out == (SCAN_NATURAL | SCAN_OUTPUT))                      \
        REWY_LAUNCH((k_fwd_scan<T, K_, V_, BV, SCAN_NATURAL | SCAN_OUTPUT>), grid, block, s, a); \
      else                                                                      \
        return hipErrorInvalidValue;                                            \
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
  const dim3 grid = scan_grid(a, a.V / BV, 1), block(256);
#define REWY_SCAN_CASE(K_, V_)                                                  \
  case K_ * 1000 + V_:                                                          \
    if constexpr (kv_ok<T, K_, V_>() && V_ >= BV && K_ * BV >= 1024 && \
                  (sizeof(T) == 2 || K_ == 32 || BV == 16)) {                             \
      REWY_LAUNCH((k_bwd_scan<T, K_, V_, BV>), grid, block, s, a);    \
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

template <typename T, int BV>
static hipError_t scans_bv(const Args& a, hipStream_t s) {
  const dim3 grid = scan_grid(a, a.V / BV, 2), block(256);
#define REWY_SCAN_CASE(K_, V_)                                                  \
  case K_ * 1000 + V_:                                                          \
    if constexpr (kv_ok<T, K_, V_>() && V_ >= BV && K_ * BV >= 1024 &&          \
                  (sizeof(T) == 2 || K_ == 32 || BV == 16)) {                   \
      REWY_LAUNCH((k_scans<T, K_, V_, BV>), grid, block, s, a);       \
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
// 32-wide value tiles wherever the kernels allow them (fp32 keeps 16 for LDS)
hipError_t launch_scans(const Args& a, int f32, hipStream_t s) {
  if (a.scan_out != SCAN_NATURAL) return hipErrorInvalidValue;
  if (f32) return a.K == 32 ? scans_bv<float, 32>(a, s) : scans_bv<float, 16>(a, s);
  return scans_bv<bf16, 32>(a, s);
}

}  // namespace rewy
