// The two serial inter-chunk scans.  One workgroup per (sequence, head,
// value tile of BV columns) walks the sequence's chunks in order; the fp32
// state tile [K x BV] stays in MFMA accumulator registers for the whole walk.
// A 1D grid dispatches eight (sequence, head) units at a time with all their
// value tiles, longest sequences first, and keeps each unit on one XCD
// (workgroup ids go round-robin over the eight XCDs), so the tiles of a unit
// share that XCD's L2 (scan_unit below).
//
// A workgroup has eight waves, two per SIMD.  Waves 0-3 (the chain) run the
// recurrence: wave w owns token tile w of the per-chunk product (R or Rbar)
// and a set of key tiles of the state.  Waves 4-7 do the per-chunk work that
// does not depend on the recurrence, beside it:
//   forward:  the output o = Qg S_c + Cq R_c of the chunk whose S_c and R_c
//             the chain has just put in LDS;
//   reverse:  Cq^T dO and Qg^T dO of the next chunk (which feed the chain as
//             fp32 addends, through LDS).
// So the chain's instruction stream holds only the dependent products, its
// operand loads and its own stores, and each SIMD can issue from the second
// wave while the chain waits on a barrier, an LDS read or an MFMA result.
// Both groups pass the same two barriers per chunk.
//
// The chunk operands a wave contracts (rows of W, F^T, F, Cq^T, Qg^T, W^T)
// go straight from global memory into MFMA operand registers, 16 bytes per
// lane, two chunks ahead.  Every global load and store inside the chunk loop
// is unconditional (clamped indices, rows past a chunk's end masked where
// they are used), so the compiler's memory counters let each use wait for
// exactly its own load and the prefetches stay in flight across steps.
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
//     Rbar_c = Cq_c^T dO_c + F_c dS_{c+1}
//     dS_c   = diag(exp2 G2_last) dS_{c+1} + Qg_c^T dO_c - W_c^T Rbar_c
#include "chunk_common.hpp"

namespace rewy {

template <int V>
using ic = std::integral_constant<int, V>;

// Value i of the lane's quad (lane 4 (l >> 2) + i): with x = glast of row
// kr + 4 (l >> 4) + (l & 3) in every lane, that is row kr + 4 (l >> 4) + i
// (DPP quad broadcast, VALU only).
__device__ __forceinline__ float glast_rows(float x, int i) {
  switch (i) {
    case 0: return dpp_mov<0x00>(x);
    case 1: return dpp_mov<0x55>(x);
    case 2: return dpp_mov<0xAA>(x);
    default: return dpp_mov<0xFF>(x);
  }
}

// Scan workgroup: the chain waves, then the side waves.
constexpr int SCAN_THREADS = 512;
constexpr int CHAIN_WAVES = 4;

// LDS tiles the chain of the forward scan shares with the output waves.
template <typename T, int K, int BV>
struct FwdTiles {
  T* Ht;  // S_c as operand, [v][k], pitch pitch<T>(K)
  T* Rt;  // R_c as operand, [v][i], pitch pitch<T>(64)
};

// The chunk range of unit (sequence rank, head) and its token range, from the
// chunk records (clamped to the inputs).
struct ScanRange {
  int n, h, c0, c1, seq_bos, seq_eos;
};
__device__ __forceinline__ ScanRange scan_range(const Args& a, int u) {
  ScanRange r;
  const int rk = u / a.H;
  r.h = u - rk * a.H;
  r.n = a.seqord[rk];  // the rk-th longest sequence
  r.c0 = a.seqoff[r.n];
  r.c1 = a.seqoff[r.n + 1];
  const ChunkInfo cfirst = load_chunk(a.chunks, r.c0 < r.c1 ? r.c0 : 0);
  const ChunkInfo clast = load_chunk(a.chunks, r.c0 < r.c1 ? r.c1 - 1 : 0);
  r.seq_bos = cfirst.bos;
  r.seq_eos = clast.bos + clast.len;
  return r;
}

// Forward scan, the chain: wave w owns token tile w of R (all value columns of
// the workgroup) and a set of key tiles of the state; it reads the W rows and
// F^T rows it contracts straight from global memory into MFMA operand
// registers (16 bytes per lane, DEPTH chunks ahead), so only S_c and R_c pass
// through LDS.  NAT: S_c and R_c are also written to global memory (the
// backward's operands).
template <typename T, int K, int V, int BV, bool NAT>
__device__ __forceinline__ void fwd_scan_chain(const Args& a, const int u, const int vt,
                                               FwdTiles<T, K, BV> sm) {
  constexpr int DEPTH = 2;
  constexpr int VE = 16 / (int)sizeof(T), KG = 4 * VE;  // elements per lane piece, per group
  constexpr int CT = BV / SUB, NKT = K / SUB;
  constexpr int NGK = K / KG, NGT = CH / KG;
  // state tiles: wave w takes key tiles w, w + 4, ... with all CT column tiles,
  // or, for K = 32, key tile w % 2 and column tile w / 2
  constexpr bool WIDE = NKT >= 4;
  constexpr int KW = WIDE ? NKT / 4 : 1, CW = WIDE ? CT : CT * NKT / 4;
  static_assert(WIDE || (NKT == 2 && CT == 2), "state tile split");
  constexpr int PK = pitch<T>(K), PA = pitch<T>(CH);
  T* const sHt = sm.Ht;
  T* const sRt = sm.Rt;

  const ScanRange sr = scan_range(a, u);
  const int H = a.H, n = sr.n, h = sr.h, c0 = sr.c0, c1 = sr.c1;
  const int w = wave_id(), l = lane_id();
  const int r16 = l & 15, g = l >> 4;
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
  uint4 ff[DEPTH][KW][NGT];  // F^T rows 16 ktile + r16, lane piece of every token group
  // G2_last of the state rows: lane l holds row kr + 4 (l >> 4) + (l & 3), and
  // each lane takes the four rows 4 (l >> 4) + i it needs from its quad
  // (glast_rows): one 4-byte load per lane instead of a 16-byte load of four
  // values that every lane of a row shares, which spent the address unit's
  // cycles on repeats
  float lam[DEPTH][KW];
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
      lam[B][j] = a.glast[cb * K + kr + 4 * g + (l & 3)];
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
  auto final_out = [&]() {
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
  };
  if (c0 >= c1) {  // empty sequence: the final state is the initial one
    final_out();
    return;
  }
  static_for<0, DEPTH>([&](auto B) {
    fetch_wu(B, c0 + B);
    fetch_fl(B, c0 + B);
  });

  auto step = [&](auto buf, int c) {
    constexpr int B = decltype(buf)::value;
    const int64_t cb = (int64_t)c * H + h;
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
    lds_barrier();  // A: S_c visible to every wave
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
    f32x4 trr[NAT ? CT : 1];
#pragma unroll
    for (int m = 0; m < CT; ++m) {
      f32x4 p = zero4();
      const T* hb = sHt + (SUB * m + r16) * PK + 4 * g;
#pragma unroll
      for (int q = 0; q < NGK; ++q) {
        if constexpr (std::is_same_v<T, bf16>) {
          const bf16x4 s0 = *reinterpret_cast<const bf16x4*>(hb + 32 * q);
          const bf16x4 s1 = *reinterpret_cast<const bf16x4*>(hb + 32 * q + SUB);
          const bf16x8 sb = __builtin_shufflevector(s0, s1, 0, 1, 2, 3, 4, 5, 6, 7);
          p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[B][q]), sb, p, 0, 0, 0);
        } else {
          const f32x4 sv = *reinterpret_cast<const f32x4*>(hb + SUB * q);
          mm16(p, __builtin_bit_cast(f32x4, wf[B][q]), sv);
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
    fetch_wu(ic<B>{}, c + DEPTH);
    lds_barrier();  // B: R_c visible to every wave
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
      for (int i = 0; i < 4; ++i) d[i] = fexp2(glast_rows(lam[B][j], i));
#pragma unroll
      for (int m = 0; m < CW; ++m) {
        const T* rb = sRt + (SUB * vtile(m) + r16) * PA + VE * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) st[j][m][i] *= d[i];
#pragma unroll
        for (int q = 0; q < NGT; ++q) mma16B<T>(st[j][m], ff[B][j][q], *reinterpret_cast<const uint4*>(rb + KG * q));
      }
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
  final_out();
}

// Forward scan, the output waves (4-7): o = Qg S_c + Cq R_c for token tile
// w - 4 of every chunk, from the S_c and R_c tiles the chain puts in LDS.  Qg
// rows are stored in the order of W (contracted with the same S operand), Cq
// row block in C-fragment order (two 16-token blocks joined per lane group, R
// read to match).
template <typename T, int K, int V, int BV>
__device__ __forceinline__ void fwd_scan_output(const Args& a, const int u, const int vt,
                                                FwdTiles<T, K, BV> sm) {
  constexpr int DEPTH = 2;
  constexpr int VE = 16 / (int)sizeof(T), KG = 4 * VE;
  constexpr int CT = BV / SUB;
  constexpr int NGK = K / KG, NGT = CH / KG;
  constexpr int PK = pitch<T>(K), PA = pitch<T>(CH);
  const T* const sHt = sm.Ht;
  const T* const sRt = sm.Rt;

  const ScanRange sr = scan_range(a, u);
  const int H = a.H, h = sr.h, c0 = sr.c0, c1 = sr.c1;
  if (c0 >= c1) return;
  const int w = wave_id() - CHAIN_WAVES, l = lane_id();
  const int r16 = l & 15, g = l >> 4;
  const int64_t gsV = (int64_t)H * V;
  using FR = typename Frag4<T>::type;
  f32x4 idf;
#pragma unroll
  for (int e = 0; e < 4; ++e) idf[e] = (4 * g + e == r16) ? 1.f : 0.f;
  const FR idt = to_frag<T>(idf);
  uint4 qf[DEPTH][NGK], cqf[DEPTH][NGT];
  auto fetch_q = [&](auto set, int c) {
    constexpr int B = decltype(set)::value;
    const int64_t cb = (int64_t)min(c, c1 - 1) * H + h;
    const T* qp = reinterpret_cast<const T*>(a.Qg) + cb * CH * K + (int64_t)(w * NGK * 64 + l) * VE;
#pragma unroll
    for (int q = 0; q < NGK; ++q) qf[B][q] = *reinterpret_cast<const uint4*>(qp + q * 64 * VE);
  };
  auto fetch_cq = [&](auto set, int c) {
    constexpr int B = decltype(set)::value;
    const int64_t cb = (int64_t)min(c, c1 - 1) * H + h;
    // Cq is lower triangular: its blocks right of the diagonal (J > w) are
    // zero and are not read (an offset past the buffer's range returns
    // zeros); blocks 2 q and 2 q + 1 joined into one operand (bf16, the slot
    // assignment of C-fragment order in common.hpp)
    const GBuf bc = gbuf(reinterpret_cast<const T*>(a.Cq) + cb * CH * CH, CH * CH * sizeof(T));
    auto off = [&](int J) { return J > w ? OOB : (uint32_t)(((w * NSUB + J) * 64 + l) * 4 * (int)sizeof(T)); };
#pragma unroll
    for (int q = 0; q < NGT; ++q) {
      if constexpr (std::is_same_v<T, bf16>) {
        const uint2 x0 = gld8(bc, off(2 * q)), x1 = gld8(bc, off(2 * q + 1));
        cqf[B][q] = uint4{x0.x, x0.y, x1.x, x1.y};
      } else {
        cqf[B][q] = gld16(bc, off(q));
      }
    }
  };
  static_for<0, DEPTH>([&](auto B) {
    fetch_q(B, c0 + B);
    fetch_cq(B, c0 + B);
  });

  // The output of a chunk is stored one step late: its Cq R product is issued
  // at the end of the chunk's step, and its transpose and store come in the
  // next step, so their latency overlaps that step's work.  pbos / plen are
  // the rows of the pending chunk; plen = 0 drops the stores (nothing pending).
  f32x4 pend[CT], ptr[CT];
  int pbos = 0, plen = 0;
#pragma unroll
  for (int m = 0; m < CT; ++m) pend[m] = zero4();
  auto out_transpose = [&]() {  // transposed by the identity product into row pieces
#pragma unroll
    for (int m = 0; m < CT; ++m) {
      ptr[m] = zero4();
      mm16(ptr[m], to_frag<T>(pend[m]), idt);
    }
  };
  auto out_store = [&]() {  // rows past the chunk's end fall outside the buffer
    const GBuf bo = gbuf(reinterpret_cast<T*>(a.o) + ((int64_t)pbos * H + h) * V, tile_bytes<T>(plen, gsV, V));
#pragma unroll
    for (int m = 0; m < CT; ++m) {
      const uint32_t off = (uint32_t)(((int64_t)(SUB * w + r16) * gsV + vt * BV + SUB * m + 4 * g) * (int64_t)sizeof(T));
      if constexpr (std::is_same_v<T, bf16>) gst8(bo, off, __builtin_bit_cast(uint2, to_frag<T>(ptr[m])));
      else gst16(bo, off, __builtin_bit_cast(uint4, ptr[m]));
    }
  };

  auto step = [&](auto buf, int c) {
    constexpr int B = decltype(buf)::value;
    const int bos = sr.seq_bos + (c - c0) * CH, len = min(CH, sr.seq_eos - bos);
    out_transpose();  // the previous chunk's output rows
    lds_barrier();    // A: S_c in LDS
    f32x4 po[CT];
#pragma unroll
    for (int m = 0; m < CT; ++m) {
      po[m] = zero4();
      const T* hb = sHt + (SUB * m + r16) * PK + 4 * g;
#pragma unroll
      for (int q = 0; q < NGK; ++q) {
        if constexpr (std::is_same_v<T, bf16>) {
          const bf16x4 s0 = *reinterpret_cast<const bf16x4*>(hb + 32 * q);
          const bf16x4 s1 = *reinterpret_cast<const bf16x4*>(hb + 32 * q + SUB);
          const bf16x8 sb = __builtin_shufflevector(s0, s1, 0, 1, 2, 3, 4, 5, 6, 7);
          po[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qf[B][q]), sb, po[m], 0, 0, 0);
        } else {
          const f32x4 sv = *reinterpret_cast<const f32x4*>(hb + SUB * q);
          mm16(po[m], __builtin_bit_cast(f32x4, qf[B][q]), sv);
        }
      }
    }
    out_store();
    fetch_q(ic<B>{}, c + DEPTH);
    lds_barrier();  // B: R_c in LDS
#pragma unroll
    for (int m = 0; m < CT; ++m) {
      const T* rb = sRt + (SUB * m + r16) * PA + 4 * g;
#pragma unroll
      for (int q = 0; q < NGT; ++q) mma16B<T>(po[m], cqf[B][q], perm_row<T>(rb, q));
      pend[m] = po[m];
    }
    pbos = bos;
    plen = len;
    fetch_cq(ic<B>{}, c + DEPTH);
  };
  for (int c = c0;;) {
    step(ic<0>{}, c);
    if (++c >= c1) break;
    step(ic<1>{}, c);
    if (++c >= c1) break;
  }
  out_transpose();  // the last chunk's output rows
  out_store();
}

// LDS of the reverse scan, shared by the chain and the side waves.  X and Y
// hold Cq^T dO and Qg^T dO of one chunk as fp32 MFMA accumulator tiles (lane
// l's four values of a 16 x 16 tile at [tile][l]), double-buffered by chunk
// parity.
template <typename T, int K, int BV>
struct BwdTiles {
  T* Dt;       // dS_{c+1} as operand, [v][k], pitch pitch<T>(K)
  T* Ot;       // [2] dO as operand, [v][j], pitch pitch<T>(64), by chunk parity
  T* Rbt;      // Rbar_c as operand, [v][i], pitch pitch<T>(64)
  f32x4* X;    // [2][NSUB * CT][64]: tile (token tile, column tile)
  f32x4* Y;    // [2][NKT * CT][64]: tile (key tile, column tile)
};

// Reverse scan, the chain: wave w owns token tile w of Rbar and a set of key
// tiles of dS; F rows and W^T rows go straight from global memory into operand
// registers; dS_{c+1} and Rbar_c pass through LDS, and Cq^T dO and Qg^T dO of
// the chunk arrive there from the side waves.
template <typename T, int K, int V, int BV>
__device__ __forceinline__ void bwd_scan_chain(const Args& a, const int u, const int vt,
                                               BwdTiles<T, K, BV> sm) {
  constexpr int DEPTH = 2;
  constexpr int VE = 16 / (int)sizeof(T), KG = 4 * VE;
  constexpr int CT = BV / SUB, NKT = K / SUB;
  constexpr int NGK = K / KG, NGT = CH / KG;
  constexpr bool WIDE = NKT >= 4;
  constexpr int KW = WIDE ? NKT / 4 : 1, CW = WIDE ? CT : CT * NKT / 4;
  static_assert(WIDE || (NKT == 2 && CT == 2), "state tile split");
  constexpr int PK = pitch<T>(K), PA = pitch<T>(CH);

  const ScanRange sr = scan_range(a, u);
  const int H = a.H, n = sr.n, h = sr.h, c0 = sr.c0, c1 = sr.c1;
  const int w = wave_id(), l = lane_id();
  const int r16 = l & 15, g = l >> 4;
  auto ktile = [&](int j) { return WIDE ? w + 4 * j : w % NKT; };
  auto vtile = [&](int m) { return WIDE ? m : (w / NKT) * CW + m; };

  uint4 ff[DEPTH][NGK];      // F row 16 w + r16 (keys)
  uint4 wf[DEPTH][KW][NGT];  // W^T row 16 ktile + r16 (tokens)
  float lam[DEPTH][KW];  // G2_last, one row per lane (as in the forward chain)
  using FR = typename Frag4<T>::type;
  // identity as the B operand of a 16-long product (C = X^T I, exact): the
  // natural-layout dS_{c+1} leaves the registers as pieces of one row
  f32x4 idf;
#pragma unroll
  for (int e = 0; e < 4; ++e) idf[e] = (4 * g + e == r16) ? 1.f : 0.f;
  const FR idt = to_frag<T>(idf);
  // chunks are walked from the last; before the first one the first is read
  // again (valid memory, never used)
  auto fetch = [&](auto set, int c) {
    constexpr int B = decltype(set)::value;
    const int64_t cb = (int64_t)max(c, c0) * H + h;
    const T* fp = reinterpret_cast<const T*>(a.F) + cb * CH * K + (int64_t)(w * NGK * 64 + l) * VE;
#pragma unroll
    for (int q = 0; q < NGK; ++q) ff[B][q] = *reinterpret_cast<const uint4*>(fp + q * 64 * VE);
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      const int kr = SUB * ktile(j);
      const T* wp = reinterpret_cast<const T*>(a.Wt) + cb * K * CH + (int64_t)(ktile(j) * NGT * 64 + l) * VE;
#pragma unroll
      for (int q = 0; q < NGT; ++q) wf[B][j][q] = *reinterpret_cast<const uint4*>(wp + q * 64 * VE);
      lam[B][j] = a.glast[cb * K + kr + 4 * g + (l & 3)];
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
  lds_barrier();  // P: the side waves' prologue (X, Y of the last chunk) meets here

  auto step = [&](auto buf, int c) {
    constexpr int B = decltype(buf)::value;
    const int64_t cb = (int64_t)c * H + h;
    const f32x4* Xc = sm.X + (c & 1) * (NSUB * CT * 64);
    const f32x4* Yc = sm.Y + (c & 1) * (NKT * CT * 64);
    // dS_{c+1}: operand [v][k] and natural [k][v].  The natural copy's
    // transposes are issued here and stored after the barrier, whose wait
    // covers their latency.
    f32x4 trd[KW][CW];
#pragma unroll
    for (int j = 0; j < KW; ++j)
#pragma unroll
      for (int m = 0; m < CW; ++m) {
        const int kr = SUB * ktile(j), vc = SUB * vtile(m);
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = tof(fromf<T>(st[j][m][i]));
        st_tile_T<T>(x, sm.Dt + vc * PK + kr, PK);
        trd[j][m] = zero4();  // column-blocked [V/16][K][16]
        mm16(trd[j][m], to_frag<T>(x), idt);
      }
    lds_barrier();  // A: dS_{c+1} visible; X_c, Y_c complete since the previous step
#pragma unroll
    for (int j = 0; j < KW; ++j)
#pragma unroll
      for (int m = 0; m < CW; ++m)
        *reinterpret_cast<FR*>(reinterpret_cast<T*>(a.dhbuf) + cb * K * V +
                               ((int64_t)(vt * CT + vtile(m)) * K + SUB * ktile(j) + r16) * SUB + 4 * g) =
            to_frag<T>(trd[j][m]);
    // Rbar = Cq^T dO + F dS+ for token tile w (rows past the end are zero: F
    // and Cq vanish there)
#pragma unroll
    for (int m = 0; m < CT; ++m) {
      f32x4 acc = Xc[(w * CT + m) * 64 + l];
      const T* db = sm.Dt + (SUB * m + r16) * PK + VE * g;
#pragma unroll
      for (int q = 0; q < NGK; ++q) mma16B<T>(acc, ff[B][q], *reinterpret_cast<const uint4*>(db + KG * q));
      st_tile_T<T>(acc, sm.Rbt + (SUB * m) * PA + SUB * w, PA);
      // Rbar in the C-fragment order of its 16 x 16 tiles: a wave writes one
      // contiguous tile
      *reinterpret_cast<FR*>(reinterpret_cast<T*>(a.Rbt) + cb * V * CH +
                             (((int64_t)(vt * CT + m) * NSUB + w) * 64 + l) * 4) = to_frag<T>(acc);
    }
    lds_barrier();  // B: Rbar_c visible
    // dS = diag(exp2 G2_last) dS+ + Qg^T dO - W^T Rbar (W^T negated by its sign bits)
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      f32x4 d;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = fexp2(glast_rows(lam[B][j], i));
      uint4 wn[NGT];
      constexpr unsigned SGN = sizeof(T) == 2 ? 0x80008000u : 0x80000000u;
#pragma unroll
      for (int q = 0; q < NGT; ++q) {
        const uint4 x = wf[B][j][q];
        wn[q] = uint4{x.x ^ SGN, x.y ^ SGN, x.z ^ SGN, x.w ^ SGN};
      }
#pragma unroll
      for (int m = 0; m < CW; ++m) {
        const T* rb = sm.Rbt + (SUB * vtile(m) + r16) * PA + VE * g;
        const f32x4 y = Yc[(ktile(j) * CT + vtile(m)) * 64 + l];
#pragma unroll
        for (int i = 0; i < 4; ++i) st[j][m][i] = st[j][m][i] * d[i] + y[i];
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

// Reverse scan, the side waves (4-7): X = Cq^T dO (token tile w - 4) and
// Y = Qg^T dO (the key tiles chain wave w - 4 holds) of the chunk after the
// chain's current one in walking order, into the X / Y buffer of that chunk's
// parity.  dO is staged into LDS transposed by these 256 threads.
template <typename T, int K, int V, int BV>
__device__ __forceinline__ void bwd_scan_side(const Args& a, const int u, const int vt,
                                              BwdTiles<T, K, BV> sm) {
  constexpr int DEPTH = 2, NTH = SCAN_THREADS - 64 * CHAIN_WAVES;
  constexpr int VE = 16 / (int)sizeof(T), KG = 4 * VE;
  constexpr int CT = BV / SUB, NKT = K / SUB;
  constexpr int NGT = CH / KG;
  constexpr bool WIDE = NKT >= 4;
  constexpr int KW = WIDE ? NKT / 4 : 1, CW = WIDE ? CT : CT * NKT / 4;
  constexpr int PA = pitch<T>(CH);
  // dO rows as staged by the threads: 8-byte pieces (4 elements)
  constexpr int OE = 8 / (int)sizeof(T), OPER = BV / OE;
  constexpr int ON = CH * BV * (int)sizeof(T) / (NTH * 8);  // dO pieces per thread
  static_assert(ON >= 1 && CH * BV * (int)sizeof(T) == NTH * 8 * ON, "dO staging split");

  const ScanRange sr = scan_range(a, u);
  const int H = a.H, h = sr.h, c0 = sr.c0, c1 = sr.c1;
  if (c0 >= c1) return;
  const int w = wave_id() - CHAIN_WAVES, l = lane_id(), tid = threadIdx.x - 64 * CHAIN_WAVES;
  const int64_t gsV = (int64_t)H * V;
  auto ktile = [&](int j) { return WIDE ? w + 4 * j : w % NKT; };
  auto vtile = [&](int m) { return WIDE ? m : (w / NKT) * CW + m; };

  uint4 cf[DEPTH][NGT];      // Cq^T row 16 w + r16 (tokens j)
  uint4 qf[DEPTH][KW][NGT];  // Qg^T row 16 ktile + r16 (tokens)
  uint2 of[DEPTH][ON];       // dO pieces
  auto chunk_of = [&](int c) { return max(c, c0); };
  auto fetch = [&](auto set, int c) {
    constexpr int B = decltype(set)::value;
    const int cc = chunk_of(c);
    const int bos = sr.seq_bos + (cc - c0) * CH, len = min(CH, sr.seq_eos - bos);
    const int64_t cb = (int64_t)cc * H + h;
    // Cq^T is upper triangular: a piece whose columns (tokens i) all lie
    // before the wave's rows is zero and is not read (an offset past the
    // buffer's range returns zeros)
    const GBuf bcq = gbuf(reinterpret_cast<const T*>(a.Cqt) + cb * CH * CH, CH * CH * sizeof(T));
#pragma unroll
    for (int q = 0; q < NGT; ++q)
      cf[B][q] = gld16(bcq, KG * (q + 1) <= SUB * w ? OOB : (uint32_t)(((w * NGT + q) * 64 + l) * VE * (int)sizeof(T)));
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      const T* qp = reinterpret_cast<const T*>(a.Qgt) + cb * K * CH + (int64_t)(ktile(j) * NGT * 64 + l) * VE;
#pragma unroll
      for (int q = 0; q < NGT; ++q) qf[B][j][q] = *reinterpret_cast<const uint4*>(qp + q * 64 * VE);
    }
    const T* op = reinterpret_cast<const T*>(a.dO) + ((int64_t)bos * H + h) * V + vt * BV;
#pragma unroll
    for (int e = 0; e < ON; ++e) {
      const int idx = tid + e * NTH, r = idx / OPER, c8 = (idx % OPER) * OE;
      of[B][e] = *reinterpret_cast<const uint2*>(op + (int64_t)min(r, len - 1) * gsV + c8);
    }
  };
  // dO of chunk c (register set B) into its LDS buffer, transposed, rows past
  // the chunk's end as zeros
  auto put_dO = [&](auto set, int c) {
    constexpr int B = decltype(set)::value;
    const int cc = chunk_of(c);
    const int bos = sr.seq_bos + (cc - c0) * CH, len = min(CH, sr.seq_eos - bos);
    T* ot = sm.Ot + (c & 1) * (BV * PA);
#pragma unroll
    for (int e = 0; e < ON; ++e) {
      const int idx = tid + e * NTH, r = idx / OPER, c8 = (idx % OPER) * OE;
      union {
        uint2 u;
        T v[OE];
      } x;
      x.u = of[B][e];
#pragma unroll
      for (int k = 0; k < OE; ++k) ot[(c8 + k) * PA + r] = r < len ? x.v[k] : fromf<T>(0.f);
    }
  };
  // X and Y of chunk c from register set B and its dO buffer
  auto products = [&](auto set, int c) {
    constexpr int B = decltype(set)::value;
    const T* ot = sm.Ot + (c & 1) * (BV * PA);
    f32x4* X = sm.X + (c & 1) * (NSUB * CT * 64);
    f32x4* Y = sm.Y + (c & 1) * (NKT * CT * 64);
    const int r16 = l & 15, g = l >> 4;
#pragma unroll
    for (int m = 0; m < CT; ++m) {
      f32x4 acc = zero4();
      const T* ob = ot + (SUB * m + r16) * PA + VE * g;
#pragma unroll
      for (int q = 0; q < NGT; ++q) mma16B<T>(acc, cf[B][q], *reinterpret_cast<const uint4*>(ob + KG * q));
      X[(w * CT + m) * 64 + l] = acc;
    }
#pragma unroll
    for (int j = 0; j < KW; ++j)
#pragma unroll
      for (int m = 0; m < CW; ++m) {
        f32x4 acc = zero4();
        const T* ob = ot + (SUB * vtile(m) + r16) * PA + VE * g;
#pragma unroll
        for (int q = 0; q < NGT; ++q) mma16B<T>(acc, qf[B][j][q], *reinterpret_cast<const uint4*>(ob + KG * q));
        Y[(ktile(j) * CT + vtile(m)) * 64 + l] = acc;
      }
  };

  // register sets by chunk: the last chunk takes set 0, the one before set 1, ...
  static_for<0, DEPTH>([&](auto B) { fetch(B, c1 - 1 - B); });
  put_dO(ic<0>{}, c1 - 1);
  lds_barrier();  // P: dO of the last chunk staged
  products(ic<0>{}, c1 - 1);
  fetch(ic<0>{}, c1 - 1 - DEPTH);

  // in the chain's step for chunk c (register set B), chunk c - 1 (set B ^ 1)
  auto step = [&](auto buf, int c) {
    constexpr int SB = decltype(buf)::value ^ 1;
    put_dO(ic<SB>{}, c - 1);
    lds_barrier();  // A
    products(ic<SB>{}, c - 1);
    fetch(ic<SB>{}, c - 1 - DEPTH);
    lds_barrier();  // B
  };
  for (int c = c1 - 1;;) {
    step(ic<0>{}, c);
    if (--c < c0) break;
    step(ic<1>{}, c);
    if (--c < c0) break;
  }
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

template <typename T, int K, int BV>
__device__ __forceinline__ FwdTiles<T, K, BV> fwd_tiles() {
  __shared__ __align__(16) T sHt[BV * pitch<T>(K)];
  __shared__ __align__(16) T sRt[BV * pitch<T>(CH)];
  return FwdTiles<T, K, BV>{sHt, sRt};
}
template <typename T, int K, int BV>
__device__ __forceinline__ BwdTiles<T, K, BV> bwd_tiles() {
  constexpr int CT = BV / SUB, NKT = K / SUB;
  __shared__ __align__(16) T sDt[BV * pitch<T>(K)];
  __shared__ __align__(16) T sOt[2 * BV * pitch<T>(CH)];
  __shared__ __align__(16) T sRbt[BV * pitch<T>(CH)];
  __shared__ f32x4 sX[2 * NSUB * CT * 64];
  __shared__ f32x4 sY[2 * NKT * CT * 64];
  return BwdTiles<T, K, BV>{sDt, sOt, sRbt, sX, sY};
}

// The forward scan with the output product (OUT has SCAN_OUTPUT; with
// SCAN_NATURAL the chain also writes S_c and R_c for the backward).
template <typename T, int K, int V, int BV, int OUT>
__global__ __launch_bounds__(SCAN_THREADS) void k_fwd_scan(Args a) {
  static_assert(OUT & SCAN_OUTPUT, "the output waves form o");
  int u, vt, sc;
  if (!scan_unit<V / BV, 1>(a, u, vt, sc)) return;
  const auto sm = fwd_tiles<T, K, BV>();
  if (wave_id() < CHAIN_WAVES)
    fwd_scan_chain<T, K, V, BV, (OUT & SCAN_NATURAL) != 0>(a, u, vt, sm);
  else
    fwd_scan_output<T, K, V, BV>(a, u, vt, sm);
}
template <typename T, int K, int V, int BV>
__global__ __launch_bounds__(SCAN_THREADS) void k_bwd_scan(Args a) {
  int u, vt, sc;
  if (!scan_unit<V / BV, 1>(a, u, vt, sc)) return;
  const auto sm = bwd_tiles<T, K, BV>();
  if (wave_id() < CHAIN_WAVES) bwd_scan_chain<T, K, V, BV>(a, u, vt, sm);
  else bwd_scan_side<T, K, V, BV>(a, u, vt, sm);
}
// Both scans of the backward under recompute in one launch: they read
// disjoint operands and write disjoint outputs, so the reverse scan (the
// longer one, dispatched first within each group of units) and the forward
// recompute scan run side by side, each on its own share of the CUs.  Wider
// value tiles halve the operand reads of each scan.  The forward recompute
// scan has no output product: its waves 4-7 only pass the chain's two
// barriers per chunk.
template <typename T, int K, int V, int BV>
__global__ __launch_bounds__(SCAN_THREADS) void k_scans(Args a) {
  int u, vt, sc;
  if (!scan_unit<V / BV, 2>(a, u, vt, sc)) return;
  if (sc == 0) {
    const auto sm = bwd_tiles<T, K, BV>();
    if (wave_id() < CHAIN_WAVES) bwd_scan_chain<T, K, V, BV>(a, u, vt, sm);
    else bwd_scan_side<T, K, V, BV>(a, u, vt, sm);
  } else if (wave_id() < CHAIN_WAVES) {
    fwd_scan_chain<T, K, V, BV, true>(a, u, vt, fwd_tiles<T, K, BV>());
  } else {
    const ScanRange sr = scan_range(a, u);
    for (int c = sr.c0; c < sr.c1; ++c) {
      lds_barrier();
      lds_barrier();
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
  const dim3 grid = scan_grid(a, a.V / BV, 1), block(SCAN_THREADS);
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
  const dim3 grid = scan_grid(a, a.V / BV, 1), block(SCAN_THREADS);
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
  const dim3 grid = scan_grid(a, a.V / BV, 2), block(SCAN_THREADS);
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
