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
#define REWY_OPAQUE_IDS
#include "chunk_ops.hpp"

namespace rewy {

// Token range of sequence n.  Device cu_seqlens are clamped to the packed
// token axis [0, B T) and made non-decreasing, so a malformed array (checked
// only when a host copy is given) yields empty or overlapping sequences but
// never a chunk outside the inputs, and never more than nc_max chunk slots.
__device__ __forceinline__ void seq_range(const Args& a, int n, int& bos, int& eos) {
  if (a.cu) {
    const int BT = a.B * a.T;
    bos = min(max(a.cu[n], 0), BT);
    eos = min(max(a.cu[n + 1], bos), BT);
  } else {
    bos = n * a.T;
    eos = bos + a.T;
  }
}

__global__ void k_chunk_table(Args a) {
  __shared__ int s_total;
  if (threadIdx.x == 0) {
    int off = 0;
    for (int n = 0; n < a.N; ++n) {
      int bos, eos;
      seq_range(a, n, bos, eos);
      a.seqoff[n] = min(off, a.nc_max);
      off += (eos - bos + CH - 1) / CH;
    }
    a.seqoff[a.N] = min(off, a.nc_max);
    s_total = min(off, a.nc_max);
  }
  __syncthreads();  // full fence: the other threads read seqoff from global memory
  const int total = s_total;
  // Scan order: sequences by chunk count, longest first (ties by index), so
  // that the scans dispatch their longest serial chains first.  Identity
  // without cu_seqlens (equal lengths) and beyond 1024 sequences.
  {
    __shared__ int s_cnt[1024];
    const bool sort = a.cu && a.N <= 1024;
    if (sort)
      for (int i = threadIdx.x; i < a.N; i += blockDim.x) s_cnt[i] = a.seqoff[i + 1] - a.seqoff[i];
    __syncthreads();
    for (int i = threadIdx.x; i < a.N; i += blockDim.x) {
      int rank = i;
      if (sort) {
        const int ni = s_cnt[i];
        rank = 0;
        for (int j = 0; j < a.N; ++j) rank += (s_cnt[j] > ni) || (s_cnt[j] == ni && j < i);
      }
      a.seqord[rank] = i;
    }
  }
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
      int bos, eos;
      seq_range(a, lo, bos, eos);
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
  REWY_LAUNCH(k_chunk_table, dim3(1), dim3(256), s, a);
  return hipGetLastError();
}

// Persistent workgroups of four waves, two per compute unit, process
// chunk-heads item = blockIdx.x + i*gridDim.x (item = chunk * H + head); while
// one workgroup waits on memory, a barrier or the serial part of the solve,
// the other computes.  LDS is two regions reused phase by phase (X: the raw,
// then centred key and query operands, then A, then E^T and Z^T; Y: the
// prefix totals, then L, then A in the operand type), which keeps a
// workgroup within half of the compute unit's LDS.  The next item's k, q,
// beta, gates and v are read into registers while the current item computes
// (k, q and beta once k and q are staged, the gates after the elementwise
// phase, v once this item's v is in Z^T; the one-column layouts issue them
// before the solve, v for the item itself).
//
// MODE: the PREP_* sets this launch writes (a compile-time constant, so the
// loop body holds no flag tests and no pointers of unused outputs).
template <typename T, int K, int V, int MODE>
__global__ __launch_bounds__(256, (MODE & PREP_EW) ? 1 : 2) void k_fwd_prep(Args) {
  // the erase/write form runs one workgroup per CU: the erase gate of the
  // thread's rows and the write gate's v pieces need registers
  constexpr bool EW = MODE & PREP_EW;
  // the gate formed from its pre-activation x, A_log and dt_bias (Args::gate_lb
  // selects the softplus or the bounded form)
  constexpr bool GIN = MODE & PREP_GIN;
  constexpr int NTH = 256, NW = NTH / 64;
  constexpr bool BF = std::is_same_v<T, bf16>;
  constexpr int PK = pitch<T>(K);   // T rows of K
  constexpr int PL = CH + 4;        // fp32 rows of 64
  constexpr int PA = pitch<T>(CH);  // T rows of 64
  using GC = GateCols<K>;
  constexpr int RS = GC::RS;
  constexpr int NSL = (GC::NG + NTH - 1) / NTH;  // gate slots (column, segment) per thread
  // bf16 with two slots per thread: the slots are adjacent columns of the same
  // rows, so the element-wise phase moves bf16 pairs (4-byte LDS and global
  // accesses, one conversion per pair)
  constexpr bool PAIR = BF && NSL == 2;
  constexpr int VE = 16 / (int)sizeof(T);

  constexpr int SZ_K = CH * PK * (int)sizeof(T), SZ_L = CH * PL * 4;
  constexpr int SZ_ET = K * PA * (int)sizeof(T), SZ_ZT = V * PA * (int)sizeof(T);
  // bf16: A (fp32) leaves X for Y, as the operand copy, before E^T and Z^T
  // are written over it; fp32: A is the operand itself and stays beside them
  constexpr int SZ_X = cmax(3 * SZ_K, BF ? cmax(SZ_L, SZ_ET + SZ_ZT) : SZ_L + SZ_ET + SZ_ZT);
  constexpr int SZ_Y = cmax(SZ_L, NSUB * K * 4);
  __shared__ __align__(16) char sX[SZ_X];
  __shared__ __align__(16) char sY[SZ_Y];
  __shared__ __align__(16) float sFac[10 * K];
  __shared__ float sMid[NSUB * K], sGf[NSUB * K], sGl[NSUB * K], sGn[K];
  __shared__ float sBeta[CH];
  __shared__ int sFlag[NSUB * (K / SUB)];  // wide (sub-chunk, 16-feature block)
  T* const sK = reinterpret_cast<T*>(sX);  // S0-S3: raw k, then Kc in place
  T* const sQ = sK + CH * PK;              //        raw q, then Qa in place
  T* const sKa = sQ + CH * PK;             //        Ka
  float* const sA = reinterpret_cast<float*>(sX);                      // S4-S5
  T* const sEt = reinterpret_cast<T*>(sX + (BF ? 0 : SZ_L));           // S5: E^T [k][j]
  T* const sZt = sEt + K * PA;                                         //     Z^T [v][j]
  float* const sTot = reinterpret_cast<float*>(sY);                    // S0-S1
  float* const sL = reinterpret_cast<float*>(sY);                      // S2-S4
  T* const sAb = reinterpret_cast<T*>(sY);                             // S5 (bf16)

  // the arguments are read through a kernarg view renewed at every phase, so
  // that pointers and per-item output addresses are re-read where used
  // instead of living (and spilling) across the item loop
  KernArgs kargs;
  auto ka = [&]() -> const Args& { return kargs.template get<Args>(); };
  const int H = ka().H;
  const int total = ka().nc_max * H;
  const int64_t gsK = (int64_t)H * K, gsV = (int64_t)H * V;

  // gate slots; their G registers hold the next item's raw gates from the end
  // of the elementwise phase (their last use) to the next item's prefix
  GC gc[NSL];
#pragma unroll
  for (int s = 0; s < NSL; ++s) {
    if constexpr (PAIR) gc[s].init_pair(threadIdx.x, s);
    else gc[s].init(threadIdx.x + s * NTH);
  }
  TileRegs<T, CH, K, NTH> pk, pq;
  // v for Z^T: bf16 threads take rows (2p, 2p + 1), p = slot % 32, and the
  // eight columns from 8 (slot / 32), so each Z^T write is one 4-byte pair of
  // tokens (conflict-free across the wave); fp32 keeps the row-piece mapping
  static constexpr int VSL = (CH / 2) * (V / 8);              // (row pair, column piece) slots
  static constexpr int VPT = BF ? (VSL + NTH - 1) / NTH : 1;  // slots per thread
  Staged<T, CH, V, NTH> pv;
  uint4 pv2[2 * VPT];
  uint4 etr[NSL][RS / VE];  // E^T of this thread's rows, from the elementwise phase to S5
  uint32_t pbeta = 0u;      // raw bits of the next item's beta for row tid
  // erase/write form: raw bits of the next item's erase gate at this thread's
  // rows and columns, and the write gate in the layout of the staged v
  uint32_t bwr[EW ? NSL : 1][EW ? RS : 1];
  // gate in the kernel: A_log of the next item's head and dt_bias of each
  // slot's column (raw bits)
  uint32_t gal = 0u, gdtb[GIN ? NSL : 1];
  uint4 pw2[EW && BF ? 2 * VPT : 1];
  Staged<T, CH, V, NTH> pw;
  // The fetches take the item's chunk record, read one item ahead (its
  // scalar load completes during the previous item instead of stalling here).
  // The next item's fetches are issued on every path, also for an empty chunk
  // slot or past the last item (bounds-checked loads read zeros there; beta's
  // row is clamped to a valid one): a fetch under a condition leaves its
  // registers with two possible sources at the loop head, and the copies that
  // merge them wait for the loads at once.
  auto fetch_kq = [&](int item, const ChunkInfo& ci, int tid) {
    const int h = item % H;
    const int64_t t0 = ci.bos;
    pk.load(gbuf(reinterpret_cast<const T*>(ka().k) + (t0 * H + h) * K, tile_bytes<T>(ci.len, gsK, K)), gsK, tid);
    pq.load(gbuf(reinterpret_cast<const T*>(ka().q) + (t0 * H + h) * K, tile_bytes<T>(ci.len, gsK, K)), gsK, tid);
    if constexpr (!EW) pbeta = ld_beta_raw(ka().beta, ka().beta_f32, (t0 + min(tid, max(ci.len - 1, 0))) * H + h);
  };
  auto fetch_v = [&](int item, const ChunkInfo& ci, int tid) {
    const int h = item % H;
    const int64_t t0 = ci.bos;
    if constexpr (BF) {
      const GBuf bv = gbuf(reinterpret_cast<const T*>(ka().v) + (t0 * H + h) * V, tile_bytes<T>(ci.len, gsV, V));
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int sl = tid + j * NTH, p = sl % 32, c0 = (sl / 32) * 8;
        const bool ok = sl < VSL;
        pv2[2 * j] = gld16(bv, ok ? (uint32_t)(((int64_t)(2 * p) * gsV + c0) * 2) : OOB);
        pv2[2 * j + 1] = gld16(bv, ok ? (uint32_t)(((int64_t)(2 * p + 1) * gsV + c0) * 2) : OOB);
        if constexpr (EW) {
          const GBuf bw = gbuf(reinterpret_cast<const T*>(ka().wg) + (t0 * H + h) * V, tile_bytes<T>(ci.len, gsV, V));
          pw2[2 * j] = gld16(bw, ok ? (uint32_t)(((int64_t)(2 * p) * gsV + c0) * 2) : OOB);
          pw2[2 * j + 1] = gld16(bw, ok ? (uint32_t)(((int64_t)(2 * p + 1) * gsV + c0) * 2) : OOB);
        }
      }
    } else {
      pv.load(reinterpret_cast<const T*>(ka().v) + (t0 * H + h) * V, gsV, ci.len, tid);
      if constexpr (EW) pw.load(reinterpret_cast<const T*>(ka().wg) + (t0 * H + h) * V, gsV, ci.len, tid);
    }
  };
  auto fetch_g = [&](int item, const ChunkInfo& ci) {
    const int h = item % H;
    if constexpr (GIN) {
      const GBuf bd = gbuf(ka().dt_bias + (int64_t)h * K, K * 4);
      if constexpr (PAIR) {
        gc[0].template load_x_pair<T>(gc[1], ka(), (int64_t)ci.bos, h, ci.len, K);
        const uint2 d2 = gld8(bd, gc[0].c * 4);
        gdtb[0] = d2.x;
        gdtb[1] = d2.y;
      } else {
#pragma unroll
        for (int s = 0; s < NSL; ++s) {
          gc[s].template load_x<T>(ka(), (int64_t)ci.bos, h, ci.len, K);
          gdtb[s] = gld4(bd, gc[s].c * 4);
        }
      }
      gal = gld4(gbuf(ka().a_log, ka().H * 4), h * 4);
    } else if constexpr (PAIR) {
      gc[0].load_pair(gc[1], ka(), (int64_t)ci.bos, h, ci.len, K);
    } else {
#pragma unroll
      for (int s = 0; s < NSL; ++s) gc[s].load(ka(), (int64_t)ci.bos, h, ci.len, K, 0);
    }
    if constexpr (EW) {  // erase gate rows past the end read as zero
      const GBuf bb = gbuf(reinterpret_cast<const T*>(ka().beta) + ((int64_t)ci.bos * H + h) * K,
                           tile_bytes<T>(ci.len, gsK, K));
#pragma unroll
      for (int s = 0; s < NSL; ++s)
#pragma unroll
        for (int r = 0; r < RS; ++r) {
          const uint32_t off = (uint32_t)((((int64_t)gc[s].seg * RS + r) * gsK + gc[s].c) * (int64_t)sizeof(T));
          if constexpr (sizeof(T) == 2) bwr[s][r] = gld2(bb, off);
          else bwr[s][r] = gld4(bb, off);
        }
    }
  };

  // (the grid never exceeds the item count, so blockIdx.x < total)
  ChunkInfo cnext = load_chunk(ka().chunks, min((int)blockIdx.x, total - 1) / H);
  fetch_kq(blockIdx.x, cnext, threadIdx.x);
  fetch_g(blockIdx.x, cnext);
  if constexpr (PAIR) fetch_v(blockIdx.x, cnext, threadIdx.x);
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    kargs.renew();
    const int tid = opaque_tid<NTH>(), w = wave_id();
    // slot indices opaque per item: addresses derived from them are recomputed
    // rather than hoisted out of the item loop (where they would stay live and
    // spill)
#pragma unroll
    for (int s = 0; s < NSL; ++s) {
      asm volatile("" : "+v"(gc[s].c), "+v"(gc[s].seg));
      __builtin_assume(gc[s].c >= 0 && gc[s].c < K && gc[s].seg >= 0 && gc[s].seg < NSUB);
    }
    const int c = item / H, h = item - c * H;
    const ChunkInfo ci = cnext;
    const int n = ci.len;
    // the next item's record (the last one again past the end: never used)
    cnext = load_chunk(ka().chunks, min(item + (int)gridDim.x, total - 1) / H);
    if (n == 0) {  // uniform: an empty chunk slot
      fetch_kq(item + gridDim.x, cnext, tid);
      fetch_g(item + gridDim.x, cnext);
      if constexpr (PAIR) fetch_v(item + gridDim.x, cnext, tid);
      continue;
    }
    const int64_t t0 = ci.bos, cb = (int64_t)c * H + h;

    // ---- S0: staged inputs into LDS, local gate prefix ----------------------
    pk.store(sK, PK, tid);
    pq.store(sQ, PK, tid);
    if (tid < CH) sBeta[tid] = tid < n ? beta_val(pbeta, ka().beta_f32) : 0.f;
    if (tid < NSUB * (K / SUB)) sFlag[tid] = 0;
    if constexpr (GIN) {
      const float ea = fexp2(__uint_as_float(gal) * LOG2E);
#pragma unroll
      for (int s = 0; s < NSL; ++s) gc[s].template kda_gate<T>(ea, __uint_as_float(gdtb[s]), ka().gate_lb);
    }
#pragma unroll
    for (int s = 0; s < NSL; ++s) gc[s].template prefix_local<GIN>(sTot, n);
    lds_barrier();
    kargs.renew();

    // ---- S1: finish the prefix, statistics ----------------------------------
    // the next item's k, q and beta (their registers are free once staged),
    // issued here so that the rest of the item covers their latency; the
    // one-column layouts issue them with this item's v and the gates before
    // the solve (below), where their registers fit without spilling
    if constexpr (PAIR) fetch_kq(item + gridDim.x, cnext, tid);
#pragma unroll
    for (int s = 0; s < NSL; ++s) gc[s].prefix_finish(sTot);
#pragma unroll
    for (int s = 0; s < NSL; ++s)
      subchunk_stats_regs(gc[s], n, sMid, sGf, sGl, sGn, sFlag,
                          (MODE & PREP_BWD_CHUNK) ? reinterpret_cast<f32x4*>(ka().Gst) + cb * NSUB * K
                                                  : nullptr);
    lds_barrier();
    kargs.renew();

    // Element-wise phase of a column pair (PAIR): the thread's two slots are
    // columns c0 = gc[0].c (even) and c0 + 1 of the same 16 rows, so every
    // LDS access, conversion and 2-byte output store of the one-column phase
    // below becomes one access of a bf16 pair.  Same arithmetic, same outputs.
    auto elementwise_pairs = [&]() {
      if (!gc[0].on) return;
      int c0 = gc[0].c;
      asm volatile("" : "+v"(c0));
      __builtin_assume(c0 >= 0 && c0 < K);
      const int sg = gc[0].seg;
      const int r0 = __builtin_amdgcn_readfirstlane(sg * RS);
      const bool seg_live = r0 < n;
      float rA[2], rB[2], cA[2], cB[2], gn[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        gn[j] = sGn[c0 + j];
        rA[j] = seg_live ? ref_recv(sMid, sGf, sFlag, sg, K, c0 + j) : gn[j];
        rB[j] = seg_live ? ref_send(sMid, sGl, sFlag, sg, K, c0 + j) : gn[j];
        cA[j] = fexp2(rA[j]);
        cB[j] = fexp2(gn[j] - rB[j]);
      }
      const float bs = ka().scale;
      constexpr int KGF = 4 * VE, NGTF = CH / KGF, NGKF = K / KGF;
      constexpr int NKBQ = K / SUB, GPQ = 16 / (4 * (int)sizeof(T));
      T* Ftd = reinterpret_cast<T*>(ka().Ft) + cb * K * CH;
      T* Qgtd = reinterpret_cast<T*>(ka().Qgt) + cb * K * CH;
      // F and Qg (orders as in the one-column phase below) in whole 16-byte
      // pieces: the four 4-byte words of a piece row come from four lanes (F:
      // a lane quad; Qg: lanes L, L ^ 1, L ^ 8, L ^ 9), which exchange their
      // words for each group of four rows (xpose4_words), so that the lane of
      // role j stores the piece of row 4 i + j of group i
      const int tl = c0 >> 1;  // the lane: column pairs run along the wave
      const int frole = tl & 3, qrole = (tl & 1) + ((tl >> 2) & 2);
      T* Fp = reinterpret_cast<T*>(ka().F) + cb * CH * K + ((sg * NGKF + c0 / KGF) * 64 + ((c0 % KGF) / VE) * 16) * VE;
      T* Qgp = reinterpret_cast<T*>(ka().Qg) + cb * CH * K +
               (((int64_t)sg * (NKBQ / GPQ) + (c0 / SUB) / GPQ) * 64 + 16 * ((c0 % SUB) / 4)) * GPQ * 4;
      auto pk2 = [](float x, float y) { return __builtin_bit_cast(uint32_t, bf16x2{(bf16)x, (bf16)y}); };
#pragma unroll
      for (int r8 = 0; r8 < RS; r8 += VE) {
        union {
          uint4 u;
          T e[VE];
        } ft[2], qt[2], et[2];
        uint32_t qw[4], fw[4];  // words of the current group of four rows
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const int r = r8 + e, row = r0 + r;
          const uint32_t k2 = *reinterpret_cast<const uint32_t*>(sK + row * PK + c0);
          const uint32_t q2 = *reinterpret_cast<const uint32_t*>(sQ + row * PK + c0);
          const float kr[2] = {__uint_as_float(k2 << 16), __uint_as_float(k2 & 0xffff0000u)};
          const float qr[2] = {__uint_as_float(q2 << 16), __uint_as_float(q2 & 0xffff0000u)};
          float vKa[2], vQa[2], vKc[2], vQg[2], vF[2];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float G = gc[j].G[r];
            const float ea = fexp2(G - rA[j]), eb = fexp2(rB[j] - G);
            float bk;  // erase factor of this row (and feature)
            if constexpr (EW) bk = __uint_as_float(bwr[j][r] << 16);
            else bk = sBeta[row];
            vKa[j] = bk * kr[j] * ea;
            vQa[j] = bs * qr[j] * ea;
            vKc[j] = kr[j] * eb;
            vQg[j] = vQa[j] * cA[j];
            vF[j] = vKc[j] * cB[j];
            et[j].e[e] = fromf<T>(vKa[j] * cA[j]);
            ft[j].e[e] = fromf<T>(vF[j]);
            qt[j].e[e] = fromf<T>(vQg[j]);
          }
          qw[e & 3] = pk2(vQg[0], vQg[1]);
          fw[e & 3] = pk2(vF[0], vF[1]);
          *reinterpret_cast<uint32_t*>(sKa + row * PK + c0) = pk2(vKa[0], vKa[1]);
          *reinterpret_cast<uint32_t*>(sQ + row * PK + c0) = pk2(vQa[0], vQa[1]);
          *reinterpret_cast<uint32_t*>(sK + row * PK + c0) = pk2(vKc[0], vKc[1]);
          if ((e & 3) == 3) {  // group of rows r8 + e - 3 .. r8 + e complete
            const int rg = r8 + e - 3;
            if constexpr (MODE & PREP_FWD_OUT) {
              xpose4_words<8>(qw);
              *reinterpret_cast<uint4*>(Qgp + (rg + qrole) * GPQ * 4) = uint4{qw[0], qw[1], qw[2], qw[3]};
            }
            if constexpr (MODE & PREP_BWD_SCAN) {
              xpose4_words<2>(fw);
              *reinterpret_cast<uint4*>(Fp + (rg + frole) * VE) = uint4{fw[0], fw[1], fw[2], fw[3]};
            }
          }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = c0 + j;
          etr[j][r8 / VE] = et[j].u;  // E^T reaches LDS in S5
          const int tk = r0 + r8, q = tk / KGF, gq = (tk % KGF) / VE;
          if constexpr (MODE & PREP_FWD_SCAN)
            *reinterpret_cast<uint4*>(Ftd + (((col / SUB) * NGTF + q) * 64 + gq * 16 + col % SUB) * VE) = ft[j].u;
          if constexpr (MODE & PREP_BWD_SCAN)
            *reinterpret_cast<uint4*>(Qgtd + (((col / SUB) * NGTF + q) * 64 + gq * 16 + col % SUB) * VE) = qt[j].u;
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = c0 + j;
        if constexpr (MODE & PREP_BWD_CHUNK) {
          float* G2d = ka().gate == 1 && col == 0 ? ka().G2t + cb * CH + r0 : nullptr;
          if (G2d)
#pragma unroll
            for (int r4 = 0; r4 < RS; r4 += 4)
              *reinterpret_cast<f32x4*>(G2d + r4) = f32x4{gc[j].G[r4], gc[j].G[r4 + 1], gc[j].G[r4 + 2], gc[j].G[r4 + 3]};
        }
        if constexpr ((MODE & (PREP_FWD_SCAN | PREP_BWD_SCAN)) != 0)
          if (sg == 0) ka().glast[cb * K + col] = gn[j];
      }
    };

    // ---- S2: pair factors; element-wise outputs and centred operands --------
    // the prefix totals are dead: L starts from zeros (strict upper parts and
    // the blocks past the chunk's end are never written)
    for (int idx = tid; idx < CH * PL / 4; idx += NTH) reinterpret_cast<f32x4*>(sL)[idx] = zero4();
    pair_factors<K>(sMid, sGf, sGl, sFlag, sFac, n, tid, NTH);
    if constexpr (PAIR) elementwise_pairs();
#pragma unroll
    for (int s = 0; s < (PAIR ? 0 : NSL); ++s) {
      // one slot at a time: interleaving the slots' element-wise work would
      // double the registers it holds live
      __builtin_amdgcn_sched_barrier(0);
      GC& g = gc[s];
      if (!g.on) continue;
      // opaque per item: keeps the compiler from hoisting these addresses out of
      // the item loop (they would have to stay live, and spill, across items)
      int col = g.c;
      asm volatile("" : "+v"(col));
      __builtin_assume(col >= 0 && col < K);
      // the thread's 16 rows lie in sub-chunk seg, the same for the whole wave
      // when a wave spans one segment (K >= 64)
      const int r0 = K >= 64 ? __builtin_amdgcn_readfirstlane(g.seg * RS) : g.seg * RS;
      const float gn = sGn[col];
      // a segment wholly past the chunk's end has no statistics; its rows hold
      // G2 = gn exactly (the prefix adds zeros there), so gn as both references
      // makes both factors 1
      const bool seg_live = r0 < n;
      const float rA = seg_live ? ref_recv(sMid, sGf, sFlag, g.seg, K, col) : gn;
      const float rB = seg_live ? ref_send(sMid, sGl, sFlag, g.seg, K, col) : gn;
      // two exponentials per row: ea = exp2(G - rA), eb = exp2(rB - G); then
      // gamma = exp2(G) = ea exp2(rA) and exp2(gn - G) = eb exp2(gn - rB), with
      // exp2(rA) <= 1 and exp2(gn - rB) <= 1.  Values that flush to zero this
      // way are below 2^-62 and multiply O(1) terms.  Rows past the chunk's end
      // hold k = q = beta = 0 and come out as zeros.
      const float cA = fexp2(rA), cB = fexp2(gn - rB);
      const float bs = ka().scale;
      // F^T and Qg^T in operand-fragment order (see kernels.hpp): 16 k rows x
      // KG tokens per fragment, this thread's VE-token groups are single
      // 16-byte pieces
      constexpr int KGF = 4 * VE, NGTF = CH / KGF;
      T* Ftd = reinterpret_cast<T*>(ka().Ft) + cb * K * CH;
      T* Qgtd = reinterpret_cast<T*>(ka().Qgt) + cb * K * CH;
      // F and Qg in operand-fragment order (row block seg, key group
      // col / KGF): this thread's 16 rows are elements VE apart in one column
      // of pieces (rows past the chunk's end are zeros)
      constexpr int NGKF = K / KGF;
      T* Fd = reinterpret_cast<T*>(ka().F) + cb * CH * K +
              ((g.seg * NGKF + col / KGF) * 64 + ((col % KGF) / VE) * 16) * VE + col % VE;
      // Qg in the order of W (pieces of GPQ 16-key groups, kernels.hpp), so the
      // forward scan contracts it with the same S operand as W: this thread's
      // 16 rows are 4 GPQ elements apart
      constexpr int NKBQ = K / SUB, GPQ = 16 / (4 * (int)sizeof(T));
      T* Qgd = reinterpret_cast<T*>(ka().Qg) + cb * CH * K +
               ((((int64_t)g.seg * (NKBQ / GPQ) + (col / SUB) / GPQ) * 64 + 16 * ((col % SUB) / 4)) * GPQ +
                (col / SUB) % GPQ) * 4 + col % 4;
#pragma unroll
      for (int r8 = 0; r8 < RS; r8 += VE) {
        union {
          uint4 u;
          T e[VE];
        } ft, qt, et;
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const int r = r8 + e, row = r0 + r;
          const T kraw = sK[row * PK + col], qraw = sQ[row * PK + col];
          const float G = g.G[r];
          const float kr = tof(kraw), qr = tof(qraw);
          const float ea = fexp2(G - rA), eb = fexp2(rB - G);
          float bk = 0.f;  // erase factor of this row (and feature)
          if constexpr (EW) bk = sizeof(T) == 2 ? __uint_as_float(bwr[s][r] << 16) : __uint_as_float(bwr[s][r]);
          else bk = sBeta[row];
          const float vKa = bk * kr * ea, vQa = bs * qr * ea, vKc = kr * eb;
          const float vE = vKa * cA, vQg = vQa * cA, vF = vKc * cB;
          if constexpr (MODE & PREP_FWD_OUT) Qgd[r * GPQ * 4] = fromf<T>(vQg);
          if constexpr (MODE & PREP_BWD_SCAN) Fd[r * VE] = fromf<T>(vF);
          sKa[row * PK + col] = fromf<T>(vKa);
          sQ[row * PK + col] = fromf<T>(vQa);
          sK[row * PK + col] = fromf<T>(vKc);
          et.e[e] = fromf<T>(vE);
          ft.e[e] = fromf<T>(vF);
          qt.e[e] = fromf<T>(vQg);
        }
        etr[s][r8 / VE] = et.u;  // E^T reaches LDS in S5
        if constexpr (MODE & PREP_FWD_SCAN) {
          const int tk = r0 + r8, q = tk / KGF, gq = (tk % KGF) / VE;
          *reinterpret_cast<uint4*>(Ftd + (((col / SUB) * NGTF + q) * 64 + gq * 16 + col % SUB) * VE) = ft.u;
        }
        if constexpr (MODE & PREP_BWD_SCAN) {
          const int tk = r0 + r8, q = tk / KGF, gq = (tk % KGF) / VE;
          *reinterpret_cast<uint4*>(Qgtd + (((col / SUB) * NGTF + q) * 64 + gq * 16 + col % SUB) * VE) = qt.u;
        }
      }
      // the scalar gate's G2 row (rows past the end hold G2 of the last row);
      // the chunk backward rebuilds G2 of a vector gate from g (or x) and the
      // statistics
      if constexpr (MODE & PREP_BWD_CHUNK) {
        float* G2d = ka().gate == 1 && col == 0 ? ka().G2t + cb * CH + r0 : nullptr;
        if (G2d)
#pragma unroll
          for (int r4 = 0; r4 < RS; r4 += 4)
            *reinterpret_cast<f32x4*>(G2d + r4) = f32x4{g.G[r4], g.G[r4 + 1], g.G[r4 + 2], g.G[r4 + 3]};
      }
      if constexpr ((MODE & (PREP_FWD_SCAN | PREP_BWD_SCAN)) != 0)
        if (g.seg == 0) ka().glast[cb * K + col] = gn;
    }
    lds_barrier();
    kargs.renew();

    // ---- S3: score tiles L (strict, fp32 in LDS) and Cq (inclusive, global) --
    // the next item's gates: their registers are free since the elementwise
    // phase
    if constexpr (PAIR) fetch_g(item + gridDim.x, cnext);
    {
      T* Cqo = reinterpret_cast<T*>(ka().Cq) + cb * CH * CH;
      using FR = typename Frag4<T>::type;
      // identity as the B operand of a 16-long product: C = X^T I turns a C
      // tile (rows 4 (l >> 4) + e, column l & 15) into row l & 15, columns
      // 4 (l >> 4) .. + 3, exactly
      f32x4 idf;
#pragma unroll
      for (int e = 0; e < 4; ++e) idf[e] = (crow(e) == ccol()) ? 1.f : 0.f;
      const FR idt = to_frag<T>(idf);
      T* Cqto = reinterpret_cast<T*>(ka().Cqt) + cb * CH * CH;
      auto store = [&](int I, int J, const f32x4& accL, const f32x4& accC) {
        f32x4 cq;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = I * SUB + crow(i), col = J * SUB + ccol();
          if (row > col) sL[row * PL + col] = accL[i];
          cq[i] = row >= col ? accC[i] : 0.f;
        }
        if constexpr (MODE & PREP_FWD_OUT) {  // C fragments of the transposed blocks (exact transpose)
          f32x4 tr = zero4();
          mm16(tr, to_frag<T>(cq), idt);
          *reinterpret_cast<FR*>(Cqo + ((I * NSUB + J) * 64 + lane_id()) * 4) = to_frag<T>(tr);
        }
        if constexpr (MODE & PREP_BWD_SCAN) st_frag_T<T>(cq, Cqto, I, J);
      };
      score_tiles_pre<T, K, true, NW>(sKa, sQ, sK, PK, sFac, sFlag, n, store);
      // diagonal sub-chunks with a wide feature block, one wave each: the
      // centred blocks by MFMA (the wide ones masked by a zero pair factor),
      // then the wide blocks pairwise
      for (int J = w; J < NSUB; J += NW)
        if (J * SUB < n && flagged(sFlag, J, K / SUB)) {
          f32x4 accL = zero4(), accC = zero4();
          score_tile<T, K, true>(sKa, sQ, sK, PK, sFac + (J * (J + 1) / 2 + J) * K, J, J, true, accL, accC);
          pairwise_diag<T, K, true, EW, GIN>(ka(), t0, h, n, J, sBeta, sFlag + J * (K / SUB), accL, accC);
          store(J, J, accL, accC);
        }
      // tiles nobody computed: zeros (rows past the end; of the upper
      // triangle only what the scans read: the forward scan reads blocks
      // J <= I only, the reverse scan skips the 16-byte pieces of C_q^T whose
      // tokens i all lie before its rows j)
      constexpr int KGQ = 4 * (16 / (int)sizeof(T));  // tokens per piece of C_q^T
      for (int t = w; t < NSUB * NSUB; t += NW) {
        const int I = t / NSUB, J = t - I * NSUB;
        if (J <= I && I * SUB < n) continue;
        if constexpr (MODE & PREP_FWD_OUT)
          if (J <= I) *reinterpret_cast<FR*>(Cqo + ((I * NSUB + J) * 64 + lane_id()) * 4) = to_frag<T>(zero4());
        if constexpr (MODE & PREP_BWD_SCAN)
          if (KGQ * ((I * SUB) / KGQ + 1) > SUB * J) st_frag_T<T>(zero4(), Cqto, I, J);
      }
    }
    lds_barrier();
    kargs.renew();

    // ---- S4: A = (I + L)^-1 in fp32 ------------------------------------------
    if constexpr (!PAIR) {  // the one-column layouts: all fetches here, before the solve
      fetch_v(item, ci, tid);
      fetch_kq(item + gridDim.x, cnext, tid);
      fetch_g(item + gridDim.x, cnext);
    }

    // A takes X (the score operands are dead); its off-diagonal blocks start
    // at zero, written here while wave 0 forms the diagonal blocks
    for (int idx = tid; idx < NSUB * NSUB * SUB * 4; idx += NTH) {
      const int blk = idx / (SUB * 4), I = blk / NSUB, J = blk - I * NSUB;
      const int rem = idx - blk * SUB * 4, rr = rem >> 2, c4 = (rem & 3) * 4;
      if (I != J) *reinterpret_cast<f32x4*>(sA + (I * SUB + rr) * PL + J * SUB + c4) = zero4();
    }
    solve_unit_lower(sL, sA, PL, n);
    if constexpr (MODE & PREP_BWD_CHUNK) {  // A^T for the chunk backward, 16-byte rows
      constexpr int VA = 16 / (int)sizeof(T), PER = CH / VA;
      T* Ato = reinterpret_cast<T*>(ka().At) + cb * CH * CH;
      for (int idx = tid; idx < CH * PER; idx += NTH) {
        const int i = idx / PER, j0 = (idx - i * PER) * VA;
        union {
          uint4 u;
          T e[VA];
        } v;
#pragma unroll
        for (int e = 0; e < VA; ++e) v.e[e] = fromf<T>(sA[(j0 + e) * PL + i]);
        *reinterpret_cast<uint4*>(Ato + i * CH + j0) = v.u;
      }
    }

    // ---- S5: W = A E, U = A Z --------------------------------------------------
    if constexpr (BF) {  // A to the operand type, into Y (L is dead)
      for (int idx = tid; idx < CH * CH / 4; idx += NTH) {
        const int i = idx / (CH / 4), j = (idx - i * (CH / 4)) * 4;
        const f32x4 x = *reinterpret_cast<const f32x4*>(sA + i * PL + j);
        bf16x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (bf16)x[e];
        *reinterpret_cast<bf16x4*>(sAb + i * PA + j) = y;
      }
      lds_barrier();  // A in fp32 is dead: E^T and Z^T go over it
      kargs.renew();
    }
    // E^T from the registers of the elementwise phase
#pragma unroll
    for (int s = 0; s < NSL; ++s) {
      if (!gc[s].on) continue;
      const int col = gc[s].c, r0 = gc[s].seg * RS;
#pragma unroll
      for (int r8 = 0; r8 < RS; r8 += VE)
        *reinterpret_cast<uint4*>(sEt + col * PA + r0 + r8) = etr[s][r8 / VE];
    }
    // Z^T = (beta v)^T from the staged v
    if constexpr (BF) {
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int sl = tid + j * NTH, p = sl % 32, c0 = (sl / 32) * 8;
        if (sl >= VSL) continue;
        union {
          uint4 u;
          T e[8];
        } v0, v1;
        v0.u = pv2[2 * j];
        v1.u = pv2[2 * j + 1];
        union {
          uint4 u;
          T e[8];
        } w0, w1;  // write gate (erase/write form)
        if constexpr (EW) {
          w0.u = pw2[2 * j];
          w1.u = pw2[2 * j + 1];
        }
        const float b0 = EW ? 0.f : sBeta[2 * p], b1 = EW ? 0.f : sBeta[2 * p + 1];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          union {
            uint32_t u;
            T hh[2];
          } z;
          z.hh[0] = fromf<T>((EW ? tof(w0.e[e]) : b0) * tof(v0.e[e]));
          z.hh[1] = fromf<T>((EW ? tof(w1.e[e]) : b1) * tof(v1.e[e]));
          *reinterpret_cast<uint32_t*>(sZt + (c0 + e) * PA + 2 * p) = z.u;
        }
      }
    } else {
      constexpr int VEC = 4, PER = V / VEC;
#pragma unroll
      for (int j = 0; j < decltype(pv)::N; ++j) {
        const int idx = tid + j * NTH;
        const int r = idx / PER, c0 = (idx - r * PER) * VEC;
        if (idx < CH * PER) {
          union {
            uint4 u;
            T e[VEC];
          } val;
          val.u = pv.r[j];
          union {
            uint4 u;
            T e[VEC];
          } wv;
          if constexpr (EW) wv.u = pw.r[j];
          const float b = EW ? 0.f : sBeta[r];
#pragma unroll
          for (int e = 0; e < VEC; ++e)
            sZt[(c0 + e) * PA + r] = fromf<T>((EW ? tof(wv.e[e]) : b) * tof(val.e[e]));
        }
      }
    }
    lds_barrier();
    kargs.renew();
    if constexpr (PAIR) fetch_v(item + gridDim.x, cnext, tid);  // the staged v is in Z^T

    // W, U in operand-fragment order (see kernels.hpp), all 64 rows (rows past
    // the chunk's end are exact zeros).  Each tile of W^T is formed once: its C
    // fragments are the 16-long A fragments of W, the pieces of the forward
    // scan, and one product with the identity turns them exactly into the C
    // fragments of the W tile, from which W^T is stored for the reverse scan.
    T* Wfo = reinterpret_cast<T*>(ka().W) + cb * CH * K;
    T* Ufo = reinterpret_cast<T*>(ka().U) + cb * CH * V;
    T* Wto = reinterpret_cast<T*>(ka().Wt) + cb * K * CH;
    constexpr bool wantW = MODE & PREP_FWD_SCAN, wantWt = MODE & PREP_BWD_SCAN, wantU = wantW;
    const T* Aop = BF ? (const T*)sAb : (const T*)sA;
    constexpr int PAo = BF ? PA : PL;
    constexpr int NKB = K / SUB, GPP = 16 / (4 * (int)sizeof(T));  // 16-long groups per piece
    constexpr int NJW = (wantW || wantWt) ? NKB / GPP : 0, NJU = wantU ? V / SUB : 0;
    using FR = typename Frag4<T>::type;
    f32x4 idf;
#pragma unroll
    for (int e = 0; e < 4; ++e) idf[e] = (crow(e) == ccol()) ? 1.f : 0.f;
    const FR idt = to_frag<T>(idf);
    for (int job = w; job < NJW + NJU; job += NW) {
      if (job < NJW) {  // W, key blocks GPP job .. + GPP - 1, every token block
        static_for<0, NSUB>([&](auto II) {
          constexpr int I = decltype(II)::value;
          // A is lower triangular: token block I needs tokens < 16 (I + 1) only
          constexpr int kd = ((SUB * (I + 1) + MM<T>::KS - 1) / MM<T>::KS) * MM<T>::KS;
          union {
            uint4 u;
            FR f[GPP];
          } piece;
          static_for<0, GPP>([&](auto hh) {
            const int kb = job * GPP + hh;
            // C tile of W^T: lane l holds keys 16 kb + 4 (l >> 4) .. + 3 of
            // token 16 I + (l & 15)
            f32x4 acc = zero4();
            mma_tile<T, true, true>(acc, sEt + (kb * SUB) * PA, PA, 1, Aop + (I * SUB) * PAo, PAo, 1, kd);
            const FR wt = to_frag<T>(acc);
            if constexpr (wantW) piece.f[hh] = wt;
            if constexpr (wantWt) {
              f32x4 tr = zero4();
              mm16(tr, wt, idt);
              st_frag_T<T>(tr, Wto, I, kb);
            }
          });
          if constexpr (wantW)
            *reinterpret_cast<uint4*>(Wfo + ((I * (NKB / GPP) + job) * 64 + lane_id()) * GPP * 4) = piece.u;
        });
      } else {  // U, value block: the C tile is the fragment piece
        const int col = (job - NJW) * SUB;
        static_for<0, NSUB>([&](auto II) {
          constexpr int I = decltype(II)::value;
          f32x4 acc = zero4();
          constexpr int kd = ((SUB * (I + 1) + MM<T>::KS - 1) / MM<T>::KS) * MM<T>::KS;
          mma_tile<T, true, true>(acc, Aop + (I * SUB) * PAo, PAo, 1, sZt + col * PA, PA, 1, kd);
          *reinterpret_cast<FR*>(Ufo + (((col / SUB) * NSUB + I) * 64 + lane_id()) * 4) = to_frag<T>(acc);
        });
      }
    }
    lds_barrier();  // LDS is rewritten by the next item
    kargs.renew();
  }
}

template <typename T, int MODE>
static hipError_t prep_m(const Args& a, hipStream_t s) {
  const int items = a.nc_max * a.H;
  const dim3 grid(std::min(items, ((MODE & PREP_EW) ? 1 : 2) * persistent_grid()), 1), block(256);
  REWY_KV_SWITCH_X(k_fwd_prep, MODE)
}

// The three output sets in use: the forward (recompute policy), the forward
// that also saves the backward's operands, and the recomputation in the
// backward; each with a shared beta or in the erase/write form.
template <typename T>
static hipError_t prep_t(const Args& a, hipStream_t s) {
  constexpr int FWD = PREP_FWD_SCAN | PREP_FWD_OUT;
  constexpr int ALL = FWD | PREP_BWD_SCAN | PREP_BWD_CHUNK;
  constexpr int BWD = PREP_FWD_SCAN | PREP_BWD_SCAN | PREP_BWD_CHUNK;
  constexpr int E = PREP_EW, GI = PREP_GIN;
  switch (a.prep_mode | (a.ew ? E : 0) | (a.gin ? GI : 0)) {
    case FWD: return prep_m<T, FWD>(a, s);
    case ALL: return prep_m<T, ALL>(a, s);
    case BWD: return prep_m<T, BWD>(a, s);
    case FWD | E: return prep_m<T, FWD | E>(a, s);
    case ALL | E: return prep_m<T, ALL | E>(a, s);
    case BWD | E: return prep_m<T, BWD | E>(a, s);
    case FWD | GI: return prep_m<T, FWD | GI>(a, s);
    case ALL | GI: return prep_m<T, ALL | GI>(a, s);
    case BWD | GI: return prep_m<T, BWD | GI>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_prep(const Args& a, int f32, hipStream_t s) {
  return f32 ? prep_t<float>(a, s) : prep_t<bf16>(a, s);
}

}  // namespace rewy
