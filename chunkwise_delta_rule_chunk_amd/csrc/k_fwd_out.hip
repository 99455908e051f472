// Chunk-parallel output (ReWY paper, "The chunk system": O = Qg S + Cq R;
// KDA blog section 6.5: read the decayed incoming state, then add the causal
// in-chunk writes).  One workgroup per (chunk, head).
#include "chunk_common.hpp"

namespace rewy {

template <typename T, int K, int V>
__global__ __launch_bounds__(256) void k_fwd_out(Args a) {
  constexpr int PK = pitch<T>(K), PA = pitch<T>(CH);
  constexpr int VE = 16 / (int)sizeof(T), KG = 4 * VE, NGK = K / KG, NGT = CH / KG;
  constexpr int NVB = V / SUB, VPW = (NVB + 3) / 4;  // value blocks, per wave
  __shared__ __align__(16) T sQg[CH * PK];
  __shared__ __align__(16) T sCq[CH * PA];

  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const ChunkInfo ci = load_chunk(a.chunks, c);
  const int len = ci.len;
  if (len == 0) return;
  const int H = a.H, w = wave_id(), l = lane_id();
  const int64_t t0 = ci.bos, cb = (int64_t)c * H + h;
  const int64_t gsK = (int64_t)H * K, gsV = (int64_t)H * V;
  // Qg and Cq are shared by the waves and go through LDS (Qg rows past the
  // chunk's end read as zero); the state S_c and R_c were written by the
  // forward scan in operand-fragment order, and each wave reads the pieces of
  // its own value blocks straight into registers.
  TileRegs<T, CH, K, 256> pq;
  TileRegs<T, CH, CH, 256> pc;
  pq.load(gbuf(reinterpret_cast<const T*>(a.Qg) + (t0 * H + h) * K, tile_bytes<T>(len, gsK, K)), gsK, tid);
  pc.load_cb(gbuf(reinterpret_cast<const T*>(a.Cq) + cb * CH * CH, CH * CH * sizeof(T)), CH, 0, tid);
  uint4 sf[VPW][NGK], rf[VPW][NGT];
  static_for<0, VPW>([&](auto jj) {
    constexpr int j = decltype(jj)::value;
    const int vb = min(w + 4 * j, NVB - 1);  // a wave without a block reads one again, unused
    const T* sp = reinterpret_cast<const T*>(a.hbufT) + ((cb * NVB + vb) * NGK * 64 + l) * VE;
    const T* rp = reinterpret_cast<const T*>(a.RT) + ((cb * NVB + vb) * NGT * 64 + l) * VE;
#pragma unroll
    for (int q = 0; q < NGK; ++q) sf[j][q] = *reinterpret_cast<const uint4*>(sp + q * 64 * VE);
#pragma unroll
    for (int q = 0; q < NGT; ++q) rf[j][q] = *reinterpret_cast<const uint4*>(rp + q * 64 * VE);
  });
  pq.store(sQg, PK, tid);
  pc.store_cb(sCq, PA, tid);
  lds_barrier();
  // o through a bounds-checked buffer (rows past the chunk's end are dropped)
  const GBuf bo = gbuf(reinterpret_cast<T*>(a.o) + (t0 * H + h) * V, tile_bytes<T>(len, gsV, V));
  const int r16 = l & 15, g = l >> 4;
  using FR = typename Frag4<T>::type;
  // identity as the B operand of a 16-long product: C = X^T I turns the C
  // tile (rows 4 g + e, column r16) into row r16, columns 4 g .. + 3, exactly
  f32x4 idf;
#pragma unroll
  for (int e = 0; e < 4; ++e) idf[e] = (4 * g + e == r16) ? 1.f : 0.f;
  const FR idt = to_frag<T>(idf);
  static_for<0, VPW>([&](auto jj) {
    constexpr int j = decltype(jj)::value;
    const int vb = w + 4 * j;
    if (vb >= NVB) return;
    static_for<0, NSUB>([&](auto II) {
      constexpr int I = decltype(II)::value;
      if (I * SUB >= len) return;
      f32x4 acc = zero4();
      const T* qa = sQg + (I * SUB + r16) * PK + VE * g;
#pragma unroll
      for (int q = 0; q < NGK; ++q) mma16B<T>(acc, *reinterpret_cast<const uint4*>(qa + KG * q), sf[j][q]);
      // Cq is lower triangular: row block I needs tokens < 16 (I + 1) only
      constexpr int nq = (SUB * (I + 1) + KG - 1) / KG;
      const T* ca = sCq + (I * SUB + r16) * PA + VE * g;
#pragma unroll
      for (int q = 0; q < nq; ++q) mma16B<T>(acc, *reinterpret_cast<const uint4*>(ca + KG * q), rf[j][q]);
      f32x4 tr = zero4();
      mm16(tr, to_frag<T>(acc), idt);
      const uint32_t off = (uint32_t)(((int64_t)(I * SUB + r16) * gsV + vb * SUB + 4 * g) * (int64_t)sizeof(T));
      if constexpr (std::is_same_v<T, bf16>) gst8(bo, off, __builtin_bit_cast(uint2, to_frag<T>(tr)));
      else gst16(bo, off, __builtin_bit_cast(uint4, tr));
    });
  });
}

template <typename T>
static hipError_t out_t(const Args& a, hipStream_t s) {
  const dim3 grid(a.nc_max, a.H), block(256);
  REWY_KV_SWITCH(k_fwd_out)
}

hipError_t launch_fwd_out(const Args& a, int f32, hipStream_t s) {
  return f32 ? out_t<float>(a, s) : out_t<bf16>(a, s);
}

}  // namespace rewy
