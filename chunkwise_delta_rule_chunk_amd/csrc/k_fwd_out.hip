// Chunk-parallel output (ReWY paper, "The chunk system": O = Qg S + Cq R;
// KDA blog section 6.5: read the decayed incoming state, then add the causal
// in-chunk writes).  One workgroup per (chunk, head).
#include "chunk_common.hpp"

namespace rewy {

template <typename T, int K, int V>
__global__ __launch_bounds__(256) void k_fwd_out(Args a) {
  constexpr int PK = pitch<T>(K), PA = pitch<T>(CH);
  __shared__ __align__(16) T sQg[CH * PK];
  __shared__ __align__(16) T sHt[V * PK];  // state S_c as operand, [v][k]
  __shared__ __align__(16) T sCq[CH * PA];
  __shared__ __align__(16) T sRt[V * PA];  // R as operand, [v][i]

  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const ChunkInfo ci = load_chunk(a.chunks, c);
  const int len = ci.len;
  if (len == 0) return;
  const int H = a.H;
  const int64_t t0 = ci.bos, cb = (int64_t)c * H + h;
  const int64_t gsK = (int64_t)H * K, gsV = (int64_t)H * V;
  // all four tiles are read before the first LDS write waits; Qg rows past
  // the chunk's end read as zero.  S_c^T and R^T were written transposed by
  // the forward scan.
  TileRegs<T, CH, K, 256> pq;
  TileRegs<T, V, K, 256> ph;
  TileRegs<T, CH, CH, 256> pc;
  TileRegs<T, V, CH, 256> pr;
  pq.load(gbuf(reinterpret_cast<const T*>(a.Qg) + (t0 * H + h) * K, tile_bytes<T>(len, gsK, K)), gsK, tid);
  ph.load(gbuf(reinterpret_cast<const T*>(a.hbufT) + cb * V * K, V * K * sizeof(T)), K, tid);
  pc.load(gbuf(reinterpret_cast<const T*>(a.Cq) + cb * CH * CH, CH * CH * sizeof(T)), CH, tid);
  pr.load(gbuf(reinterpret_cast<const T*>(a.RT) + cb * V * CH, V * CH * sizeof(T)), CH, tid);
  pq.store(sQg, PK, tid);
  ph.store(sHt, PK, tid);
  pc.store(sCq, PA, tid);
  pr.store(sRt, PA, tid);
  lds_barrier();
  T* og = reinterpret_cast<T*>(a.o) + (t0 * H + h) * V;
  const int w = wave_id();
  for (int vb = w; vb < V / SUB; vb += 4) {
    static_for<0, NSUB>([&](auto II) {
      constexpr int I = decltype(II)::value;
      if (I * SUB >= len) return;
      f32x4 acc = zero4();
      mma_tile<T, true, true>(acc, sQg + I * SUB * PK, PK, 1, sHt + vb * SUB * PK, PK, 1, K);
      // Cq is lower triangular: row block I needs tokens < 16 (I + 1) only
      constexpr int kd = ((SUB * (I + 1) + MM<T>::KS - 1) / MM<T>::KS) * MM<T>::KS;
      mma_tile<T, true, true>(acc, sCq + I * SUB * PA, PA, 1, sRt + vb * SUB * PA, PA, 1, kd);
      st_tile<T>(acc, og + (I * SUB) * gsV + vb * SUB, (int)gsV, 1, len - I * SUB);
    });
  }
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
