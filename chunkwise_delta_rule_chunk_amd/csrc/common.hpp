// Device-side building blocks shared by the gfx950 kernels of the chunkwise
// gated delta rule: element types, MFMA fragment loads, LDS tile movers and
// the per-chunk index record.
//
// MFMA tiles are 16x16.  bf16 operands use v_mfma_f32_16x16x32_bf16 (32-long
// contraction per instruction); fp32 operands use v_mfma_f32_16x16x4_f32.
// For both, lane l of a wave holds row (l & 15) of an A fragment / column
// (l & 15) of a B fragment, and contraction slots
//   bf16: k0 + 8*(l >> 4) + e, e = 0..7        fp32: k0 + (l >> 4)
// The result lives as acc[i] = C[4*(l >> 4) + i][l & 15], i = 0..3.
// A and B fragments use the same slot convention, so any consistent slot
// assignment gives the exact product.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rewy {

using bf16 = __bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;          // chunk length (tokens)
constexpr int SUB = 16;         // sub-chunk = MFMA tile edge
constexpr int NSUB = CH / SUB;  // sub-chunks per chunk
constexpr float LOG2E = 1.4426950408889634f;
// Largest in-block gate range (log2 units) for which midpoint-centred factors
// exp2(+-(G - mid)) stay inside 2^64; wider diagonal blocks take the pairwise path.
constexpr float CENTRE_MAX_RANGE = 128.f;

// One chunk of one sequence: tokens [bos, bos + len) of the packed token axis.
struct ChunkInfo {
  int seq;  // sequence index
  int bos;  // first token (row of the [B*T] token axis)
  int len;  // valid tokens, 0 for an unused slot
  int pos;  // chunk index within its sequence
};

// Lane and wave index.  A translation unit whose kernels loop over many work
// items in one workgroup defines REWY_OPAQUE_IDS before its first include: the
// indices are then opaque at every use, so the compiler cannot hoist address
// arithmetic derived from them out of the item loop (hoisted values stay live
// across items and spill).  Elsewhere they are plain, so the usual common
// subexpressions are shared.
#ifdef REWY_OPAQUE_IDS
__device__ __forceinline__ int lane_id() {
  int l = threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  return l;
}
__device__ __forceinline__ int wave_id() {
  int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  asm volatile("" : "+s"(w));
  return w;
}
#else
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
#endif
// Thread index made opaque to the optimiser.  Persistent item loops take it
// once per item: otherwise the compiler hoists address arithmetic derived from
// it out of the loop, and the hoisted values stay live (and spill) across items.
template <int NTH>
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  // still a thread of an NTH-thread workgroup: index checks that hold for
  // every thread (whole tiles) fold away
  __builtin_assume(t >= 0 && t < NTH);
  return t;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations
// and meets the other waves, but leaves global loads and stores in flight (a
// full __syncthreads() fence also drains them, which would stall every barrier
// on outstanding prefetches and output stores).  Global memory is never used
// to communicate between the threads of one workgroup in these kernels.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 2^x with the hardware instruction (v_exp_f32): about 1 ulp, results below
// the normal range flush to zero.  Every use is a gate factor or decay whose
// values that small are negligible against the terms they scale.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float LN2 = 0.6931471805599453f;
// softplus(z) = log(1 + exp(z)) = max(z, 0) + log(1 + exp(-|z|)), by the
// hardware exp2 and log2 (no overflow for large |z|; below z ~ -17 the
// result is 0 where the exact value is below 4e-8)
__device__ __forceinline__ float softplus(float z) {
  return fmaxf(z, 0.f) + LN2 * __builtin_amdgcn_logf(1.f + fexp2(-fabsf(z) * LOG2E));
}
// softplus(z) and its derivative, the logistic sigmoid 1 / (1 + exp(-z)),
// from one exponential e = exp(-|z|): sigmoid = (z >= 0 ? 1 : e) / (1 + e)
__device__ __forceinline__ void softplus_sigmoid(float z, float& sp, float& sg) {
  const float e = fexp2(-fabsf(z) * LOG2E);
  sp = fmaxf(z, 0.f) + LN2 * __builtin_amdgcn_logf(1.f + e);
  sg = (z >= 0.f ? 1.f : e) * __builtin_amdgcn_rcpf(1.f + e);
}

// logistic sigmoid 1 / (1 + exp(-u)): 0 and 1 in the limits (the reciprocal
// of infinity is zero)
__device__ __forceinline__ float sigmoid_f(float u) {
  return __builtin_amdgcn_rcpf(1.f + fexp2(-u * LOG2E));
}

// Sums across the wave's four 16-lane rows (the same lane of each row), by
// the row swaps of gfx950 (VALU, no LDS).  v_permlane16_swap on two copies of
// x returns, in every lane, x of the even and of the odd row of its row pair
// (0, 1) or (2, 3); v_permlane32_swap returns x of rows (0 or 1) and (2 or
// 3) with the lane's own parity.
// x summed over the four rows
__device__ __forceinline__ float rows_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float p = __uint_as_float(r[0]) + __uint_as_float(r[1]);  // pair sum
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
// x summed over the rows q >= q4 (the lane's own row q4 and the later ones)
__device__ __forceinline__ float rows_suffix_sum(float x, int q4) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float p = __uint_as_float(r[0]) + __uint_as_float(r[1]);  // pair sum
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
  return ((q4 & 1) ? x : p) + (q4 < 2 ? __uint_as_float(s[1]) : 0.f);
}
// x summed over the rows q < q4 (zero in row 0)
__device__ __forceinline__ float rows_prefix_excl(float x, int q4) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float p = __uint_as_float(r[0]) + __uint_as_float(r[1]);  // pair sum
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
  return ((q4 & 1) ? __uint_as_float(r[0]) : 0.f) + (q4 >= 2 ? __uint_as_float(s[0]) : 0.f);
}

// Sum over the 16 lanes of each row of the wave (lanes 16 r .. 16 r + 15),
// returned to every lane of the row, by DPP lane moves: the two quad
// permutations [1,0,3,2] and [2,3,0,1], then the half-row mirror (lane i of
// 8 reads lane 7 - i, in the other quad) and the row mirror (lane i reads
// 15 - i, in the other half).  Each step pairs lanes whose partial sums cover
// disjoint lanes, and runs on the VALU (no LDS traffic, no wait).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

// 4 x 4 exchange of 4-byte words among the lanes L, L ^ 1, L ^ M and
// L ^ M ^ 1 (M = 2 or 8: one 16-lane row).  The lane of role
// j = (L & 1) + 2 [L & M] enters with w[k], its word for item k, and leaves
// with w[k] = the item-j word of the lane of role k.  Two butterfly stages of
// DPP lane moves (partner L ^ 1, then L ^ M); no LDS.
template <int M>
__device__ __forceinline__ void xpose4_words(uint32_t (&w)[4]) {
  static_assert(M == 2 || M == 8, "partner lanes within a 16-lane row");
  constexpr int C2 = M == 2 ? 0x4E : 0x128;  // quad_perm [2,3,0,1] / row_ror:8
  const int l = lane_id();
  const bool p1 = l & 1, p2 = l & M;
#pragma unroll
  for (int k0 = 0; k0 < 4; k0 += 2) {  // items k0, k0 + 1 with the partner L ^ 1
    const uint32_t x = p1 ? w[k0] : w[k0 + 1];
    const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);
    if (p1) w[k0] = y;
    else w[k0 + 1] = y;
  }
#pragma unroll
  for (int k0 = 0; k0 < 2; ++k0) {  // items k0, k0 + 2 with the partner L ^ M
    const uint32_t x = p2 ? w[k0] : w[k0 + 2];
    const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, C2, 0xF, 0xF, false);
    if (p2) w[k0] = y;
    else w[k0 + 2] = y;
  }
}

template <typename T>
__device__ __forceinline__ float tof(T x) { return (float)x; }
template <typename T>
__device__ __forceinline__ T fromf(float x) { return (T)x; }

template <typename T>
struct MM;
template <>
struct MM<bf16> {
  static constexpr int KS = 32;
  using frag = bf16x8;
};
template <>
struct MM<float> {
  static constexpr int KS = 4;
  using frag = float;
};

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Operand fragment of a k-step starting at k0.  Element (r, k) of the operand
// is p[r * rs + k * ks] with r = lane & 15 (row of A / column of B).  KC means
// ks == 1 and rows are 16-byte aligned, so one vector read serves the lane.
template <typename T, bool KC>
__device__ __forceinline__ typename MM<T>::frag ldfrag(const T* p, int rs, int ks, int k0) {
  const int l = lane_id();
  const int r = l & 15, g = l >> 4;
  if constexpr (std::is_same_v<T, bf16>) {
    const int kb = k0 + g * 8;
    if constexpr (KC) {
      return *reinterpret_cast<const bf16x8*>(p + r * rs + kb);
    } else {
      bf16x8 f;
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = p[r * rs + (kb + e) * ks];
      return f;
    }
  } else {
    return p[r * rs + (k0 + g) * ks];
  }
}

// acc += A[16 x kd] * B[kd x 16]; A(m,k) = a[m*a_rs + k*a_ks], B(k,n) = b[n*b_rs + k*b_ks].
template <typename T, bool AKC, bool BKC>
__device__ __forceinline__ void mma_tile(f32x4& acc, const T* a, int a_rs, int a_ks, const T* b,
                                         int b_rs, int b_ks, int kd) {
  for (int k0 = 0; k0 < kd; k0 += MM<T>::KS)
    acc = mma(ldfrag<T, AKC>(a, a_rs, a_ks, k0), ldfrag<T, BKC>(b, b_rs, b_ks, k0), acc);
}

// acc += A[16 x 16] * B[16 x 16] (a 16-long contraction, e.g. one sub-chunk of
// tokens).  bf16 uses v_mfma_f32_16x16x16_bf16 with slots 4*(l >> 4) + e.
template <typename T, bool AKC, bool BKC>
__device__ __forceinline__ void mma_k16(f32x4& acc, const T* a, int a_rs, int a_ks, const T* b,
                                        int b_rs, int b_ks) {
  if constexpr (std::is_same_v<T, bf16>) {
    const int l = lane_id();
    const int r = l & 15, kb = (l >> 4) * 4;
    bf16x4 fa, fb;
    if constexpr (AKC) {
      fa = *reinterpret_cast<const bf16x4*>(a + r * a_rs + kb);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) fa[e] = a[r * a_rs + (kb + e) * a_ks];
    }
    if constexpr (BKC) {
      fb = *reinterpret_cast<const bf16x4*>(b + r * b_rs + kb);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) fb[e] = b[r * b_rs + (kb + e) * b_ks];
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(fa, fb, acc, 0, 0, 0);
  } else {
    mma_tile<float, false, false>(acc, a, a_rs, a_ks, b, b_rs, b_ks, 16);
  }
}

// Row/column of the C fragment held by this lane.
__device__ __forceinline__ int crow(int i) { return ((lane_id() >> 4) << 2) + i; }
__device__ __forceinline__ int ccol() { return lane_id() & 15; }

// Store a C tile: dst(m, n) = dst[m * rs + n * cs], rows m < mmax only.
template <typename U>
__device__ __forceinline__ void st_tile(const f32x4& acc, U* dst, int rs, int cs, int mmax = 16) {
  const int n = ccol();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = crow(i);
    if (m < mmax) dst[m * rs + n * cs] = fromf<U>(acc[i]);
  }
}

// Store a C tile transposed: dst[n * rs + m] for m = 4*(l>>4) .. +3 as one vector.
template <typename U>
__device__ __forceinline__ void st_tile_T(const f32x4& acc, U* dst, int rs) {
  const int n = ccol(), m0 = crow(0);
  if constexpr (std::is_same_v<U, bf16>) {
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (bf16)acc[i];
    *reinterpret_cast<bf16x4*>(dst + n * rs + m0) = v;
  } else {
    *reinterpret_cast<f32x4*>(dst + n * rs + m0) = acc;
  }
}

// Copy rows [0, nvalid) of a [nrows x C] tile from global (row stride gs
// elements) into LDS (row stride ls), zero-filling rows [nvalid, nrows).
// 16-byte vectors; C * sizeof(T) must be a multiple of 16, as must gs and ls.
template <typename T, int C>
__device__ __forceinline__ void g2s(T* s, int ls, const T* g, int64_t gs, int nvalid, int nrows,
                                    int tid, int nthr) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int PER = C / VEC;
  for (int idx = tid; idx < nrows * PER; idx += nthr) {
    const int r = idx / PER, c = (idx - r * PER) * VEC;
    uint4 val = {0u, 0u, 0u, 0u};
    if (r < nvalid) val = *reinterpret_cast<const uint4*>(g + (int64_t)r * gs + c);
    *reinterpret_cast<uint4*>(s + r * ls + c) = val;
  }
}

// Transposing copy: s[c * ls + r] = g[r * gs + c] for rows r < nvalid, zero for
// r in [nvalid, nrows).
template <typename T, int C>
__device__ __forceinline__ void g2s_T(T* s, int ls, const T* g, int64_t gs, int nvalid, int nrows,
                                      int tid, int nthr) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int PER = C / VEC;
  for (int idx = tid; idx < nrows * PER; idx += nthr) {
    const int r = idx / PER, c = (idx - r * PER) * VEC;
    union {
      uint4 u;
      T e[VEC];
    } val;
    val.u = uint4{0u, 0u, 0u, 0u};
    if (r < nvalid) val.u = *reinterpret_cast<const uint4*>(g + (int64_t)r * gs + c);
#pragma unroll
    for (int e = 0; e < VEC; ++e) s[(c + e) * ls + r] = val.e[e];
  }
}

// Copy rows [0, nvalid) of an LDS tile back to global with 16-byte vectors.
template <typename T, int C>
__device__ __forceinline__ void s2g(T* g, int64_t gs, const T* s, int ls, int nvalid, int tid,
                                    int nthr) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int PER = C / VEC;
  for (int idx = tid; idx < nvalid * PER; idx += nthr) {
    const int r = idx / PER, c = (idx - r * PER) * VEC;
    *reinterpret_cast<uint4*>(g + (int64_t)r * gs + c) =
        *reinterpret_cast<const uint4*>(s + r * ls + c);
  }
}

// Register staging of a [ROWS x COLS] tile for software prefetch: load() issues
// the global reads (rows >= nvalid read as zero), store() writes the tile into
// LDS later, so the load latency overlaps whatever runs in between.
template <typename T, int ROWS, int COLS, int NTH>
struct Staged {
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int PER = COLS / VEC;
  static constexpr int TOTAL = ROWS * PER;
  static constexpr int N = (TOTAL + NTH - 1) / NTH;
  static_assert(COLS % VEC == 0, "row length must be a multiple of 16 bytes");
  uint4 r[N];
  __device__ __forceinline__ void load(const T* g, int64_t gs, int nvalid, int tid) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int idx = tid + j * NTH;
      const int row = idx / PER, c = (idx - row * PER) * VEC;
      r[j] = uint4{0u, 0u, 0u, 0u};
      if (idx < TOTAL && row < nvalid) r[j] = *reinterpret_cast<const uint4*>(g + (int64_t)row * gs + c);
    }
  }
  __device__ __forceinline__ void store(T* s, int ls, int tid) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int idx = tid + j * NTH;
      const int row = idx / PER, c = (idx - row * PER) * VEC;
      if (idx < TOTAL) *reinterpret_cast<uint4*>(s + row * ls + c) = r[j];
    }
  }
  // transposed store: s[c * ls + row] = tile[row][c]
  __device__ __forceinline__ void store_T(T* s, int ls, int tid) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int idx = tid + j * NTH;
      const int row = idx / PER, c = (idx - row * PER) * VEC;
      if (idx < TOTAL) {
        union {
          uint4 u;
          T e[VEC];
        } v;
        v.u = r[j];
#pragma unroll
        for (int e = 0; e < VEC; ++e) s[(c + e) * ls + row] = v.e[e];
      }
    }
  }
};

// The chunk record c read through the scalar data cache (c uniform over the
// wave).  Records are written by an earlier kernel, and the scalar cache is
// invalidated at every dispatch.  A scalar load is counted apart from the
// vector memory counter, so waiting for it does not also wait for every
// global load and store the wave still has in flight, as waiting for a
// vector load of the record would.
__device__ __forceinline__ ChunkInfo load_chunk(const ChunkInfo* p, int c) {
  static_assert(sizeof(ChunkInfo) == 4 * sizeof(int), "record layout");
  const auto* q = (const __attribute__((address_space(4))) int*)p + 4 * c;
  ChunkInfo r;
  r.seq = q[0];
  r.bos = q[1];
  r.len = q[2];
  r.pos = q[3];
  return r;
}

// A view of the kernel's arguments in the kernarg segment (the kernel's only
// argument is the Args record at its start).  Reading a field through it is a
// scalar load that hits the scalar cache.  After renew(), the compiler can no
// longer reuse values loaded or addresses derived before it, so they need not
// stay in scalar registers across a long kernel: a persistent kernel whose
// argument pointers and per-item addresses all stayed live spilled them to
// vector-register lanes and reloaded them one lane read at a time.
struct KernArgs {
  const __attribute__((address_space(4))) char* p;
  __device__ __forceinline__ KernArgs() : p((const __attribute__((address_space(4))) char*)__builtin_amdgcn_kernarg_segment_ptr()) {}
  template <typename A>
  __device__ __forceinline__ const A& get() const { return *(const A*)(const char*)p; }
  __device__ __forceinline__ void renew() { asm volatile("" : "+s"(p)); }
};

// ---- operand-fragment order ---------------------------------------------------
// A tile with 64-long rows stored so that the MFMA operand fragments of a row
// block are contiguous: with VE = 16 / sizeof(T) and KG = 4 VE, piece
// ((rb * 64/KG + q) * 64 + l) holds row 16 rb + (l & 15), columns
// KG q + VE (l >> 4) + e, e < VE (one 16-byte load per lane per fragment).
// Store of the transposed C tile of a 16 x 16 product X (rows 16 I + 4 (l >> 4)
// + i, column 16 J + (l & 15) of X) into such a tile of X^T: row 16 J + (l & 15),
// columns 16 I + 4 (l >> 4) .. + 3, four consecutive elements of one piece.
template <typename T>
__device__ __forceinline__ void st_frag_T(const f32x4& acc, T* tile, int I, int J) {
  constexpr int VE = 16 / (int)sizeof(T), KG = 4 * VE, NG = CH / KG;
  const int l = lane_id(), c0 = SUB * I + 4 * (l >> 4);
  T* p = tile + ((J * NG + c0 / KG) * 64 + ((c0 % KG) / VE) * 16 + (l & 15)) * VE + c0 % VE;
  if constexpr (std::is_same_v<T, bf16>) {
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (bf16)acc[i];
    *reinterpret_cast<bf16x4*>(p) = v;
  } else {
    *reinterpret_cast<f32x4*>(p) = acc;
  }
}

// acc += A B over one 16-byte lane group: lane l supplies 16 bytes of row
// (l & 15) of A and of column (l & 15) of B, at contraction slots
// VE (l >> 4) + e of the group (VE = 16 / sizeof(T)).  bf16: one 16x16x32
// MFMA; fp32: four 16x16x4 MFMAs, step e taking element e of every lane.
template <typename T>
__device__ __forceinline__ void mma16B(f32x4& acc, uint4 a, uint4 b) {
  if constexpr (std::is_same_v<T, bf16>) {
    union {
      uint4 u;
      bf16x8 v;
    } x, y;
    x.u = a;
    y.u = b;
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.v, y.v, acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
}

// C-fragment order: a matrix stored as the C fragments of its 16 x 16 blocks,
// block (rb, cb) at piece (rb * ncb + cb) * 64 + l, four elements per lane,
// M[16 rb + 4 (l >> 4) + i][16 cb + (l & 15)] for i < 4.  That piece is the
// 16-long B fragment of M (and A fragment of M^T) for a contraction over M's
// row index.  The operand of one lane group of a contraction over rows
// 32 q .. 32 q + 31 joins blocks 2 q and 2 q + 1 (bf16: slot 8 (l >> 4) + e
// is row 32 q + 4 (l >> 4) + e, slot 8 (l >> 4) + 4 + e is row
// 32 q + 16 + 4 (l >> 4) + e; fp32 takes rows 16 q .. 16 q + 15 from block q);
// perm_row() reads the other operand's row with the same slot assignment.
// row points at element 4 (l >> 4) of the row (LDS)
template <typename T>
__device__ __forceinline__ uint4 perm_row(const T* row, int q) {
  if constexpr (std::is_same_v<T, bf16>) {
    const uint2 x0 = *reinterpret_cast<const uint2*>(row + 32 * q);
    const uint2 x1 = *reinterpret_cast<const uint2*>(row + 32 * q + 16);
    return uint4{x0.x, x0.y, x1.x, x1.y};
  } else {
    return *reinterpret_cast<const uint4*>(row + 16 * q);
  }
}

// ---- bounds-checked global access ------------------------------------------
// A buffer resource over [base, base + bytes): the hardware range check makes
// an access at an offset >= bytes read zeros and drops a store there, so an
// access guarded per lane (rows past a chunk's end) is one unconditional
// instruction.  Unconditional memory instructions keep the compiler's count
// of outstanding vector memory operations exact, so a use waits for its own
// load only and not for every load and store still in flight.
constexpr uint32_t OOB = 0x80000000u;  // an offset beyond every range used here
struct GBuf {
  __amdgpu_buffer_rsrc_t r;
};
__device__ __forceinline__ GBuf gbuf(const void* base, uint32_t bytes) {
  // 0x00020000: raw (unswizzled, unformatted) 32-bit-element buffer on gfx9
  return GBuf{__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000)};
}
// Bytes spanned by nrows rows (stride rs elements) whose first cols elements
// are in range.
template <typename T>
__device__ __forceinline__ uint32_t tile_bytes(int nrows, int64_t rs, int cols) {
  return nrows <= 0 ? 0u : (uint32_t)(((int64_t)(nrows - 1) * rs + cols) * (int64_t)sizeof(T));
}
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 gld16(const GBuf& b, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(b.r, off, 0, 0);
  return uint4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ uint2 gld8(const GBuf& b, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(b.r, off, 0, 0);
  return uint2{v[0], v[1]};
}
__device__ __forceinline__ uint32_t gld4(const GBuf& b, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(b.r, off, 0, 0);
}
__device__ __forceinline__ uint32_t gld2(const GBuf& b, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(b.r, off, 0, 0);
}
__device__ __forceinline__ void gst16(const GBuf& b, uint32_t off, uint4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, x.w}, b.r, off, 0, 0);
}
__device__ __forceinline__ void gst8(const GBuf& b, uint32_t off, uint2 x) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{x.x, x.y}, b.r, off, 0, 0);
}
__device__ __forceinline__ void gst4(const GBuf& b, uint32_t off, uint32_t x) {
  __builtin_amdgcn_raw_buffer_store_b32(x, b.r, off, 0, 0);
}
__device__ __forceinline__ void gst2(const GBuf& b, uint32_t off, uint32_t x) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)x, b.r, off, 0, 0);
}

// A [ROWS x COLS] tile read into registers with one unconditional 16-byte load
// per piece (rows out of the buffer's range read as zero), then written to
// LDS: every load of the tile is issued before the first LDS write waits.
template <typename T, int ROWS, int COLS, int NTH>
struct TileRegs {
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int PER = COLS / VEC;
  static constexpr int TOTAL = ROWS * PER;
  static constexpr int N = (TOTAL + NTH - 1) / NTH;
  static_assert(COLS % VEC == 0, "row length must be a multiple of 16 bytes");
  uint4 r[N];
  // tile rows at stride gs elements from the buffer's base
  __device__ __forceinline__ void load(const GBuf& b, int64_t gs, int tid) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int idx = tid + j * NTH;
      const int row = idx / PER, c = (idx - row * PER) * VEC;
      r[j] = gld16(b, idx < TOTAL ? (uint32_t)(((int64_t)row * gs + c) * (int64_t)sizeof(T)) : OOB);
    }
  }
  __device__ __forceinline__ void store(T* s, int ls, int tid) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int idx = tid + j * NTH;
      const int row = idx / PER, c = (idx - row * PER) * VEC;
      if (idx < TOTAL) *reinterpret_cast<uint4*>(s + row * ls + c) = r[j];
    }
  }
  // The same tile from a column-blocked matrix [COLS/16][rt rows][16] (each
  // 16-column block row-major): rows row0 .. row0 + ROWS - 1.  Consecutive
  // threads take consecutive pieces of one block, so a wave reads contiguous
  // memory; store_cb() puts each piece at its row and column in LDS.
  static constexpr int SP = 16 / VEC;  // pieces per row of a block
  static_assert(COLS % 16 == 0, "column blocks of 16");
  __device__ __forceinline__ void load_cb(const GBuf& b, int rt, int row0, int tid) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int idx = tid + j * NTH;
      const int sub = idx % SP, rr = (idx / SP) % ROWS, blk = idx / (SP * ROWS);
      r[j] = gld16(b, idx < TOTAL ? (uint32_t)((((int64_t)blk * rt + row0 + rr) * 16 + sub * VEC) * (int64_t)sizeof(T))
                                  : OOB);
    }
  }
  __device__ __forceinline__ void store_cb(T* s, int ls, int tid) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int idx = tid + j * NTH;
      const int sub = idx % SP, rr = (idx / SP) % ROWS, blk = idx / (SP * ROWS);
      if (idx < TOTAL) *reinterpret_cast<uint4*>(s + rr * ls + blk * 16 + sub * VEC) = r[j];
    }
  }
};

// beta may be stored as bf16 or fp32 independently of the feature dtype.
// ld_beta_raw() issues the load and returns the element's raw bits; the value
// is decoded by beta_val() where it is used, so the wait for the load falls
// there and not at the load.
__device__ __forceinline__ uint32_t ld_beta_raw(const void* p, int is_f32, int64_t idx) {
  if (is_f32) return reinterpret_cast<const uint32_t*>(p)[idx];
  return reinterpret_cast<const uint16_t*>(p)[idx];
}
__device__ __forceinline__ float beta_val(uint32_t raw, int is_f32) {
  return __uint_as_float(is_f32 ? raw : raw << 16);
}
__device__ __forceinline__ float ld_beta(const void* p, int is_f32, int64_t idx) {
  return is_f32 ? reinterpret_cast<const float*>(p)[idx]
                : (float)reinterpret_cast<const bf16*>(p)[idx];
}
__device__ __forceinline__ void st_beta(void* p, int is_f32, int64_t idx, float v) {
  if (is_f32)
    reinterpret_cast<float*>(p)[idx] = v;
  else
    reinterpret_cast<bf16*>(p)[idx] = (bf16)v;
}

// ---- register-fragment products -------------------------------------------
// Four values along a 16-long contraction held by one lane: the A-operand
// fragment of row (l & 15) or the B-operand fragment of column (l & 15).
template <typename T>
struct Frag4;
template <>
struct Frag4<bf16> {
  using type = bf16x4;
};
template <>
struct Frag4<float> {
  using type = f32x4;
};

// acc += A[16 x 16] B[16 x 16] with both operands given as lane fragments: lane
// l supplies A(l & 15, 4 (l >> 4) + e) and B(4 (l >> 4) + e, l & 15), e = 0..3.
// fp32 runs four 16x16x4 steps, step e taking contraction slot 4 (l >> 4) + e.
__device__ __forceinline__ void mm16(f32x4& acc, bf16x4 a, bf16x4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mm16(f32x4& acc, f32x4 a, f32x4 b) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ typename Frag4<T>::type to_frag(const f32x4& x) {
  if constexpr (std::is_same_v<T, bf16>) {
    bf16x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (bf16)x[e];
    return r;
  } else {
    return x;
  }
}

// x ~ hi + lo in bf16: hi = x rounded to nearest, lo = (x - hi) rounded.  One
// pair conversion gives both hi values; their fp32 values are the lower and
// upper halves of its bits moved into place.  The packed word passes an empty
// asm statement, so the compiler keeps the pair conversion instead of
// converting each element again on its own.
__device__ __forceinline__ void split_bf16(const f32x4& x, bf16x4& hi, bf16x4& lo) {
  uint32_t hb[2], lb[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    hb[p] = __builtin_bit_cast(uint32_t, bf16x2{(bf16)x[2 * p], (bf16)x[2 * p + 1]});
    asm("" : "+v"(hb[p]));
    const float h0 = __uint_as_float(hb[p] << 16), h1 = __uint_as_float(hb[p] & 0xffff0000u);
    lb[p] = __builtin_bit_cast(uint32_t, bf16x2{(bf16)(x[2 * p] - h0), (bf16)(x[2 * p + 1] - h1)});
  }
  hi = __builtin_bit_cast(bf16x4, u32x2{hb[0], hb[1]});
  lo = __builtin_bit_cast(bf16x4, u32x2{lb[0], lb[1]});
}

// acc += M x (hi + lo) for a sending operand x given in fp32 (bf16: two MFMAs).
template <typename T>
__device__ __forceinline__ void mm16_split(f32x4& acc, typename Frag4<T>::type m, const f32x4& x) {
  if constexpr (std::is_same_v<T, bf16>) {
    bf16x4 hi, lo;
    split_bf16(x, hi, lo);
    mm16(acc, m, hi);
    mm16(acc, m, lo);
  } else {
    mm16(acc, m, x);
  }
}

// Compile-time loop: f(std::integral_constant<int, i>) for i in [B, E).  Every
// register array below is indexed by such constants only (an index the
// compiler cannot resolve would move the array to scratch memory).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// arr[I] for a wave-uniform I, by selects
template <typename X>
__device__ __forceinline__ X pick(const X (&arr)[NSUB], int I) {
  X r = arr[0];
  static_for<1, NSUB>([&](auto J) {
    if (I == J) r = arr[J];
  });
  return r;
}
__device__ __forceinline__ float comp(const f32x4& x, int e) {
  return e == 0 ? x[0] : e == 1 ? x[1] : e == 2 ? x[2] : x[3];
}

// LDS row pitch (elements) for a row of C elements of type T: +16 bytes of
// padding keeps 16-byte alignment and spreads rows over the banks.
template <typename T>
constexpr int pitch(int C) {
  return C + 16 / (int)sizeof(T);
}

}  // namespace rewy
