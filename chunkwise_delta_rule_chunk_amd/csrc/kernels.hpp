// Kernel argument record and host-side launchers of the gfx950 kernels.
// One record carries every pointer a pass may touch; each kernel reads the
// fields it needs.  Intermediate buffers live in the caller's workspace (or,
// for the save-all policy, in the caller's `saved` buffer).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace rewy {

struct Args {
  // problem
  int B, T, H, K, V, N;     // T = tokens per batch row (total tokens when packed)
  int nc_max;               // chunk slots (upper bound on the number of chunks)
  int gate;                 // 0 none, 1 scalar, 2 vector
  int beta_f32;             // beta / dbeta stored as fp32 (else bf16)
  float scale;
  const int* cu;            // device cu_seqlens [N+1] or nullptr
  // chunk index (workspace)
  ChunkInfo* chunks;        // [nc_max]
  int* seqoff;              // [N+1] first chunk slot of each sequence
  int* seqord;              // [N] scan order: sequences by chunk count, longest first
  // inputs
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;         // beta [BT,H]; in the erase/write form the erase gate b [BT,H,K]
  const void* wg;           // erase/write form: the write gate w [BT,H,V], else nullptr
  int ew;                   // 1 for the erase/write form
  // gate in the kernel, from the pre-activation x [BT,H,K] (feature dtype),
  // A_log [H], dt_bias [H,K], z = x + dt_bias[h, k]:
  //   gate_lb == 0:  g = -exp(A_log[h]) softplus(z)
  //   gate_lb < 0:   g = gate_lb sigmoid(exp(A_log[h]) z)   (bounded form)
  const void* gx;
  const float* a_log;
  const float* dt_bias;
  float gate_lb;
  int gin;                  // 1 when the gate is formed in the kernels
  const float* h0;
  const void* dO;
  const float* dht;
  // outputs
  void* o;
  float* ht;
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  void* dbeta;              // dbeta [BT,H]; in the erase/write form db [BT,H,K]
  void* dw;                 // erase/write form: dw [BT,H,V]
  void* dgx;                // gate in the kernel: dx [BT,H,K] (feature dtype)
  float* da_log;            // gate in the kernel: dA_log [H]
  float* ddt_bias;          // gate in the kernel: ddt_bias [H,K]
  float* gpart;             // gate in the kernel: per (chunk, head, wave) partial sums
  float* dh0;
  // Forward intermediates.  Token-major tensors are [BT,H,*]; chunk tiles are
  // [nc_max,H,rows,64] with all 64 token columns written (zeros past the
  // chunk's end).  Each product reads its operands with the contraction index
  // contiguous, so tiles that are contracted over tokens are stored with the
  // token index last (the "t" tiles).
  //
  // The forward scan's operands are stored in operand-fragment order, one
  // [64 x K] or [64 x V] tile per (chunk, head), so that each MFMA operand a
  // wave needs is one contiguous load of 16 bytes per lane (VE = 16 / sizeof
  // element, KG = 4 VE contraction slots per fragment, lane l, e < VE):
  //   W  piece ((tw * K/(16 GPP) + q) * 64 + l) holds, GPP = 16 / (4 sizeof element) groups
  //      of four, W[16 tw + (l & 15)][16 (GPP q + hh) + 4 (l >> 4) + e], hh < GPP, e < 4
  //      (the C fragments of W^T tiles, which are the 16-long A fragments of W)
  //   Ft piece ((tk * 64/KG + q) * 64 + l) holds F[KG q + VE (l >> 4) + e][16 tk + (l & 15)]
  //   U  piece ((tv * 4 + tw) * 64 + l) holds U[16 tw + 4 (l >> 4) + i][16 tv + (l & 15)], i < 4
  // (U in the C-fragment layout of the R tile it is subtracted from).  The
  // reverse scan's operands F, Wt, Qgt and Cqt are stored the same way (F
  // like W, the "t" tiles like Ft).
  int prep_mode;  // PREP_* bits: which of the sets below k_fwd_prep writes
  void* W;       // A E                 [nc,H,64,K] fragment order   forward scan (R = U - W S)
  void* Ft;      // F^T, F = K exp2(Gn - G) [nc,H,K,64] fragment order   forward scan (S += F^T R)
  void* U;       // A Z                 [nc,H,64,V] fragment order   forward scan
  float* glast;  // G2 at the last row  [nc,H,K]     both scans
  void* Qg;      // s Q exp2(G)         [nc,H,64,K] in the order of W   forward scan output product
  void* Cq;      // tril_incl(Qg Y^T)   [nc,H,4,4,64 lanes,4]: block (I, J) holds the C fragment of
                 // (Cq_IJ)^T, i.e. Cq[16 I + (l & 15)][16 J + 4 (l >> 4) + e]   forward scan output product
  void* F;       // F                   [nc,H,64,K] fragment order   reverse scan (Rbar = F dS+)
  void* Wt;      // W^T                 [nc,H,K,64] fragment order   reverse scan (dS -= W^T Rbar)
  void* Qgt;     // Qg^T                [nc,H,K,64] fragment order   reverse scan (dS += Qg^T dO)
  void* Cqt;     // Cq^T                [nc,H,64,64] fragment order  reverse scan (Rbar += Cq^T dO)
  void* hbuf;    // state entering each chunk [nc,H,V/16,K,16] dtype (column-blocked)
  void* R;       // corrections U - W S [nc,H,V/16,64,16] dtype (column-blocked, zero past the end)
  int scan_out;  // SCAN_* bits: whether the forward scan writes hbuf/R and whether it forms o
  void* At;      // A^T                 [nc,H,64,64] chunk backward (P = A^T Rbar)
  float* G2t;    // G2 of a scalar gate [nc,H,64] (rows past the end: G2 of the last row); the
                 // chunk backward rebuilds G2 of a vector gate from g (or x) and Gst
  float* Gst;    // sub-chunk gate statistics [nc,H,4,K] of float4 {G2 at the first row,
                 // G2 at the last valid row, midpoint (max+min)/2, range max-min}
  // backward intermediates
  void* Rbt;     // correction adjoint Rbar [nc,H,V/16,4,64 lanes,4] dtype, C-fragment order of its 16x16 tiles
  void* dhbuf;   // adjoint of the state leaving each chunk [nc,H,V/16,K,16] dtype (column-blocked)
  // separate producer-consumer schedule: what the producer hands over
  void* Pbuf;    // P = A^T Rbar [nc,H,64,V] dtype (rounded as the consumers read it)
  void* Dfrag;   // D as operand fragments [nc,H,4 waves,4 blocks,2,64 lanes,4] dtype
  float* Ddiag;  // diagonal blocks of D [nc,H,4,16,16] fp32
  float* dbw;    // write part of dbeta [nc,H,64] fp32
};

constexpr int SCAN_NATURAL = 1;  // hbuf, R (read by the chunk backward)
constexpr int SCAN_OUTPUT = 2;   // o = Qg S + Cq R, formed by the forward scan

constexpr int PREP_FWD_SCAN = 1;  // W, Ft, U, glast
constexpr int PREP_FWD_OUT = 2;   // Qg, Cq
constexpr int PREP_BWD_SCAN = 4;  // F, Wt, Qgt, Cqt, glast
constexpr int PREP_BWD_CHUNK = 8; // At, Gst, G2t (scalar gate)
// The erase/write form: beta holds the erase gate b [.., K] and wg the write
// gate w [.., V] (both in the feature dtype); E = b gamma K and Z = w V.
constexpr int PREP_EW = 16;
// The gate formed in the kernel from its pre-activation (Args::gx).
constexpr int PREP_GIN = 32;

// The kernel this thread enqueued last (its host-side stub), so that the
// tracing hook can name each launch exactly as the profiler does.
const void*& last_kernel();
// Every launch goes through this macro: one launch of KERNEL (a possibly
// parenthesised template-id) with no dynamic LDS, recorded in last_kernel().
#define REWY_LAUNCH(KERNEL, GRID, BLOCK, STREAM, ...)                             \
  do {                                                                          \
    ::rewy::last_kernel() = reinterpret_cast<const void*>(&KERNEL);             \
    hipLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, STREAM, __VA_ARGS__);            \
  } while (0)

// Launchers: enqueue on `stream`; return the hipError_t of the launch.
hipError_t launch_chunk_table(const Args& a, hipStream_t s);
hipError_t launch_fwd_prep(const Args& a, int dtype_f32, hipStream_t s);
// Value-tile width of the scans: 16 or 32 columns per workgroup, chosen so
// that the number of workgroups covers the chip.
int scan_bv(const Args& a, int dtype_f32);
hipError_t launch_fwd_scan(const Args& a, int dtype_f32, hipStream_t s);
hipError_t launch_bwd_scan(const Args& a, int dtype_f32, hipStream_t s);
// the forward scan (natural outputs) and the reverse scan in one launch
hipError_t launch_scans(const Args& a, int dtype_f32, hipStream_t s);
hipError_t launch_bwd_chunk(const Args& a, int dtype_f32, hipStream_t s);
// the separate schedule of the chunk backward: producer, then consumers
hipError_t launch_bwd_producer(const Args& a, int dtype_f32, hipStream_t s);
hipError_t launch_bwd_consumers(const Args& a, int dtype_f32, hipStream_t s);
// the gate-in-kernel parameter gradients from the chunk backward's partials
hipError_t launch_gate_reduce(const Args& a, hipStream_t s);
// the token-serial forward (decode)
hipError_t launch_recurrent(const Args& a, int dtype_f32, hipStream_t s);

}  // namespace rewy
