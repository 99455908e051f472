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
  // inputs
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
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
  void* dbeta;
  float* dh0;
  // forward intermediates (token-major [BT,H,*] or chunk-major [nc_max,H,*,*])
  void* W;       // A E              [BT,H,K]   dtype
  void* U;       // A Z              [BT,H,V]   dtype
  void* F;       // K exp2(Gn - G)   [BT,H,K]   dtype
  void* Qg;      // s Q exp2(G)      [BT,H,K]   dtype
  void* Cq;      // tril_incl(Qg Y^T) [nc,H,64,64] dtype
  float* glast;  // G2 at the last row [nc,H,K] fp32
  void* hbuf;    // state entering each chunk [nc,H,K,V] dtype
  void* R;       // corrections U - W S [BT,H,V] dtype
  // backward intermediates
  void* Rb;      // accumulated correction adjoint [BT,H,V] dtype
  void* dhbuf;   // adjoint of the state leaving each chunk [nc,H,K,V] dtype
  void* P;       // shared sensitivity A^T Rbar [BT,H,V] dtype
  void* D;       // -tril_strict(P R^T) [nc,H,64,64] dtype
  void* Hq;      // tril_incl(dO R^T)   [nc,H,64,64] dtype
  float* dbw;    // write part of dbeta, <V_i, P_i>  [BT,H] fp32
};

// Scan tile width over the value axis (one workgroup per sequence, head and
// value tile).
constexpr int SCAN_BV = 32;

// Launchers: enqueue on `stream`; return the hipError_t of the launch.
hipError_t launch_chunk_table(const Args& a, hipStream_t s);
hipError_t launch_fwd_prep(const Args& a, int dtype_f32, hipStream_t s);
hipError_t launch_fwd_scan(const Args& a, int dtype_f32, hipStream_t s);
hipError_t launch_fwd_out(const Args& a, int dtype_f32, hipStream_t s);
hipError_t launch_bwd_scan(const Args& a, int dtype_f32, hipStream_t s);
hipError_t launch_bwd_prod(const Args& a, int dtype_f32, hipStream_t s);
hipError_t launch_bwd_cons(const Args& a, int dtype_f32, hipStream_t s);

}  // namespace rewy
