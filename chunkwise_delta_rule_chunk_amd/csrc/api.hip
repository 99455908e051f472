// Host side of the C ABI declared in include/rewy.h: argument validation,
// workspace planning and the launch sequence of each pass.  Nothing here
// allocates device memory or waits for the device.
#include <cxxabi.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "rewy.h"

#define REWY_API extern "C" __attribute__((visibility("default")))

namespace rewy {

const void*& last_kernel() {
  static thread_local const void* k = nullptr;
  return k;
}

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

constexpr size_t ALIGN = 256;
size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Plan {
  int B, T, H, K, V, N, nc_max;
  int64_t BT;  // packed tokens
  bool f32, beta_f32;
  int gate, policy;
  int sched;   // REWY_SCHEDULE_* of the chunk backward
  size_t esz;
};

// Schedule of the chunk backward for later calls (rewy_bwd_schedule).
std::atomic<int> g_schedule{REWY_SCHEDULE_JOINT};

int kv_supported(int K, int V, bool f32) {
  auto ok = [](int x) { return x == 32 || x == 64 || x == 128; };
  if (!ok(K) || !ok(V)) return 0;
  if (f32 && (K > 64 || V > 64)) return 0;
  return 1;
}

int make_plan(const rewy_desc* d, Plan& p) {
  if (!d) return fail(REWY_EINVAL, "desc is NULL");
  if (d->B <= 0 || d->T < 0 || d->H <= 0 || d->K <= 0 || d->V <= 0)
    return fail(REWY_EINVAL, "bad shape B=%d T=%d H=%d K=%d V=%d", d->B, d->T, d->H, d->K, d->V);
  if (d->dtype != REWY_BF16 && d->dtype != REWY_F32) return fail(REWY_EINVAL, "bad dtype %d", d->dtype);
  if (d->beta_dtype != REWY_BF16 && d->beta_dtype != REWY_F32)
    return fail(REWY_EINVAL, "bad beta_dtype %d", d->beta_dtype);
  if (d->gate < REWY_GATE_NONE || d->gate > REWY_GATE_VECTOR) return fail(REWY_EINVAL, "bad gate %d", d->gate);
  if (d->policy != REWY_RECOMPUTE && d->policy != REWY_SAVE) return fail(REWY_EINVAL, "bad policy %d", d->policy);
  if (d->K > 256) return fail(REWY_EINVAL, "K=%d exceeds 256", d->K);
  const bool f32 = d->dtype == REWY_F32;
  if (!kv_supported(d->K, d->V, f32))
    return fail(REWY_EUNSUPPORTED, "K=%d V=%d not supported for %s (K, V in {32,64,128}; fp32 <= 64)",
                d->K, d->V, f32 ? "fp32" : "bf16");
  p.B = d->B; p.T = d->T; p.H = d->H; p.K = d->K; p.V = d->V;
  p.sched = g_schedule.load();
  p.f32 = f32; p.beta_f32 = d->beta_dtype == REWY_F32; p.gate = d->gate; p.policy = d->policy;
  p.esz = f32 ? 4 : 2;
  p.BT = (int64_t)d->B * d->T;
  if (p.BT >= (int64_t)1 << 31) return fail(REWY_EINVAL, "B*T=%lld exceeds int32", (long long)p.BT);
  if (d->cu_seqlens) {
    if (d->B != 1) return fail(REWY_EINVAL, "cu_seqlens requires B == 1 (got B=%d)", d->B);
    if (d->N <= 0) return fail(REWY_EINVAL, "cu_seqlens requires N >= 1 (got N=%d)", d->N);
    p.N = d->N;
    if (d->cu_seqlens_host) {
      const int32_t* cu = d->cu_seqlens_host;
      if (cu[0] != 0 || cu[p.N] != d->T)
        return fail(REWY_EINVAL, "cu_seqlens must start at 0 and end at T=%d", d->T);
      for (int i = 0; i < p.N; ++i)
        if (cu[i + 1] < cu[i]) return fail(REWY_EINVAL, "cu_seqlens not ascending at %d", i);
    }
    // Chunk slots: sum over sequences of ceil(len / 64) <= ceil(T / 64) + N.
    // The bound, not the exact count, so that every buffer layout (workspace
    // and saved) is the same whether or not the host copy is passed.
    p.nc_max = (int)std::min<int64_t>((int64_t)(d->T + CH - 1) / CH + p.N, INT32_MAX);
  } else {
    if (d->N != 0 && d->N != d->B) return fail(REWY_EINVAL, "N=%d must equal B=%d without cu_seqlens", d->N, d->B);
    p.N = d->B;
    p.nc_max = d->B * ((d->T + CH - 1) / CH);
  }
  return REWY_OK;
}

// Buffer layout.  `saved` holds what the backward reads from the forward under
// the save-all policy; everything else is scratch in the workspace.  The
// reverse set is what the reverse scan and the chunk backward read:
// F Wt Qgt Cqt (reverse scan) and At G2t Gst (chunk backward; G2t only for a
// scalar gate).
//   recompute: ws = [index | glast | W Ft U | (fwd) Qg Cq
//                                           | (bwd) hbuf R reverse set Rbt dhbuf]
//   save-all:  saved = [glast hbuf R | reverse set]
//              ws (fwd) = [index | W Ft U Qg Cq],  ws (bwd) = [index | Rbt dhbuf]
// The forward of the recompute policy writes neither hbuf nor R, so they share
// the output operands' space with the rest of the backward's buffers.  The
// backward with the gate formed in the kernel appends the per-wave partial
// sums of the gate parameters' gradients to its workspace (phase 2).
struct Layout {
  size_t chunks, seqoff, seqord;
  size_t glast, hbuf, R;             // read by output and backward
  size_t W, Ft, U;                   // forward scan operands
  size_t Qg, Cq;                     // output-product operands
  size_t F, Wt, Qgt, Cqt;            // reverse scan operands
  size_t At, G2t, Gst;               // chunk backward operands
  size_t Rbt, dhbuf;                 // written by the reverse scan
  size_t Pbuf, Dfrag, Ddiag, dbw;    // separate schedule: producer to consumers
  size_t gpart;                      // gate in the kernel: [nc,H,NSUB,K] then [nc,H,NSUB] fp32
  size_t ws_fwd, ws_bwd, ws_gin, saved;
};

Layout layout(const Plan& p) {
  Layout L{};
  const size_t nc = p.nc_max, H = p.H, K = p.K, V = p.V, e = p.esz;
  const size_t tileK = nc * H * K * CH * e, tileV = nc * H * V * CH * e;
  const size_t tile64 = nc * H * CH * CH * e, states = nc * H * K * V * e;
  const size_t g2 = p.gate == REWY_GATE_SCALAR ? nc * H * CH * 4 : 0;  // G2 row of a scalar gate
  size_t off = 0;
  auto take = [&](size_t& o, size_t bytes) { const size_t r = o; o += up(bytes); return r; };
  auto take_reverse = [&](size_t& o) {
    L.F = take(o, tileK);
    L.Wt = take(o, tileK);
    L.Qgt = take(o, tileK);
    L.Cqt = take(o, tile64);
    L.At = take(o, tile64);
    L.G2t = take(o, g2);
    L.Gst = take(o, nc * H * NSUB * K * 16);
  };
  L.chunks = take(off, nc * sizeof(ChunkInfo));
  L.seqoff = take(off, (size_t)(p.N + 1) * 4);
  L.seqord = take(off, (size_t)p.N * 4);
  const size_t head = off;
  const bool save = p.policy == REWY_SAVE;
  size_t s = save ? 0 : off;
  L.glast = take(s, nc * H * K * 4);
  if (save) {
    L.hbuf = take(s, states);
    L.R = take(s, tileV);
    take_reverse(s);
    L.saved = s;
    off = head;
  } else {
    off = s;
  }
  L.W = take(off, tileK);
  L.Ft = take(off, tileK);
  L.U = take(off, tileV);
  const size_t after_scan = off;
  L.Qg = take(off, tileK);
  L.Cq = take(off, tile64);
  L.ws_fwd = off;
  if (save) {
    off = head;
  } else {
    off = after_scan;  // the backward's buffers share the output operands' space
    L.hbuf = take(off, states);
    L.R = take(off, tileV);
    take_reverse(off);
  }
  L.Rbt = take(off, tileV);
  L.dhbuf = take(off, states);
  if (p.sched == REWY_SCHEDULE_SEPARATE) {
    L.Pbuf = take(off, tileV);
    L.Dfrag = take(off, nc * H * NSUB * NSUB * 2 * 64 * 4 * e);
    L.Ddiag = take(off, nc * H * NSUB * SUB * SUB * 4);
    L.dbw = take(off, nc * H * CH * 4);
  }
  L.ws_bwd = off;
  L.gpart = take(off, nc * H * NSUB * (K + 1) * 4);
  L.ws_gin = off;
  return L;
}

__global__ void k_copy_or_zero(float* dst, const float* src, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src ? src[i] : 0.f;
}

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(REWY_EHIP, "%s: %s", what, hipGetErrorString(e));
  return REWY_OK;
}

int copy_state(float* dst, const float* src, int64_t n, hipStream_t s) {
  if (!dst || n == 0) return REWY_OK;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
  REWY_LAUNCH(k_copy_or_zero, dim3(blocks), dim3(256), s, dst, src, n);
  return hip_check(hipGetLastError(), "state copy");
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

void fill_common(Args& a, const Plan& p, const rewy_desc* d, char* ws, char* sv,
                 const Layout& L) {
  memset(&a, 0, sizeof(a));
  a.B = p.B; a.T = p.T; a.H = p.H; a.K = p.K; a.V = p.V; a.N = p.N; a.nc_max = p.nc_max;
  a.gate = p.gate; a.beta_f32 = p.beta_f32; a.scale = d->scale; a.cu = d->cu_seqlens;
  a.chunks = reinterpret_cast<ChunkInfo*>(ws + L.chunks);
  a.seqoff = reinterpret_cast<int*>(ws + L.seqoff);
  a.seqord = reinterpret_cast<int*>(ws + L.seqord);
  char* fs = p.policy == REWY_SAVE ? sv : ws;  // where the saved set lives
  a.glast = reinterpret_cast<float*>(fs + L.glast);
  a.hbuf = fs + L.hbuf; a.R = fs + L.R;
  a.F = fs + L.F; a.Wt = fs + L.Wt; a.Qgt = fs + L.Qgt; a.Cqt = fs + L.Cqt;
  a.W = ws + L.W; a.Ft = ws + L.Ft; a.U = ws + L.U; a.Qg = ws + L.Qg; a.Cq = ws + L.Cq;
  a.At = fs + L.At;
  a.G2t = reinterpret_cast<float*>(fs + L.G2t);
  a.Gst = reinterpret_cast<float*>(fs + L.Gst);
  a.Rbt = ws + L.Rbt; a.dhbuf = ws + L.dhbuf;
  if (p.sched == REWY_SCHEDULE_SEPARATE) {
    a.Pbuf = ws + L.Pbuf;
    a.Dfrag = ws + L.Dfrag;
    a.Ddiag = reinterpret_cast<float*>(ws + L.Ddiag);
    a.dbw = reinterpret_cast<float*>(ws + L.dbw);
  }
}

int check_tensor_ptrs(const void* const* ps, const char* const* names, int n) {
  for (int i = 0; i < n; ++i) {
    if (!ps[i]) return fail(REWY_EINVAL, "%s is NULL", names[i]);
    if (!aligned(ps[i], 16)) return fail(REWY_EINVAL, "%s is not 16-byte aligned", names[i]);
  }
  return REWY_OK;
}

// ---- tracing: event pairs around every launch, per thread ------------------
struct TraceRec {
  const void* fn;  // host stub of the launched kernel
  hipStream_t s;
  hipEvent_t e0, e1;
};
struct Tracer {
  bool on = false;
  char only[64] = {0};  // empty: every launch
  std::vector<TraceRec> recs;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  hipEvent_t ev() {
    if (used == pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
};
thread_local Tracer g_tr;

// `stage` is the kernel's template name, which rewy_trace_select matches
template <typename F>
hipError_t traced(const char* stage, hipStream_t s, F&& launch) {
  if (!g_tr.on || (g_tr.only[0] && strcmp(g_tr.only, stage) != 0)) return launch();
  TraceRec r{nullptr, s, g_tr.ev(), g_tr.ev()};
  if (r.e0) hipEventRecord(r.e0, s);
  last_kernel() = nullptr;
  const hipError_t e = launch();
  if (r.e1) hipEventRecord(r.e1, s);
  r.fn = last_kernel();
  if (r.e0 && r.e1 && r.fn) g_tr.recs.push_back(r);
  return e;
}

// The kernel's name as the profiler reports it: the symbol of the launched
// instantiation (every template argument included), demangled where the
// host's demangler can.
std::string kernel_name(const TraceRec& r) {
  const char* m = hipKernelNameRefByPtr(r.fn, r.s);
  if (!m) return "unknown";
  int st = 0;
  char* d = abi::__cxa_demangle(m, nullptr, nullptr, &st);
  // the mangled symbol where the demangler cannot read it (the bfloat16 type
  // code DF16b), as rocprofv3 prints it then
  std::string out = (st == 0 && d) ? std::string(d) : std::string(m);
  free(d);
  return out;
}

// Forward chunk stages shared by rewy_fwd and the recompute in rewy_bwd.
int run_forward_stages(const Args& a, bool f32, bool with_scan, hipStream_t s) {
  int rc;
  if ((rc = hip_check(traced("k_chunk_table", s, [&] { return launch_chunk_table(a, s); }),
                      "chunk table")))
    return rc;
  if ((rc = hip_check(traced("k_fwd_prep", s, [&] { return launch_fwd_prep(a, f32, s); }),
                      "forward prep")))
    return rc;
  if (with_scan &&
      (rc = hip_check(traced("k_fwd_scan", s, [&] { return launch_fwd_scan(a, f32, s); }),
                      "forward scan")))
    return rc;
  return REWY_OK;
}

}  // namespace
}  // namespace rewy

using namespace rewy;

REWY_API size_t rewy_workspace_bytes(const rewy_desc* d, int phase) {
  Plan p;
  if (make_plan(d, p) != REWY_OK) return 0;
  const Layout L = layout(p);
  if (phase == 2 && p.gate != REWY_GATE_VECTOR) {
    fail(REWY_EINVAL, "phase 2 (the gate formed in the kernel) needs gate == VECTOR");
    return 0;
  }
  if (phase < 0 || phase > 2) {
    fail(REWY_EINVAL, "bad phase %d", phase);
    return 0;
  }
  return phase == 0 ? L.ws_fwd : phase == 1 ? L.ws_bwd : L.ws_gin;
}

REWY_API size_t rewy_saved_bytes(const rewy_desc* d) {
  Plan p;
  if (make_plan(d, p) != REWY_OK) return 0;
  return layout(p).saved;
}

namespace rewy {
namespace {
// The gate formed in the kernel: pre-activation x [BT,H,K] (feature dtype),
// A_log [H] and dt_bias [H,K] (fp32).
struct GateIn {
  const void* x;
  const float* a_log;
  const float* dt_bias;
  float lower_bound;  // 0: softplus form; [-5, 0): bounded form
};

int check_gate_in(const Plan& p, const GateIn* gi) {
  if (p.gate != REWY_GATE_VECTOR) return fail(REWY_EINVAL, "the gate formed in the kernel needs gate == VECTOR");
  if (!gi->x || !gi->a_log || !gi->dt_bias) return fail(REWY_EINVAL, "x, A_log and dt_bias must be given");
  if (!aligned(gi->x, 16) || !aligned(gi->dt_bias, 16) || !aligned(gi->a_log, 4))
    return fail(REWY_EINVAL, "x and dt_bias must be 16-byte aligned, A_log 4-byte aligned");
  const float lb = gi->lower_bound;
  if (!(lb == 0.f || (lb >= -5.f && lb < 0.f)))
    return fail(REWY_EINVAL, "lower_bound must be 0 (softplus form) or in [-5, 0) (got %g)", (double)lb);
  return REWY_OK;
}

// The forward of every form: beta [BT,H] (shared erase/write factor), or
// with wg non-null the erase gate b [BT,H,K] in `beta` and the write gate w
// [BT,H,V] in `wg`, both in the feature dtype; with gi non-null the vector
// gate is formed in the kernel from gi (and g is not given).
int forward_impl(const rewy_desc* d, const void* q, const void* k, const void* v, const float* g,
                 const void* beta, const void* wg, const GateIn* gi, const float* h0, void* o,
                 float* ht, void* saved, void* workspace, size_t ws_bytes, void* stream) {
  Plan p;
  int rc = make_plan(d, p);
  if (rc) return rc;
  const bool ew = wg != nullptr;
  if (ew && d->beta_dtype != d->dtype)
    return fail(REWY_EUNSUPPORTED, "the erase/write gates must have the feature dtype");
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t state_n = (int64_t)p.N * p.H * p.K * p.V;
  if (p.BT == 0) return copy_state(ht, h0, state_n, s);
  {
    const void* ps[] = {q, k, v, beta, o};
    const char* nm[] = {"q", "k", "v", "beta", "o"};
    if ((rc = check_tensor_ptrs(ps, nm, 5))) return rc;
  }
  if (gi) {
    if ((rc = check_gate_in(p, gi))) return rc;
  } else if ((p.gate != REWY_GATE_NONE) != (g != nullptr)) {
    return fail(REWY_EINVAL, "g must be given exactly when gate != NONE");
  }
  if (g && !aligned(g, 16)) return fail(REWY_EINVAL, "g is not 16-byte aligned");
  const Layout L = layout(p);
  if (!workspace || !aligned(workspace, ALIGN) || ws_bytes < L.ws_fwd)
    return fail(REWY_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", L.ws_fwd,
                ws_bytes);
  if (p.policy == REWY_SAVE && (!saved || !aligned(saved, ALIGN)))
    return fail(REWY_EWORKSPACE, "policy SAVE needs a 256-byte aligned saved buffer of %zu bytes",
                L.saved);
  Args a;
  fill_common(a, p, d, static_cast<char*>(workspace), static_cast<char*>(saved), L);
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.h0 = h0; a.o = o; a.ht = ht;
  a.wg = wg; a.ew = ew;
  if (gi) {
    a.g = nullptr; a.gx = gi->x; a.a_log = gi->a_log; a.dt_bias = gi->dt_bias; a.gin = 1;
    a.gate_lb = gi->lower_bound;
  }
  if (ew && !aligned(wg, 16)) return fail(REWY_EINVAL, "w is not 16-byte aligned");
  a.prep_mode = PREP_FWD_SCAN | PREP_FWD_OUT |
                (p.policy == REWY_SAVE ? PREP_BWD_SCAN | PREP_BWD_CHUNK : 0);
  a.scan_out = SCAN_OUTPUT | (p.policy == REWY_SAVE ? SCAN_NATURAL : 0);
  return run_forward_stages(a, p.f32, true, s);
}
}  // namespace
}  // namespace rewy

REWY_API int rewy_fwd(const rewy_desc* d, const void* q, const void* k, const void* v,
                      const float* g, const void* beta, const float* h0, void* o, float* ht,
                      void* saved, void* workspace, size_t ws_bytes, void* stream) {
  return forward_impl(d, q, k, v, g, beta, nullptr, nullptr, h0, o, ht, saved, workspace, ws_bytes,
                      stream);
}

// ---- the allocation-free forward ---------------------------------------------
// Its workspace is this file-scope device array, one copy per GPU (the loader
// places it in each device's memory when the library's code is loaded there,
// and it stays until the process ends).  In host code `scratch` only names the
// symbol: its device address comes from hipGetSymbolAddress, once per device,
// and only that address is ever handed to kernels.
namespace rewy {
static __device__ __align__(256) unsigned char scratch[REWY_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES] = {};

// The device address of `scratch` on the current device (resolved on the first
// call there), or nullptr with the error recorded.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
    fail(REWY_EHIP, "allocation-free forward: no current device (or more than %d)", MAX_DEVICES);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      fail(REWY_EHIP, "allocation-free forward: hipGetSymbolAddress: %s", hipGetErrorString(e));
      return nullptr;
    }
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}
}  // namespace
}  // namespace rewy

REWY_API int rewy_fwd_noalloc(const rewy_desc* d, const void* q, const void* k, const void* v,
                              const float* g, const void* beta, const float* h0, void* o,
                              float* ht, void* saved, void* stream) {
  // the size check comes first and touches no device
  Plan p;
  const int rc = make_plan(d, p);
  if (rc) return rc;
  const size_t need = layout(p).ws_fwd;
  if (need > (size_t)REWY_NOALLOC_SCRATCH_BYTES)
    return fail(REWY_EWORKSPACE,
                "rewy_fwd_noalloc: this problem needs %zu bytes of workspace, above the %zu-byte "
                "device scratch of the allocation-free forward (use rewy_fwd with a workspace)",
                need, (size_t)REWY_NOALLOC_SCRATCH_BYTES);
  if (stream) {  // kernels and the scratch address must belong to the stream's device
    int sdev = -1, cur = -1;
    if (hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev) != hipSuccess ||
        hipGetDevice(&cur) != hipSuccess)
      return fail(REWY_EHIP, "rewy_fwd_noalloc: cannot query the stream's device");
    if (sdev != cur)
      return fail(REWY_EINVAL, "rewy_fwd_noalloc: the stream belongs to device %d, the current "
                  "device is %d", sdev, cur);
  }
  void* ws = scratch_on_current_device();
  if (!ws) return REWY_EHIP;
  return forward_impl(d, q, k, v, g, beta, nullptr, nullptr, h0, o, ht, saved, ws,
                      (size_t)REWY_NOALLOC_SCRATCH_BYTES, stream);
}

REWY_API int rewy_fwd_kda_gate(const rewy_desc* d, const void* q, const void* k, const void* v,
                               const void* x, const float* a_log, const float* dt_bias,
                               float lower_bound, const void* beta, const float* h0, void* o,
                               float* ht, void* saved, void* workspace, size_t ws_bytes,
                               void* stream) {
  const GateIn gi{x, a_log, dt_bias, lower_bound};
  return forward_impl(d, q, k, v, nullptr, beta, nullptr, &gi, h0, o, ht, saved, workspace,
                      ws_bytes, stream);
}

REWY_API int rewy_fwd_gdn2(const rewy_desc* d, const void* q, const void* k, const void* v,
                           const float* g, const void* b, const void* w, const float* h0, void* o,
                           float* ht, void* saved, void* workspace, size_t ws_bytes, void* stream) {
  if (!b || !w) return fail(REWY_EINVAL, "b and w must be given");
  return forward_impl(d, q, k, v, g, b, w, nullptr, h0, o, ht, saved, workspace, ws_bytes, stream);
}

namespace rewy {
namespace {
// The token-serial forward; with wg non-null the erase/write form (b in
// `beta`, w in `wg`, both in the feature dtype).
int recurrent_impl(const rewy_desc* d, const void* q, const void* k, const void* v,
                   const float* g, const void* beta, const void* wg, const float* h0, void* o,
                   float* ht, void* stream) {
  Plan p;
  int rc = make_plan(d, p);
  if (rc) return rc;
  const bool ew = wg != nullptr;
  if (ew && d->beta_dtype != d->dtype)
    return fail(REWY_EUNSUPPORTED, "the erase/write gates must have the feature dtype");
  if (ew && !aligned(wg, 16)) return fail(REWY_EINVAL, "w is not 16-byte aligned");
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t state_n = (int64_t)p.N * p.H * p.K * p.V;
  if (p.BT == 0) return copy_state(ht, h0, state_n, s);
  {
    const void* ps[] = {q, k, v, beta, o};
    const char* nm[] = {"q", "k", "v", "beta", "o"};
    if ((rc = check_tensor_ptrs(ps, nm, 5))) return rc;
  }
  if ((p.gate != REWY_GATE_NONE) != (g != nullptr))
    return fail(REWY_EINVAL, "g must be given exactly when gate != NONE");
  if (g && !aligned(g, 16)) return fail(REWY_EINVAL, "g is not 16-byte aligned");
  Args a;
  memset(&a, 0, sizeof(a));
  a.B = p.B; a.T = p.T; a.H = p.H; a.K = p.K; a.V = p.V; a.N = p.N;
  a.gate = p.gate; a.beta_f32 = p.beta_f32; a.scale = d->scale; a.cu = d->cu_seqlens;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.h0 = h0; a.o = o; a.ht = ht;
  a.wg = wg; a.ew = ew;
  return hip_check(traced("k_recurrent", s,
                          [&] { return launch_recurrent(a, p.f32, s); }),
                   "recurrent forward");
}
}  // namespace
}  // namespace rewy

REWY_API int rewy_recurrent_fwd(const rewy_desc* d, const void* q, const void* k, const void* v,
                                const float* g, const void* beta, const float* h0, void* o,
                                float* ht, void* stream) {
  return recurrent_impl(d, q, k, v, g, beta, nullptr, h0, o, ht, stream);
}

REWY_API int rewy_recurrent_fwd_gdn2(const rewy_desc* d, const void* q, const void* k,
                                     const void* v, const float* g, const void* b, const void* w,
                                     const float* h0, void* o, float* ht, void* stream) {
  if (!b || !w) return fail(REWY_EINVAL, "b and w must be given");
  return recurrent_impl(d, q, k, v, g, b, w, h0, o, ht, stream);
}

namespace rewy {
namespace {
// Gradients of the gate formed in the kernel: dx [BT,H,K] (feature dtype),
// dA_log [H] and ddt_bias [H,K] (fp32, overwritten).
struct GateInGrad {
  void* dx;
  float* da_log;
  float* ddt_bias;
};

// The backward of every form; with wg non-null, `dbeta` receives db [BT,H,K]
// and `dw` receives dw [BT,H,V] (feature dtype); with gi non-null the gate is
// formed in the kernel and gg receives its gradients in place of dg.
int backward_impl(const rewy_desc* d, const void* q, const void* k, const void* v, const float* g,
                  const void* beta, const void* wg, const GateIn* gi, const float* h0,
                  const void* dO, const float* dht, const void* saved, void* dq, void* dk, void* dv,
                  float* dg, void* dbeta, void* dw, const GateInGrad* gg, float* dh0,
                  void* workspace, size_t ws_bytes, void* stream) {
  Plan p;
  int rc = make_plan(d, p);
  if (rc) return rc;
  const bool ew = wg != nullptr;
  if (ew && d->beta_dtype != d->dtype)
    return fail(REWY_EUNSUPPORTED, "the erase/write gates must have the feature dtype");
  if (ew && (!dw || !aligned(wg, 16) || !aligned(dw, 16)))
    return fail(REWY_EINVAL, "w and dw must be given, 16-byte aligned");
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (h0 && !dh0) return fail(REWY_EINVAL, "dh0 must be given when h0 is given");
  const int64_t state_n = (int64_t)p.N * p.H * p.K * p.V;
  if (p.BT == 0) return copy_state(dh0, dht, state_n, s);
  {
    const void* ps[] = {q, k, v, beta, dO, dq, dk, dv, dbeta};
    const char* nm[] = {"q", "k", "v", "beta", "dO", "dq", "dk", "dv", "dbeta"};
    if ((rc = check_tensor_ptrs(ps, nm, 9))) return rc;
  }
  if (gi) {
    if ((rc = check_gate_in(p, gi))) return rc;
    if (!gg->dx || !gg->da_log || !gg->ddt_bias)
      return fail(REWY_EINVAL, "dx, dA_log and ddt_bias must be given");
    if (!aligned(gg->dx, 16)) return fail(REWY_EINVAL, "dx is not 16-byte aligned");
  } else {
    if ((p.gate != REWY_GATE_NONE) != (g != nullptr))
      return fail(REWY_EINVAL, "g must be given exactly when gate != NONE");
    if ((p.gate != REWY_GATE_NONE) != (dg != nullptr))
      return fail(REWY_EINVAL, "dg must be given exactly when gate != NONE");
    if ((g && !aligned(g, 16)) || (dg && !aligned(dg, 16)))
      return fail(REWY_EINVAL, "g / dg must be 16-byte aligned");
  }
  const Layout L = layout(p);
  const size_t need = gi ? L.ws_gin : L.ws_bwd;
  if (!workspace || !aligned(workspace, ALIGN) || ws_bytes < need)
    return fail(REWY_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                ws_bytes);
  if (p.policy == REWY_SAVE && (!saved || !aligned(saved, ALIGN)))
    return fail(REWY_EWORKSPACE, "policy SAVE needs the saved buffer written by rewy_fwd");
  Args a;
  fill_common(a, p, d, static_cast<char*>(workspace),
              const_cast<char*>(static_cast<const char*>(saved)), L);
  a.prep_mode = PREP_FWD_SCAN | PREP_BWD_SCAN | PREP_BWD_CHUNK;
  a.scan_out = SCAN_NATURAL;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.h0 = h0; a.dO = dO; a.dht = dht;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
  a.wg = wg; a.ew = ew; a.dw = dw;
  if (gi) {
    a.g = nullptr; a.dg = nullptr;
    a.gx = gi->x; a.a_log = gi->a_log; a.dt_bias = gi->dt_bias; a.gin = 1;
    a.gate_lb = gi->lower_bound;
    a.dgx = gg->dx; a.da_log = gg->da_log; a.ddt_bias = gg->ddt_bias;
    a.gpart = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.gpart);
  }
  const bool f32 = p.f32;
  if (p.policy == REWY_RECOMPUTE) {
    // prep again, then the forward scan and the reverse scan side by side
    if ((rc = run_forward_stages(a, f32, false, s))) return rc;
    if ((rc = hip_check(traced("k_scans", s, [&] { return launch_scans(a, f32, s); }),
                        "forward and reverse scans")))
      return rc;
  } else {
    if ((rc = hip_check(traced("k_chunk_table", s, [&] { return launch_chunk_table(a, s); }),
                        "chunk table")))
      return rc;
    if ((rc = hip_check(traced("k_bwd_scan", s, [&] { return launch_bwd_scan(a, f32, s); }),
                        "reverse scan")))
      return rc;
  }
  // the separate schedule serves the shared-beta forms; the others run joint
  if (p.sched == REWY_SCHEDULE_SEPARATE && !ew && !gi) {
    if ((rc = hip_check(traced("k_bwd_chunk", s, [&] { return launch_bwd_producer(a, f32, s); }),
                        "chunk backward producer")))
      return rc;
    if ((rc = hip_check(traced("k_bwd_chunk", s, [&] { return launch_bwd_consumers(a, f32, s); }),
                        "chunk backward consumers")))
      return rc;
  } else if ((rc = hip_check(traced("k_bwd_chunk", s, [&] { return launch_bwd_chunk(a, f32, s); }),
                             "chunk backward"))) {
    return rc;
  }
  if (gi && (rc = hip_check(traced("k_gate_reduce", s, [&] { return launch_gate_reduce(a, s); }),
                            "gate parameter gradients")))
    return rc;
  return REWY_OK;
}
}  // namespace
}  // namespace rewy

REWY_API int rewy_bwd(const rewy_desc* d, const void* q, const void* k, const void* v,
                      const float* g, const void* beta, const float* h0, const void* dO,
                      const float* dht, const void* saved, void* dq, void* dk, void* dv,
                      float* dg, void* dbeta, float* dh0, void* workspace, size_t ws_bytes,
                      void* stream) {
  return backward_impl(d, q, k, v, g, beta, nullptr, nullptr, h0, dO, dht, saved, dq, dk, dv, dg,
                       dbeta, nullptr, nullptr, dh0, workspace, ws_bytes, stream);
}

REWY_API int rewy_bwd_kda_gate(const rewy_desc* d, const void* q, const void* k, const void* v,
                               const void* x, const float* a_log, const float* dt_bias,
                               float lower_bound, const void* beta, const float* h0,
                               const void* dO, const float* dht, const void* saved, void* dq,
                               void* dk, void* dv, void* dx, float* da_log, float* ddt_bias,
                               void* dbeta, float* dh0, void* workspace, size_t ws_bytes,
                               void* stream) {
  const GateIn gi{x, a_log, dt_bias, lower_bound};
  const GateInGrad gg{dx, da_log, ddt_bias};
  return backward_impl(d, q, k, v, nullptr, beta, nullptr, &gi, h0, dO, dht, saved, dq, dk, dv,
                       nullptr, dbeta, nullptr, &gg, dh0, workspace, ws_bytes, stream);
}

REWY_API int rewy_bwd_gdn2(const rewy_desc* d, const void* q, const void* k, const void* v,
                           const float* g, const void* b, const void* w, const float* h0,
                           const void* dO, const float* dht, const void* saved, void* dq, void* dk,
                           void* dv, float* dg, void* db, void* dw, float* dh0, void* workspace,
                           size_t ws_bytes, void* stream) {
  if (!b || !w) return fail(REWY_EINVAL, "b and w must be given");
  return backward_impl(d, q, k, v, g, b, w, nullptr, h0, dO, dht, saved, dq, dk, dv, dg, db, dw,
                       nullptr, dh0, workspace, ws_bytes, stream);
}

REWY_API int rewy_bwd_schedule(int schedule) {
  if (schedule < 0) return g_schedule.load();
  if (schedule != REWY_SCHEDULE_JOINT && schedule != REWY_SCHEDULE_SEPARATE)
    return fail(REWY_EINVAL, "bad schedule %d", schedule);
  return g_schedule.exchange(schedule);
}

REWY_API int rewy_trace_begin(void) {
  g_tr.recs.clear();
  g_tr.used = 0;
  g_tr.on = true;
  return REWY_OK;
}

REWY_API int rewy_trace_select(const char* stage) {
  if (stage && strlen(stage) >= sizeof(g_tr.only)) return fail(REWY_EINVAL, "trace stage name too long");
  snprintf(g_tr.only, sizeof(g_tr.only), "%s", stage ? stage : "");
  return REWY_OK;
}

REWY_API int rewy_trace_end(rewy_trace_entry* out, int cap) {
  g_tr.on = false;
  if (!out && cap > 0) return fail(REWY_EINVAL, "trace output is NULL");
  std::vector<rewy_trace_entry> agg;
  for (const TraceRec& r : g_tr.recs) {
    if (hipEventSynchronize(r.e1) != hipSuccess) return fail(REWY_EHIP, "trace synchronise");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess) return fail(REWY_EHIP, "trace elapsed");
    const std::string name = kernel_name(r);
    size_t i = 0;
    while (i < agg.size() && strcmp(agg[i].kernel, name.c_str()) != 0) ++i;
    if (i == agg.size()) {
      rewy_trace_entry e{};
      snprintf(e.kernel, sizeof(e.kernel), "%s", name.c_str());
      agg.push_back(e);
    }
    agg[i].total_ms += ms;
    agg[i].launches += 1;
  }
  g_tr.recs.clear();
  g_tr.used = 0;
  const int n = (int)std::min<size_t>(agg.size(), (size_t)std::max(cap, 0));
  for (int i = 0; i < n; ++i) out[i] = agg[i];
  return (int)agg.size();
}

REWY_API const char* rewy_status_string(int status) {
  switch (status) {
    case REWY_OK: return "REWY_OK";
    case REWY_EINVAL: return "REWY_EINVAL";
    case REWY_EUNSUPPORTED: return "REWY_EUNSUPPORTED";
    case REWY_EWORKSPACE: return "REWY_EWORKSPACE";
    case REWY_EHIP: return "REWY_EHIP";
    default: return "REWY_UNKNOWN";
  }
}

REWY_API const char* rewy_last_error(void) { return g_err; }
