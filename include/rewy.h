/*
 * rewy.h -- C ABI of the MI355X (gfx950) chunkwise gated delta-rule operator
 * with the ReWY backward.  librewy.so exports exactly the functions below.
 *
 * What the operator computes (ReWY paper, "Background / Delta-rule operators",
 * Table 1; KDA blog, section 4 boxed equations).  For every sequence n and head
 * h, with the state S in [K,V] layout (fp32), tokens t in order:
 *     S~  = diag(exp g_t) S                 decay (g_t natural log, <= 0 expected)
 *     r_t = beta_t (v_t - S~^T k_t)         predict from the decayed state, correct
 *     S   = S~ + k_t r_t^T                  rank-one write
 *     o_t = S^T (scale * q_t)               read after the write
 * Gate kinds (Table 1): NONE = DeltaNet (g = 0), SCALAR = Gated DeltaNet (one g
 * per token and head), VECTOR = KDA (one g per token, head and key channel).
 * rewy_fwd returns o and the final states; rewy_bwd returns the gradients of
 * l = <dO, o> + <dht, ht> with respect to q, k, v, g, beta and h0, computed in
 * the chunkwise WY form (Appendix A) with the ReWY local pullback (Algorithm 1:
 * P = A^T Rbar, D = -tril_strict(P R^T)), matrix-intra contractions for the
 * vector gate (section 3.3) and the Gram-free reduction for the scalar gate
 * (section 3.4), in the complete reverse order of Appendix 10.
 *
 * Layouts (all row-major, contiguous, token-major as in the pages' code):
 *   q, k            [B, T, H, K]   dtype
 *   v, o, dO        [B, T, H, V]   dtype
 *   g               NULL (NONE) | [B, T, H] fp32 (SCALAR) | [B, T, H, K] fp32 (VECTOR)
 *   beta, dbeta     [B, T, H]      beta_dtype
 *   h0, ht, dht, dh0 [N, H, K, V]  fp32
 *   dq, dk [B,T,H,K] dtype; dv [B,T,H,V] dtype; dg same shape as g, fp32.
 * With cu_seqlens (device int32, N+1 ascending offsets, [0] = 0, [N] = T) the
 * batch must be B = 1 and the N sequences are packed along T; chunks of 64
 * tokens restart at every sequence start and the last chunk of a sequence may
 * be partial.  Without it, N = B and every batch row is one sequence.
 * cu_seqlens is validated on the host only when its host copy is given; the
 * kernels clamp the device array to [0, T] and to non-decreasing offsets, so
 * a malformed array gives wrong results but never an access outside the
 * caller's buffers.  Workspace and saved layouts are sized by the bound
 * ceil(T / 64) + N chunk slots and do not depend on the host copy.
 *
 * Ownership and execution.  Every pointer except desc and cu_seqlens_host is a
 * device pointer owned by the caller.  The library never allocates device
 * memory and keeps no state between calls: scratch comes from the caller's
 * workspace (size from rewy_workspace_bytes) and, for the save-all policy,
 * forward intermediates go to the caller's `saved` buffer (size from
 * rewy_saved_bytes), which must stay unchanged, together with the inputs,
 * between rewy_fwd and rewy_bwd.  All work is enqueued on `stream` (a
 * hipStream_t; NULL = the null stream) and the call returns without waiting.
 * Outputs are overwritten, never accumulated into.  Calls on distinct streams
 * with distinct buffers may run concurrently.  No atomics: results are
 * bitwise reproducible for a given shape.
 *
 * Errors.  Arguments are checked on the host before anything is enqueued; a
 * failed check returns a negative rewy_status and has no side effect.
 * rewy_last_error() gives a thread-local text for the last failure.  Faults
 * inside kernels surface asynchronously at the caller's next synchronisation.
 */
#ifndef REWY_H
#define REWY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    REWY_OK = 0,
    REWY_EINVAL = -1,       /* malformed argument (null pointer, bad shape, bad cu_seqlens) */
    REWY_EUNSUPPORTED = -2, /* valid request the library does not implement (K, V not in {32,64,128}) */
    REWY_EWORKSPACE = -3,   /* workspace or saved buffer too small or misaligned */
    REWY_EHIP = -4          /* a HIP launch or copy reported an error */
} rewy_status;

typedef enum { REWY_GATE_NONE = 0, REWY_GATE_SCALAR = 1, REWY_GATE_VECTOR = 2 } rewy_gate;
typedef enum { REWY_BF16 = 0, REWY_F32 = 1 } rewy_dtype;
/* Saving policies of the ReWY paper (section 4.1): RECOMPUTE re-runs the forward
 * chunk stages inside rewy_bwd; SAVE keeps them from rewy_fwd in `saved`. */
typedef enum { REWY_RECOMPUTE = 0, REWY_SAVE = 1 } rewy_policy;

typedef struct {
    int32_t B, T, H, K, V;          /* K, V in {32, 64, 128} */
    int32_t N;                      /* sequences: B without cu_seqlens, else len(cu_seqlens)-1 */
    const int32_t *cu_seqlens;      /* device [N+1] or NULL */
    const int32_t *cu_seqlens_host; /* optional host copy of cu_seqlens, validated if given */
    int32_t dtype;                  /* rewy_dtype of q, k, v, o, dO, dq, dk, dv */
    int32_t beta_dtype;             /* rewy_dtype of beta and dbeta */
    int32_t gate;                   /* rewy_gate */
    int32_t policy;                 /* rewy_policy */
    float scale;                    /* query scale, usually K^-1/2 */
} rewy_desc;

/* Bytes of device workspace a call needs: phase 0 = rewy_fwd (and the other
 * forwards), 1 = rewy_bwd and rewy_bwd_gdn2, 2 = rewy_bwd_kda_gate (phase 1
 * plus the per-chunk partial sums of the gate parameters' gradients; needs
 * gate == VECTOR).  Returns 0 for an invalid descriptor or phase (see
 * rewy_last_error). */
size_t rewy_workspace_bytes(const rewy_desc *d, int phase);

/* Bytes of the `saved` buffer for policy SAVE (0 for RECOMPUTE). */
size_t rewy_saved_bytes(const rewy_desc *d);

/* Forward.  h0 may be NULL (zero initial state); ht may be NULL (final state
 * not returned); saved must be non-NULL for policy SAVE.  workspace must be
 * 256-byte aligned and at least rewy_workspace_bytes(d, 0) long. */
int rewy_fwd(const rewy_desc *d, const void *q, const void *k, const void *v,
             const float *g, const void *beta, const float *h0,
             void *o, float *ht, void *saved,
             void *workspace, size_t ws_bytes, void *stream);

/* Backward.  dht may be NULL (zero terminal adjoint).  dg must be NULL exactly
 * when gate == NONE.  dh0 must be non-NULL when h0 is non-NULL and may be
 * non-NULL otherwise (then it is the gradient for a zero initial state).
 * For policy SAVE, `saved` must hold what rewy_fwd wrote for the same inputs;
 * for RECOMPUTE it is ignored. */
int rewy_bwd(const rewy_desc *d, const void *q, const void *k, const void *v,
             const float *g, const void *beta, const float *h0,
             const void *dO, const float *dht, const void *saved,
             void *dq, void *dk, void *dv, float *dg, void *dbeta, float *dh0,
             void *workspace, size_t ws_bytes, void *stream);

/* Forward without any allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Computes exactly what rewy_fwd computes (the same kernels
 * in the same order: bitwise the same o, ht and saved buffer), with the
 * workspace taken from a device array of REWY_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends.  The caller
 * still passes every input and output (and, for policy SAVE, the saved
 * buffer).  A problem whose rewy_workspace_bytes(d, 0) exceeds that size
 * returns REWY_EWORKSPACE before anything is enqueued; at K = V = 128 in bf16
 * the forward needs about 1.2 KB per token and head, so the scratch serves up
 * to about 110 k token-heads (e.g. T = 3.5 k at H = 32).  The stream must
 * belong to the current device.  Every call on one GPU uses the same scratch:
 * calls that overlap in time on one GPU (different streams, or threads)
 * race and must be serialised by the caller.  Nothing in the scratch needs
 * clearing between calls: every element a call reads, it has written first. */
#define REWY_NOALLOC_SCRATCH_BYTES (128u << 20)
int rewy_fwd_noalloc(const rewy_desc *d, const void *q, const void *k, const void *v,
                     const float *g, const void *beta, const float *h0,
                     void *o, float *ht, void *saved, void *stream);

/* The erase/write form (ReWY paper Table 1, GDN2 row; GDN2 spec section 2):
 * independent erase and write vector gates in place of the shared beta,
 *     r_t = w_t * v_t - S~^T (b_t * k_t),   S = S~ + k_t r_t^T,
 * so that E = b gamma K and Z = w V in the chunk form.  b is [B,T,H,K] and w
 * [B,T,H,V], both in the feature dtype (beta_dtype must equal dtype, else
 * REWY_EUNSUPPORTED); with b = w = beta the result is rewy_fwd's.  Everything
 * else (descriptor, workspace and saved sizes, ownership, errors) is as for
 * rewy_fwd / rewy_bwd; the backward returns db [B,T,H,K] and dw [B,T,H,V] in
 * the feature dtype, element by element, in place of dbeta. */
int rewy_fwd_gdn2(const rewy_desc *d, const void *q, const void *k, const void *v,
                  const float *g, const void *b, const void *w, const float *h0,
                  void *o, float *ht, void *saved,
                  void *workspace, size_t ws_bytes, void *stream);
int rewy_bwd_gdn2(const rewy_desc *d, const void *q, const void *k, const void *v,
                  const float *g, const void *b, const void *w, const float *h0,
                  const void *dO, const float *dht, const void *saved,
                  void *dq, void *dk, void *dv, float *dg, void *db, void *dw, float *dh0,
                  void *workspace, size_t ws_bytes, void *stream);

/* The vector gate formed inside the kernels from its pre-activation (GDN2
 * spec section 4.4, the KDA gate, and section 3 for the bounded form; KDA
 * blog section 6 for the operator).  With z = x[t,h,k] + dt_bias[h,k]:
 *     lower_bound == 0:          g = -exp(A_log[h]) * softplus(z)
 *     -5 <= lower_bound < 0:     g = lower_bound * sigmoid(exp(A_log[h]) * z)
 * (any other lower_bound, NaN included, returns REWY_EINVAL), so the fp32
 * log-decay g [B,T,H,K] is never read from or written to memory.
 * gate must be VECTOR.  x is [B,T,H,K] in the feature dtype, 16-byte aligned;
 * A_log is fp32 [H]; dt_bias is fp32 [H,K], 16-byte aligned.  The result is
 * rewy_fwd's / rewy_bwd's with g formed by the formula above in fp32.  The
 * backward returns, in place of dg, dx [B,T,H,K] (feature dtype) and the fp32
 * parameter gradients dA_log [H] and ddt_bias [H,K], summed over every token
 * of every sequence and overwritten (not accumulated into); its workspace is
 * rewy_workspace_bytes(d, 2).  The sums over chunks are taken in a fixed
 * order, so repeated calls give identical results.  Everything else
 * (descriptor, saved buffer, ownership, errors) is as for rewy_fwd / rewy_bwd;
 * the saved buffer of rewy_fwd_kda_gate serves rewy_bwd_kda_gate only. */
int rewy_fwd_kda_gate(const rewy_desc *d, const void *q, const void *k, const void *v,
                      const void *x, const float *a_log, const float *dt_bias, float lower_bound,
                      const void *beta, const float *h0, void *o, float *ht, void *saved,
                      void *workspace, size_t ws_bytes, void *stream);
int rewy_bwd_kda_gate(const rewy_desc *d, const void *q, const void *k, const void *v,
                      const void *x, const float *a_log, const float *dt_bias, float lower_bound,
                      const void *beta, const float *h0,
                      const void *dO, const float *dht, const void *saved,
                      void *dq, void *dk, void *dv, void *dx, float *da_log, float *ddt_bias,
                      void *dbeta, float *dh0,
                      void *workspace, size_t ws_bytes, void *stream);

/* Token-serial forward for decoding (the pages' fused recurrent form of the
 * same recurrence: ReWY paper, Background / Delta-rule operators; KDA blog
 * section 4): o_t = S_t^T (s q_t) with the state updated one token at a time,
 * decay -> predict -> correct -> write -> read.  Same descriptor and tensors as
 * rewy_fwd (the policy is ignored) and no workspace or saved buffer: the
 * fp32 state of each (sequence, head) stays on chip from h0 to ht.  h0 and ht
 * may be NULL (zero initial state; final state not returned).  Meant for short
 * continuations, e.g. one new token per sequence with h0/ht carried between
 * calls; long prompts are faster through rewy_fwd.  Argument errors return a
 * negative status before anything is enqueued. */
int rewy_recurrent_fwd(const rewy_desc *d, const void *q, const void *k, const void *v,
                       const float *g, const void *beta, const float *h0,
                       void *o, float *ht, void *stream);

/* Token-serial forward of the erase/write form (GDN2 spec section 3, the
 * recurrent kernel; ReWY paper Table 1, GDN2 row): r_t = w_t * v_t -
 * S~^T (b_t * k_t), S = S~ + k_t r_t^T, with b [B,T,H,K] and w [B,T,H,V] in the
 * feature dtype (beta_dtype must equal dtype, else REWY_EUNSUPPORTED).  All
 * else as rewy_recurrent_fwd; with b = w = beta it computes the same as it. */
int rewy_recurrent_fwd_gdn2(const rewy_desc *d, const void *q, const void *k, const void *v,
                            const float *g, const void *b, const void *w, const float *h0,
                            void *o, float *ht, void *stream);

/* Schedule of the chunk backward (ReWY paper, "Execution and numerical
 * precision", joint and separate consumers).  JOINT (the default): one kernel
 * per chunk-head forms the shared sensitivity P = A^T Rbar and D =
 * -tril_strict(P R^T) and consumes them on chip.  SEPARATE: a producer kernel
 * writes P, D and the write part of dbeta to the workspace and a consumer
 * kernel reads them back; the results are bitwise those of JOINT, the
 * workspace (rewy_workspace_bytes phase 1) grows by about 580 B per token and
 * head at K = V = 128 in bf16.  Applies to later rewy_bwd calls from every
 * thread (the erase/write form and the gate formed in the kernels always run
 * JOINT); workspace sizes follow the schedule in force when they are queried,
 * so query them after setting it.  Returns the previous schedule; a negative
 * argument only returns the current one; an unknown schedule returns
 * REWY_EINVAL and changes nothing. */
typedef enum { REWY_SCHEDULE_JOINT = 0, REWY_SCHEDULE_SEPARATE = 1 } rewy_schedule;
int rewy_bwd_schedule(int schedule);

/* Per-kernel timing (a tracing aid: device events, as in the ReWY paper's timing
 * protocol).  After rewy_trace_begin(), calls made by this thread
 * record a HIP event pair on the call's stream around every kernel they
 * enqueue.  rewy_trace_end() waits for the recorded events, stops recording and
 * fills at most `cap` entries, one per launched instantiation, named by its
 * symbol with every template argument exactly as rocprofv3 reports it
 * (demangled where the host's demangler can, e.g. "rewy::k_chunk_table(rewy::Args)",
 * else mangled, e.g. "_ZN4rewy10k_fwd_prepIDF16bLi128ELi128ELi13EEEvNS_4ArgsE"
 * for the bfloat16 instantiations), with the summed
 * elapsed milliseconds and the launch count; it returns the number of
 * entries, or a negative rewy_status.  Not for use under graph capture.
 * Events are created once per thread and reused. */
typedef struct {
    char kernel[96];
    double total_ms;
    int launches;
} rewy_trace_entry;

int rewy_trace_begin(void);
int rewy_trace_end(rewy_trace_entry *out, int cap);

/* Restricts this thread's trace to the launches of one kernel, named by its
 * template name without arguments ("k_fwd_prep", "k_scans", ...; every
 * instantiation of it), so that a timed run pays for
 * one event pair per launch of that kernel only.  NULL (the default) traces
 * every launch.  Applies from the next call; the name is copied.  Returns
 * REWY_OK, or REWY_EINVAL for a name longer than 63 characters. */
int rewy_trace_select(const char *stage);

/* Name of a rewy_status value. */
const char *rewy_status_string(int status);

/* Thread-local description of the last failed call on this thread. */
const char *rewy_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* REWY_H */
