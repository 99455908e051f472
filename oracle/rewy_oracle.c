/*
 * FP64 CPU oracle for the chunkwise gated delta rule -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain definition of the operator: the token-by-token
 * recurrence and its exact reverse-mode derivative, evaluated in double
 * precision, one (sequence, head) pair per OpenMP thread.  It knows nothing
 * about chunks, WY factors, MFMA tiles or the HIP library and shares no code
 * with them.  Only the test-suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load it.
 *
 * Recurrence (ReWY paper, "Background / Delta-rule operators" and Table 1;
 * KDA blog, section 4 boxed equations and the five-line [K,V] reference loop).
 * Per token t, with the state S in [K,V] layout (key rows, value columns):
 *     a_t   = exp(g_t)                      decay: vector (KDA), scalar (GDN), 1 (DeltaNet)
 *     S~    = diag(a_t) S_{t-1}             forget
 *     r_t   = w_t * v_t - S~^T (b_t * k_t)  predict from the gated key, correct
 *     S_t   = S~ + k_t r_t^T                rank-one write along k_t
 *     o_t   = S_t^T (scale * q_t)           read, including the current write
 * The erase gate b_t (length K) and the write gate w_t (length V) are kept
 * separate so that special cases can be reached (b = 0, w = 1 is plain
 * additive linear attention; the public operator passes b = w = beta * 1).
 *
 * Reverse mode.  Loss l = sum_t <dO_t, o_t> + <dS_T, S_T>.  Walking t down,
 * Sig is the running adjoint of S_t:
 *     Sig   += (scale q_t) dO_t^T
 *     dq_t   = scale * S_t dO_t
 *     dk_t   = Sig r_t
 *     dr     = Sig^T k_t
 *     u      = S~ dr
 *     dv_t   = w_t * dr ;   dw_t = v_t * dr
 *     dk_t  += -b_t * u ;   db_t = -k_t * u        (no division by beta anywhere)
 *     Sig~   = Sig - (b_t * k_t) dr^T              adjoint of S~
 *     da_k   = sum_v Sig~_kv S_{t-1,kv}
 *     dg_t   = da * a_t   (vector) ; sum_k da_k a_k (scalar)
 *     Sig    = diag(a_t) Sig~
 * dS0 = Sig after token 0.  g is the natural-log decay, so no ln 2 factor
 * appears.  States are recomputed in the reverse sweep from checkpoints kept
 * every CKPT tokens, so memory per thread is about (T/CKPT + CKPT) K V doubles.
 *
 * Layouts (row-major, token-major as in the operator):
 *   q, k : [T_total, H, K]      v, o, dO : [T_total, H, V]
 *   g    : [T_total, H, K] (gate_kind 2) or [T_total, H] (gate_kind 1) or NULL (0)
 *   b    : [T_total, H, K]      w        : [T_total, H, V]
 *   h0, ht, dht, dh0 : [N, H, K, V]
 *   cu   : N+1 ascending token offsets; sequence n spans [cu[n], cu[n+1]).
 * Gradients: dq, dk, db : [T_total,H,K]; dv, dw : [T_total,H,V];
 *   dg : same shape as g.  All outputs are overwritten.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define CKPT 64

typedef struct {
    int64_t N, H, K, V;
    const int64_t *cu;
    const double *q, *k, *v, *g, *b, *w, *h0;
    int gate_kind;
    double scale;
} prob_t;

/* decay factors a[0..K) for token t, head h */
static void decay(const prob_t *P, int64_t t, int64_t h, double *a) {
    int64_t K = P->K;
    if (P->gate_kind == 2) {
        const double *gt = P->g + (t * P->H + h) * K;
        for (int64_t i = 0; i < K; i++) a[i] = exp(gt[i]);
    } else if (P->gate_kind == 1) {
        double e = exp(P->g[t * P->H + h]);
        for (int64_t i = 0; i < K; i++) a[i] = e;
    } else {
        for (int64_t i = 0; i < K; i++) a[i] = 1.0;
    }
}

/* One forward token step: S (in: S_{t-1}, out: S_t), writes r and o if non-NULL. */
static void step(const prob_t *P, int64_t t, int64_t h, double *S, double *a,
                 double *bk, double *r, double *o) {
    int64_t K = P->K, V = P->V, H = P->H;
    const double *kt = P->k + (t * H + h) * K;
    const double *vt = P->v + (t * H + h) * V;
    const double *bt = P->b + (t * H + h) * K;
    const double *wt = P->w + (t * H + h) * V;
    decay(P, t, h, a);
    for (int64_t i = 0; i < K; i++) {
        double ai = a[i];
        double *row = S + i * V;
        for (int64_t j = 0; j < V; j++) row[j] *= ai;
        bk[i] = bt[i] * kt[i];
    }
    for (int64_t j = 0; j < V; j++) r[j] = wt[j] * vt[j];
    for (int64_t i = 0; i < K; i++) {
        double c = bk[i];
        const double *row = S + i * V;
        for (int64_t j = 0; j < V; j++) r[j] -= c * row[j];
    }
    for (int64_t i = 0; i < K; i++) {
        double c = kt[i];
        double *row = S + i * V;
        for (int64_t j = 0; j < V; j++) row[j] += c * r[j];
    }
    if (o) {
        const double *qt = P->q + (t * H + h) * K;
        for (int64_t j = 0; j < V; j++) o[j] = 0.0;
        for (int64_t i = 0; i < K; i++) {
            double c = P->scale * qt[i];
            const double *row = S + i * V;
            for (int64_t j = 0; j < V; j++) o[j] += c * row[j];
        }
    }
}

static void load_h0(const prob_t *P, int64_t n, int64_t h, double *S) {
    int64_t KV = P->K * P->V;
    if (P->h0) memcpy(S, P->h0 + (n * P->H + h) * KV, (size_t)KV * sizeof(double));
    else memset(S, 0, (size_t)KV * sizeof(double));
}

int rewy_oracle_fwd(int64_t N, const int64_t *cu, int64_t H, int64_t K, int64_t V,
                    const double *q, const double *k, const double *v, const double *g,
                    int gate_kind, const double *b, const double *w, double scale,
                    const double *h0, double *o, double *ht, int nthreads) {
    prob_t P = {N, H, K, V, cu, q, k, v, g, b, w, h0, gate_kind, scale};
    int64_t units = N * H;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; u++) {
        int64_t n = u / H, h = u % H;
        double *S = (double *)malloc((size_t)(K * V + 2 * K + V) * sizeof(double));
        if (!S) { err = 1; continue; }
        double *a = S + K * V, *bk = a + K, *r = bk + K;
        load_h0(&P, n, h, S);
        for (int64_t t = cu[n]; t < cu[n + 1]; t++)
            step(&P, t, h, S, a, bk, r, o + (t * H + h) * V);
        if (ht) memcpy(ht + (n * H + h) * K * V, S, (size_t)(K * V) * sizeof(double));
        free(S);
    }
    return err ? -1 : 0;
}

int rewy_oracle_bwd(int64_t N, const int64_t *cu, int64_t H, int64_t K, int64_t V,
                    const double *q, const double *k, const double *v, const double *g,
                    int gate_kind, const double *b, const double *w, double scale,
                    const double *h0, const double *dO, const double *dht,
                    double *dq, double *dk, double *dv, double *dg, double *db,
                    double *dw, double *dh0, int nthreads) {
    prob_t P = {N, H, K, V, cu, q, k, v, g, b, w, h0, gate_kind, scale};
    int64_t units = N * H;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; u++) {
        int64_t n = u / H, h = u % H;
        int64_t bos = cu[n], eos = cu[n + 1], L = eos - bos;
        int64_t KV = K * V;
        int64_t nck = (L + CKPT - 1) / CKPT;
        /* checkpoints: state entering each CKPT-token segment */
        double *ck = (double *)malloc((size_t)((nck > 0 ? nck : 1) * KV) * sizeof(double));
        /* segment states S_{t-1} for each token of one segment, plus S_t of its last */
        double *seg = (double *)malloc((size_t)((CKPT + 1) * KV) * sizeof(double));
        double *Sig = (double *)malloc((size_t)(KV + 4 * K + 3 * V) * sizeof(double));
        if (!ck || !seg || !Sig) { err = 1; free(ck); free(seg); free(Sig); continue; }
        double *a = Sig + KV, *bk = a + K, *uu = bk + K, *da = uu + K;
        double *r = da + K, *dr = r + V, *tmp = dr + V;
        /* forward sweep: checkpoints only */
        load_h0(&P, n, h, seg);
        for (int64_t c = 0; c < nck; c++) {
            memcpy(ck + c * KV, seg, (size_t)KV * sizeof(double));
            int64_t t1 = bos + (c + 1) * CKPT < eos ? bos + (c + 1) * CKPT : eos;
            for (int64_t t = bos + c * CKPT; t < t1; t++) step(&P, t, h, seg, a, bk, r, NULL);
        }
        /* terminal adjoint */
        if (dht) memcpy(Sig, dht + (n * H + h) * KV, (size_t)KV * sizeof(double));
        else memset(Sig, 0, (size_t)KV * sizeof(double));
        for (int64_t c = nck - 1; c >= 0; c--) {
            int64_t t0 = bos + c * CKPT;
            int64_t t1 = t0 + CKPT < eos ? t0 + CKPT : eos;
            int64_t m = t1 - t0;
            /* seg[j] = S_{t0+j-1} (state before token t0+j); seg[m] = S_{t1-1} */
            memcpy(seg, ck + c * KV, (size_t)KV * sizeof(double));
            for (int64_t j = 0; j < m; j++) {
                memcpy(seg + (j + 1) * KV, seg + j * KV, (size_t)KV * sizeof(double));
                step(&P, t0 + j, h, seg + (j + 1) * KV, a, bk, r, NULL);
            }
            for (int64_t j = m - 1; j >= 0; j--) {
                int64_t t = t0 + j;
                const double *Sprev = seg + j * KV;   /* S_{t-1} */
                const double *St = seg + (j + 1) * KV; /* S_t */
                const double *qt = q + (t * H + h) * K;
                const double *kt = k + (t * H + h) * K;
                const double *vt = v + (t * H + h) * V;
                const double *bt = b + (t * H + h) * K;
                const double *wt = w + (t * H + h) * V;
                const double *dot = dO + (t * H + h) * V;
                double *dqt = dq + (t * H + h) * K;
                double *dkt = dk + (t * H + h) * K;
                double *dbt = db + (t * H + h) * K;
                double *dvt = dv + (t * H + h) * V;
                double *dwt = dw + (t * H + h) * V;
                decay(&P, t, h, a);
                /* r_t = w v - (diag(a) S_{t-1})^T (b k) */
                for (int64_t jv = 0; jv < V; jv++) r[jv] = wt[jv] * vt[jv];
                for (int64_t i = 0; i < K; i++) {
                    double c = bt[i] * kt[i] * a[i];
                    const double *row = Sprev + i * V;
                    for (int64_t jv = 0; jv < V; jv++) r[jv] -= c * row[jv];
                }
                /* Sig += (s q) dO^T */
                for (int64_t i = 0; i < K; i++) {
                    double c = scale * qt[i];
                    double *row = Sig + i * V;
                    for (int64_t jv = 0; jv < V; jv++) row[jv] += c * dot[jv];
                }
                /* dq = s S_t dO */
                for (int64_t i = 0; i < K; i++) {
                    const double *row = St + i * V;
                    double acc = 0.0;
                    for (int64_t jv = 0; jv < V; jv++) acc += row[jv] * dot[jv];
                    dqt[i] = scale * acc;
                }
                /* dk = Sig r ; dr = Sig^T k */
                for (int64_t jv = 0; jv < V; jv++) dr[jv] = 0.0;
                for (int64_t i = 0; i < K; i++) {
                    const double *row = Sig + i * V;
                    double acc = 0.0, c = kt[i];
                    for (int64_t jv = 0; jv < V; jv++) {
                        acc += row[jv] * r[jv];
                        dr[jv] += c * row[jv];
                    }
                    dkt[i] = acc;
                }
                /* u = S~ dr, with S~ = diag(a) S_{t-1} */
                for (int64_t i = 0; i < K; i++) {
                    const double *row = Sprev + i * V;
                    double acc = 0.0;
                    for (int64_t jv = 0; jv < V; jv++) acc += row[jv] * dr[jv];
                    uu[i] = a[i] * acc;
                }
                for (int64_t jv = 0; jv < V; jv++) {
                    dvt[jv] = wt[jv] * dr[jv];
                    dwt[jv] = vt[jv] * dr[jv];
                }
                for (int64_t i = 0; i < K; i++) {
                    dkt[i] += -bt[i] * uu[i];
                    dbt[i] = -kt[i] * uu[i];
                }
                /* Sig~ = Sig - (b k) dr^T ; da = rowsum(Sig~ * S_{t-1}) ; Sig = diag(a) Sig~ */
                for (int64_t i = 0; i < K; i++) {
                    double c = bt[i] * kt[i];
                    double *row = Sig + i * V;
                    const double *prow = Sprev + i * V;
                    double acc = 0.0;
                    for (int64_t jv = 0; jv < V; jv++) {
                        double s = row[jv] - c * dr[jv];
                        acc += s * prow[jv];
                        row[jv] = a[i] * s;
                    }
                    da[i] = acc;
                }
                if (gate_kind == 2) {
                    double *dgt = dg + (t * H + h) * K;
                    for (int64_t i = 0; i < K; i++) dgt[i] = da[i] * a[i];
                } else if (gate_kind == 1) {
                    double acc = 0.0;
                    for (int64_t i = 0; i < K; i++) acc += da[i] * a[i];
                    dg[t * H + h] = acc;
                }
            }
        }
        if (dh0) memcpy(dh0 + (n * H + h) * KV, Sig, (size_t)KV * sizeof(double));
        (void)tmp;
        free(ck); free(seg); free(Sig);
    }
    return err ? -1 : 0;
}
