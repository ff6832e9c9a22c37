/*
 * gdr_oracle.c -- plain fp64 CPU oracle for the gated delta-rule backward.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check and the benchmark's
 * CPU-baseline leg load this library. It shares no code, header, table or
 * helper with the HIP path, and the HIP path never calls it.
 *
 * What it computes (per sequence n and value head h, tokens t = 1..T_n):
 *   The recurrence is the one the "kernel_fun kda bwd_intra" page (module
 *   docstring) and the FlashQLA issue #30 page (fused_bwd.py, CONSUMER_S/A
 *   steps) both decompose chunkwise:
 *     a_t = 2^{g_t}                       (per channel, or one scalar per head)
 *     P_t = Diag(a_t) S_{t-1}
 *     e_t = v_t - P_t^T k_t
 *     S_t = P_t + beta_t k_t e_t^T        (= (I - b k k^T) Diag(2^g) S + b k v^T)
 *     o_t = scale * S_t^T q_t
 *   with S_0 = h0 and the scalar objective
 *     L = sum_t <do_t, o_t> + <dht, S_T>_F.
 *   The chunked form on the pages is an exact rewrite of this recurrence, so the
 *   oracle computes the plain gradient of L token by token, with no chunking.
 *
 * Reverse recurrence (derived by hand from the forward above; Lam = dL/dS_t):
 *   Lam = dht
 *   for t = T..1:
 *     Lam += scale q_t do_t^T               (o_t reads S_t)
 *     dq_t  = scale S_t do_t
 *     db_t  = k_t^T Lam e_t
 *     de    = beta_t Lam^T k_t
 *     dk_t  = beta_t Lam e_t - P_t de
 *     dv_t  = de
 *     dP    = Lam - k_t de^T
 *     dg_t  = ln2 * a_t (.) rowsum_v(dP (.) S_{t-1})   (scalar gate: full sum)
 *     Lam   = Diag(a_t) dP
 *   dh0 = Lam
 *
 * Gates are raw per-token log2 values (not cumulated); dg is the gradient with
 * respect to those raw values. GQA: value head h reads q/k head h / (H/Hg), and
 * dq/dk are summed over the value heads of a group. Varlen: every sequence
 * restarts from its own h0 and ends at its own dht.
 *
 * Memory: S is checkpointed every `seg` tokens (about sqrt(T_n)) and recomputed
 * inside each segment on the way back.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_LN2 0.69314718055994530942

typedef struct {
    int64_t B, T;
    int32_t H, Hg, K, V, gate_scalar, n_seqs, chunk;
    double scale;
    const int32_t *cu;
    const double *q, *k, *v, *g, *beta, *h0, *do_, *dht;
    double *dq, *dk, *dv, *dg, *db, *dh0, *o, *ht, *h_chunks, *dh_chunks;
    const int64_t *chunk_off; /* per sequence, first global chunk index */
} oracle_args;

/* token-major offsets into [B,T,X,D] tensors */
static inline int64_t tok_off(const oracle_args *a, int64_t b, int64_t t, int64_t nx,
                              int64_t x, int64_t d) {
    return ((b * a->T + t) * nx + x) * d;
}

/* a_t for value head h at (b, t): K values (broadcast for the scalar gate) */
static void decay(const oracle_args *a, int64_t b, int64_t t, int32_t h, double *out) {
    if (a->gate_scalar) {
        double x = exp2(a->g[(b * a->T + t) * a->H + h]);
        for (int d = 0; d < a->K; ++d) out[d] = x;
    } else {
        const double *gp = a->g + tok_off(a, b, t, a->H, h, a->K);
        for (int d = 0; d < a->K; ++d) out[d] = exp2(gp[d]);
    }
}

/* One forward step: S (K x V) is S_{t-1} on entry and S_t on exit.
   P (K x V) and e (V) receive P_t and e_t. */
static void fwd_step(const oracle_args *a, int64_t b, int64_t t, int32_t h, double *S,
                     double *P, double *e, double *at) {
    const int K = a->K, V = a->V;
    const int32_t hk = h / (a->H / a->Hg);
    const double *kt = a->k + tok_off(a, b, t, a->Hg, hk, K);
    const double *vt = a->v + tok_off(a, b, t, a->H, h, V);
    const double bt = a->beta[(b * a->T + t) * a->H + h];
    decay(a, b, t, h, at);
    for (int i = 0; i < K; ++i)
        for (int j = 0; j < V; ++j) P[i * V + j] = at[i] * S[i * V + j];
    for (int j = 0; j < V; ++j) {
        double s = 0.0;
        for (int i = 0; i < K; ++i) s += P[i * V + j] * kt[i];
        e[j] = vt[j] - s;
    }
    for (int i = 0; i < K; ++i)
        for (int j = 0; j < V; ++j) S[i * V + j] = P[i * V + j] + bt * kt[i] * e[j];
}

static void readout(const oracle_args *a, int64_t b, int64_t t, int32_t h, const double *S) {
    const int K = a->K, V = a->V;
    const int32_t hk = h / (a->H / a->Hg);
    const double *qt = a->q + tok_off(a, b, t, a->Hg, hk, K);
    double *ot = a->o + tok_off(a, b, t, a->H, h, V);
    for (int j = 0; j < V; ++j) {
        double s = 0.0;
        for (int i = 0; i < K; ++i) s += S[i * V + j] * qt[i];
        ot[j] = a->scale * s;
    }
}

/* Full forward + reverse for one (sequence n, value head h). */
static int run_head(const oracle_args *a, int32_t n, int32_t h) {
    const int K = a->K, V = a->V;
    const int64_t KV = (int64_t)K * V;
    int64_t b, t0, len;
    if (a->cu) {
        b = 0;
        t0 = a->cu[n];
        len = (int64_t)a->cu[n + 1] - a->cu[n];
    } else {
        b = n;
        t0 = 0;
        len = a->T;
    }
    const int32_t hk = h / (a->H / a->Hg);
    const int want_bwd = a->dq != NULL;
    int64_t seg = 1;
    while (seg * seg < len) ++seg;
    const int64_t nseg = len > 0 ? (len + seg - 1) / seg : 0;

    double *S = calloc(KV, sizeof(double));
    double *P = malloc(KV * sizeof(double));
    double *dP = malloc(KV * sizeof(double));
    double *Lam = malloc(KV * sizeof(double));
    double *e = malloc(V * sizeof(double));
    double *de = malloc(V * sizeof(double));
    double *at = malloc(K * sizeof(double));
    double *lame = malloc(K * sizeof(double));
    double *ck = malloc((size_t)(nseg > 0 ? nseg : 1) * KV * sizeof(double));
    double *sb = malloc((size_t)seg * KV * sizeof(double));
    if (!S || !P || !dP || !Lam || !e || !de || !at || !lame || !ck || !sb) {
        free(S); free(P); free(dP); free(Lam); free(e); free(de); free(at);
        free(lame); free(ck); free(sb);
        return -1;
    }
    const int64_t sh = ((int64_t)n * a->H + h) * KV; /* [N,H,K,V] offset */
    if (a->h0) memcpy(S, a->h0 + sh, KV * sizeof(double));

    /* forward: checkpoints, optional o / ht / per-chunk states */
    for (int64_t i = 0; i < len; ++i) {
        if (i % seg == 0) memcpy(ck + (i / seg) * KV, S, KV * sizeof(double));
        if (a->h_chunks && i % a->chunk == 0) {
            int64_t c = a->chunk_off[n] + i / a->chunk;
            memcpy(a->h_chunks + (c * a->H + h) * KV, S, KV * sizeof(double));
        }
        fwd_step(a, b, t0 + i, h, S, P, e, at);
        if (a->o) readout(a, b, t0 + i, h, S);
    }
    if (a->ht) memcpy(a->ht + sh, S, KV * sizeof(double));

    if (want_bwd) {
        if (a->dht) memcpy(Lam, a->dht + sh, KV * sizeof(double));
        else memset(Lam, 0, KV * sizeof(double));
        for (int64_t si = nseg - 1; si >= 0; --si) {
            const int64_t i0 = si * seg;
            const int64_t i1 = (i0 + seg < len) ? i0 + seg : len;
            /* recompute S_{t-1} for every token of the segment */
            memcpy(S, ck + si * KV, KV * sizeof(double));
            for (int64_t i = i0; i < i1; ++i) {
                memcpy(sb + (i - i0) * KV, S, KV * sizeof(double));
                fwd_step(a, b, t0 + i, h, S, P, e, at);
            }
            for (int64_t i = i1 - 1; i >= i0; --i) {
                const int64_t t = t0 + i;
                const double *Sprev = sb + (i - i0) * KV;
                /* rebuild P_t, e_t, S_t from S_{t-1} */
                memcpy(S, Sprev, KV * sizeof(double));
                fwd_step(a, b, t, h, S, P, e, at);
                /* dL/dS_t at the end of chunk c (before adding o_t's term) */
                if (a->dh_chunks && ((i + 1) % a->chunk == 0 || i + 1 == len)) {
                    int64_t c = a->chunk_off[n] + i / a->chunk;
                    memcpy(a->dh_chunks + (c * a->H + h) * KV, Lam, KV * sizeof(double));
                }
                const double *qt = a->q + tok_off(a, b, t, a->Hg, hk, K);
                const double *kt = a->k + tok_off(a, b, t, a->Hg, hk, K);
                const double *dot = a->do_ + tok_off(a, b, t, a->H, h, V);
                const double bt = a->beta[(b * a->T + t) * a->H + h];
                double *dqt = a->dq + tok_off(a, b, t, a->Hg, hk, K);
                double *dkt = a->dk + tok_off(a, b, t, a->Hg, hk, K);
                double *dvt = a->dv + tok_off(a, b, t, a->H, h, V);
                /* Lam += scale q do^T ; dq = scale S_t do */
                for (int r = 0; r < K; ++r) {
                    double s = 0.0;
                    for (int c = 0; c < V; ++c) {
                        Lam[r * V + c] += a->scale * qt[r] * dot[c];
                        s += S[r * V + c] * dot[c];
                    }
                    dqt[r] += a->scale * s;
                }
                /* Lam e, db, de */
                double dbt = 0.0;
                for (int r = 0; r < K; ++r) {
                    double s = 0.0;
                    for (int c = 0; c < V; ++c) s += Lam[r * V + c] * e[c];
                    lame[r] = s;
                    dbt += kt[r] * s;
                }
                for (int c = 0; c < V; ++c) {
                    double s = 0.0;
                    for (int r = 0; r < K; ++r) s += Lam[r * V + c] * kt[r];
                    de[c] = bt * s;
                    dvt[c] = de[c];
                }
                a->db[(b * a->T + t) * a->H + h] = dbt;
                /* dk = beta Lam e - P de */
                for (int r = 0; r < K; ++r) {
                    double s = 0.0;
                    for (int c = 0; c < V; ++c) s += P[r * V + c] * de[c];
                    dkt[r] += bt * lame[r] - s;
                }
                /* dP = Lam - k de^T ; dg ; Lam = Diag(a) dP */
                double gs = 0.0;
                for (int r = 0; r < K; ++r) {
                    double s = 0.0;
                    for (int c = 0; c < V; ++c) {
                        double x = Lam[r * V + c] - kt[r] * de[c];
                        dP[r * V + c] = x;
                        s += x * Sprev[r * V + c];
                    }
                    if (a->gate_scalar) gs += at[r] * s;
                    else a->dg[tok_off(a, b, t, a->H, h, K) + r] = ORACLE_LN2 * at[r] * s;
                    for (int c = 0; c < V; ++c) Lam[r * V + c] = at[r] * dP[r * V + c];
                }
                if (a->gate_scalar) a->dg[(b * a->T + t) * a->H + h] = ORACLE_LN2 * gs;
            }
        }
        memcpy(a->dh0 + sh, Lam, KV * sizeof(double));
    }
    free(S); free(P); free(dP); free(Lam); free(e); free(de); free(at);
    free(lame); free(ck); free(sb);
    return 0;
}

/*
 * Layouts (all contiguous row-major, fp64):
 *   q, k, dq, dk [B,T,Hg,K]; v, do, dv, o [B,T,H,V];
 *   g, dg [B,T,H,K] (per-channel) or [B,T,H] (scalar); beta, db [B,T,H];
 *   h0, dht, dh0, ht [N,H,K,V] with N = n_seqs (varlen) or B.
 * cu_seqlens: host int32 [n_seqs+1] (then B must be 1) or NULL.
 * h0 / dht NULL mean zero. Pass dq == NULL for a forward-only run (then dk,
 * dv, dg, db, dh0 are ignored). o, ht may be NULL.
 * h_chunks / dh_chunks (may be NULL): [total_chunks, H, K, V], the state before
 * each chunk of `chunk` tokens and dL/dS after each chunk's last token, global
 * chunk index = sequences in order, chunks in order.
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int gdr_oracle_run(int64_t B, int64_t T, int32_t H, int32_t Hg, int32_t K, int32_t V,
                   int32_t gate_scalar, double scale, const int32_t *cu_seqlens,
                   int32_t n_seqs, const double *q, const double *k, const double *v,
                   const double *g, const double *beta, const double *h0,
                   const double *do_, const double *dht, double *dq, double *dk,
                   double *dv, double *dg, double *db, double *dh0, double *o,
                   double *ht, int32_t chunk, double *h_chunks, double *dh_chunks) {
    if (B <= 0 || T < 0 || H <= 0 || Hg <= 0 || K <= 0 || V <= 0 || H % Hg) return -1;
    if (cu_seqlens && (B != 1 || n_seqs <= 0)) return -1;
    if ((h_chunks || dh_chunks) && chunk <= 0) return -1;
    oracle_args a = {0};
    a.B = B; a.T = T; a.H = H; a.Hg = Hg; a.K = K; a.V = V;
    a.gate_scalar = gate_scalar; a.scale = scale; a.cu = cu_seqlens;
    a.n_seqs = cu_seqlens ? n_seqs : (int32_t)B;
    a.chunk = chunk;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.h0 = h0; a.do_ = do_; a.dht = dht;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.db = db; a.dh0 = dh0;
    a.o = o; a.ht = ht; a.h_chunks = h_chunks; a.dh_chunks = dh_chunks;
    const int32_t N = a.n_seqs;
    int64_t *coff = malloc(((size_t)N + 1) * sizeof(int64_t));
    if (!coff) return -1;
    coff[0] = 0;
    for (int32_t n = 0; n < N; ++n) {
        int64_t len = cu_seqlens ? (int64_t)cu_seqlens[n + 1] - cu_seqlens[n] : T;
        if (len < 0) { free(coff); return -1; }
        coff[n + 1] = coff[n] + (chunk > 0 ? (len + chunk - 1) / chunk : 0);
    }
    a.chunk_off = coff;
    if (dq) {
        memset(dq, 0, (size_t)(B * T * Hg * K) * sizeof(double));
        memset(dk, 0, (size_t)(B * T * Hg * K) * sizeof(double));
    }
    const int32_t G = H / Hg;
    int err = 0;
    /* one task per (sequence, q/k head): the task owns every value head of the
       group, so the group sum of dq/dk needs no synchronisation */
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t task = 0; task < (int64_t)N * Hg; ++task) {
        int32_t n = (int32_t)(task / Hg), hk = (int32_t)(task % Hg);
        for (int32_t j = 0; j < G; ++j) err |= run_head(&a, n, hk * G + j);
    }
    free(coff);
    return err ? -1 : 0;
}

int gdr_oracle_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
