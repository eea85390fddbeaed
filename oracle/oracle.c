/*
 * Plain, slow fp64 CPU oracle for the ATMA global-layer hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file: only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code, header, table or helper with the HIP
 * library; it reads fp64 arrays (inputs widened exactly from whatever precision the
 * caller holds) and writes fp64 results.
 *
 * Sources (the ATMA paper, "ATMA: Long-Context Language Modeling via Polar Attention
 * and Gated-Delta Compression Memory", arXiv 2606.25156):
 *   - gated-delta memory: Section 3.3, the single displayed equation
 *         M_t = gamma_t M_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  r_t = M_t q_t.
 *     Here gamma_t is called alpha (per-token decay), M is called S (state, Dv x Dk),
 *     r is called o.
 *   - Polar attention: Section 3.2 equation (temperature t_i and null floor nu_i);
 *     Appendix C.2 (one softmax over the masked real-key logits plus one virtual
 *     null logit, channels computed from the resulting weights); Appendix A.2
 *     (direction c_i = s_i / max(||s_i||, eps), magnitude mu_i = tanh(beta log(1+m_eff)));
 *     Appendix C.3 and its Table 6 (streaming statistics M, L, Q2, S; n_eff = L^2/Q2,
 *     m_eff = n_eff L / Z, direction = normalize(S + p_null v_null)).
 *
 * Readings taken where the pages are silent (each is listed with its reason in the
 * repository's design notes):
 *   - score scale: real logit = t_i * (q_i . k_j) / sqrt(D)  (standard scaled dot product);
 *   - n_i = number of real keys visible to query i under the causal mask (i+1, 0-based i);
 *   - natural logarithms; softplus(x) = log(1 + e^x);
 *   - the null logit is t_i * nu_i (same temperature as the real logits);
 *   - Z = real mass + null mass (the full partition of the single softmax);
 *   - output o_i = mu_i * c_i;
 *   - eps = caller-supplied (1e-12 by convention), applied to the Z-normalised s_i;
 *   - parameters are per head; temp_raw and null_slope_raw pass through softplus.
 *
 * Every entry point parallelises only over independent (batch, head) pairs or query
 * rows with plain pthreads; the arithmetic of one task is a straight loop.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------- */
/* thread pool: run fn(task, ctx) for task = 0..ntasks-1 over nthreads threads  */
/* ------------------------------------------------------------------------- */
typedef void (*task_fn)(long task, void* ctx);
typedef struct { task_fn fn; void* ctx; long ntasks; int tid, nthreads; } worker_arg;

static void* worker_main(void* p) {
    worker_arg* a = (worker_arg*)p;
    for (long t = a->tid; t < a->ntasks; t += a->nthreads) a->fn(t, a->ctx);
    return NULL;
}

static int resolve_threads(int nthreads, long ntasks) {
    if (nthreads <= 0) {
        long n = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = n > 0 ? (int)n : 1;
    }
    if (nthreads > ntasks) nthreads = (int)(ntasks > 0 ? ntasks : 1);
    if (nthreads > 256) nthreads = 256;
    return nthreads;
}

static void run_tasks(task_fn fn, void* ctx, long ntasks, int nthreads) {
    nthreads = resolve_threads(nthreads, ntasks);
    if (nthreads == 1) {
        for (long t = 0; t < ntasks; ++t) fn(t, ctx);
        return;
    }
    pthread_t th[256];
    worker_arg args[256];
    for (int i = 0; i < nthreads; ++i) {
        args[i].fn = fn; args[i].ctx = ctx; args[i].ntasks = ntasks;
        args[i].tid = i; args[i].nthreads = nthreads;
        pthread_create(&th[i], NULL, worker_main, &args[i]);
    }
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
}

/* Number of threads the oracle would use for a given task count (reported by benchmarks). */
int oracle_threads_used(int nthreads, long ntasks) { return resolve_threads(nthreads, ntasks); }

/* ========================================================================= */
/* Gated-delta memory, sequential definition (Section 3.3 equation)          */
/* ========================================================================= */
/* Layouts (row-major, last index fastest):
 *   q, k  [B, T, H, Dk];  v [B, T, H, Dv];  alpha, beta [B, T, H];
 *   init_state, final_state [B, H, Dv, Dk] (init may be NULL = zero state);
 *   o [B, T, H, Dv];  states (optional, may be NULL) [B, T, H, Dv, Dk] = S_t after token t. */
typedef struct {
    int B, T, H, Dk, Dv;
    const double *q, *k, *v, *alpha, *beta, *init;
    double *o, *final_state, *states;
} gdn_ctx;

static void gdn_seq_task(long task, void* p) {
    const gdn_ctx* c = (const gdn_ctx*)p;
    const int b = (int)(task / c->H), h = (int)(task % c->H);
    const int Dk = c->Dk, Dv = c->Dv, H = c->H;
    double* S = (double*)calloc((size_t)Dv * Dk, sizeof(double));
    double* u = (double*)malloc((size_t)Dv * sizeof(double));
    if (c->init) memcpy(S, c->init + ((size_t)b * H + h) * Dv * Dk, sizeof(double) * Dv * Dk);
    for (int t = 0; t < c->T; ++t) {
        const size_t tok = ((size_t)b * c->T + t) * H + h;
        const double* qt = c->q + tok * Dk;
        const double* kt = c->k + tok * Dk;
        const double* vt = c->v + tok * Dv;
        const double a = c->alpha[tok], be = c->beta[tok];
        /* u = S_{t-1} k_t */
        for (int r = 0; r < Dv; ++r) {
            double s = 0.0;
            for (int j = 0; j < Dk; ++j) s += S[r * Dk + j] * kt[j];
            u[r] = s;
        }
        /* S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
         *     = alpha_t (S_{t-1} - beta_t u k_t^T) + beta_t v_t k_t^T */
        for (int r = 0; r < Dv; ++r)
            for (int j = 0; j < Dk; ++j)
                S[r * Dk + j] = a * (S[r * Dk + j] - be * u[r] * kt[j]) + be * vt[r] * kt[j];
        /* o_t = S_t q_t */
        double* ot = c->o + tok * Dv;
        for (int r = 0; r < Dv; ++r) {
            double s = 0.0;
            for (int j = 0; j < Dk; ++j) s += S[r * Dk + j] * qt[j];
            ot[r] = s;
        }
        if (c->states) memcpy(c->states + tok * Dv * Dk, S, sizeof(double) * Dv * Dk);
    }
    if (c->final_state) memcpy(c->final_state + ((size_t)b * H + h) * Dv * Dk, S, sizeof(double) * Dv * Dk);
    free(S);
    free(u);
}

int oracle_gdn_sequential(int B, int T, int H, int Dk, int Dv,
                          const double* q, const double* k, const double* v,
                          const double* alpha, const double* beta, const double* init_state,
                          double* o, double* final_state, double* states, int nthreads) {
    if (B < 1 || T < 0 || H < 1 || Dk < 1 || Dv < 1 || !q || !k || !v || !alpha || !beta || !o) return -1;
    gdn_ctx c = {B, T, H, Dk, Dv, q, k, v, alpha, beta, init_state, o, final_state, states};
    run_tasks(gdn_seq_task, &c, (long)B * H, nthreads);
    return 0;
}

/* ========================================================================= */
/* Gated-delta memory, chunked form (exact algebraic rewrite of Section 3.3)  */
/* ========================================================================= */
/* Writing S_t = alpha_t S_{t-1} + delta_t k_t^T with
 * delta_t = beta_t (v_t - alpha_t S_{t-1} k_t) and unrolling inside a chunk of n tokens
 * that starts from state S_in (g_r = sum_{s<=r} log alpha_s, r = 0..n-1):
 *   A[r][s] = beta_r exp(g_r - g_s) (k_r . k_s)            for s < r, else 0
 *   T = (I + A)^{-1}                                        (unit lower triangular)
 *   W = T diag(beta * exp(g)) K,   U = T diag(beta) V
 *   Delta = U - W S_in^T                                    (row r = delta_r)
 *   O = diag(exp(g)) Q S_in^T + lower_incl(Q K^T * exp(g_r - g_s)) Delta
 *   S_out = exp(g_{n-1}) S_in + Delta^T diag(exp(g_{n-1} - g)) K
 * Each step below is one of these lines, computed with plain loops. */
typedef struct { gdn_ctx g; int C; } gdn_chunk_ctx;

static void gdn_chunk_task(long task, void* p) {
    const gdn_chunk_ctx* cc = (const gdn_chunk_ctx*)p;
    const gdn_ctx* c = &cc->g;
    const int b = (int)(task / c->H), h = (int)(task % c->H);
    const int Dk = c->Dk, Dv = c->Dv, H = c->H, C = cc->C;
    double* S = (double*)calloc((size_t)Dv * Dk, sizeof(double));
    double* g = (double*)malloc(sizeof(double) * C);
    double* A = (double*)malloc(sizeof(double) * C * C);
    double* Ti = (double*)malloc(sizeof(double) * C * C);
    double* W = (double*)malloc(sizeof(double) * C * Dk);
    double* U = (double*)malloc(sizeof(double) * C * Dv);
    double* Dl = (double*)malloc(sizeof(double) * C * Dv);
    double* Sn = (double*)malloc(sizeof(double) * Dv * Dk);
    if (c->init) memcpy(S, c->init + ((size_t)b * H + h) * Dv * Dk, sizeof(double) * Dv * Dk);
#define TOK(t) (((size_t)b * c->T + (t)) * H + h)
    for (int t0 = 0; t0 < c->T; t0 += C) {
        const int n = (c->T - t0 < C) ? c->T - t0 : C;
        /* g_r: cumulative log-decay inside the chunk */
        double acc = 0.0;
        for (int r = 0; r < n; ++r) { acc += log(c->alpha[TOK(t0 + r)]); g[r] = acc; }
        /* A (strictly lower) */
        for (int r = 0; r < n; ++r)
            for (int s = 0; s < n; ++s) {
                double val = 0.0;
                if (s < r) {
                    const double* kr = c->k + TOK(t0 + r) * Dk;
                    const double* ks = c->k + TOK(t0 + s) * Dk;
                    double d = 0.0;
                    for (int j = 0; j < Dk; ++j) d += kr[j] * ks[j];
                    val = c->beta[TOK(t0 + r)] * exp(g[r] - g[s]) * d;
                }
                A[r * n + s] = val;
            }
        /* T = (I + A)^{-1} by forward substitution, column by column:
         * T[r][j] = [r==j] - sum_{s<r} A[r][s] T[s][j] */
        for (int j = 0; j < n; ++j)
            for (int r = 0; r < n; ++r) {
                double val = (r == j) ? 1.0 : 0.0;
                for (int s = 0; s < r; ++s) val -= A[r * n + s] * Ti[s * n + j];
                Ti[r * n + j] = val;
            }
        /* W = T diag(beta e^g) K ;  U = T diag(beta) V */
        for (int r = 0; r < n; ++r) {
            for (int j = 0; j < Dk; ++j) {
                double s_ = 0.0;
                for (int s = 0; s < n; ++s)
                    s_ += Ti[r * n + s] * c->beta[TOK(t0 + s)] * exp(g[s]) * c->k[TOK(t0 + s) * Dk + j];
                W[r * Dk + j] = s_;
            }
            for (int j = 0; j < Dv; ++j) {
                double s_ = 0.0;
                for (int s = 0; s < n; ++s)
                    s_ += Ti[r * n + s] * c->beta[TOK(t0 + s)] * c->v[TOK(t0 + s) * Dv + j];
                U[r * Dv + j] = s_;
            }
        }
        /* Delta = U - W S_in^T */
        for (int r = 0; r < n; ++r)
            for (int i = 0; i < Dv; ++i) {
                double s_ = 0.0;
                for (int j = 0; j < Dk; ++j) s_ += W[r * Dk + j] * S[i * Dk + j];
                Dl[r * Dv + i] = U[r * Dv + i] - s_;
            }
        /* O = diag(e^g) Q S_in^T + lower_incl(Q K^T * e^{g_r - g_s}) Delta */
        for (int r = 0; r < n; ++r) {
            const double* qr = c->q + TOK(t0 + r) * Dk;
            double* orow = c->o + TOK(t0 + r) * Dv;
            for (int i = 0; i < Dv; ++i) {
                double s_ = 0.0;
                for (int j = 0; j < Dk; ++j) s_ += qr[j] * S[i * Dk + j];
                orow[i] = exp(g[r]) * s_;
            }
            for (int s = 0; s <= r; ++s) {
                const double* ks = c->k + TOK(t0 + s) * Dk;
                double d = 0.0;
                for (int j = 0; j < Dk; ++j) d += qr[j] * ks[j];
                const double pw = d * exp(g[r] - g[s]);
                for (int i = 0; i < Dv; ++i) orow[i] += pw * Dl[s * Dv + i];
            }
        }
        /* S_out = e^{g_{n-1}} S_in + Delta^T diag(e^{g_{n-1} - g}) K */
        for (int i = 0; i < Dv; ++i)
            for (int j = 0; j < Dk; ++j) {
                double s_ = exp(g[n - 1]) * S[i * Dk + j];
                for (int r = 0; r < n; ++r)
                    s_ += Dl[r * Dv + i] * exp(g[n - 1] - g[r]) * c->k[TOK(t0 + r) * Dk + j];
                Sn[i * Dk + j] = s_;
            }
        memcpy(S, Sn, sizeof(double) * Dv * Dk);
    }
#undef TOK
    if (c->final_state) memcpy(c->final_state + ((size_t)b * H + h) * Dv * Dk, S, sizeof(double) * Dv * Dk);
    free(S); free(g); free(A); free(Ti); free(W); free(U); free(Dl); free(Sn);
}

int oracle_gdn_chunked(int B, int T, int H, int Dk, int Dv, int C,
                       const double* q, const double* k, const double* v,
                       const double* alpha, const double* beta, const double* init_state,
                       double* o, double* final_state, int nthreads) {
    if (B < 1 || T < 0 || H < 1 || Dk < 1 || Dv < 1 || C < 1 || !q || !k || !v || !alpha || !beta || !o) return -1;
    gdn_chunk_ctx cc = {{B, T, H, Dk, Dv, q, k, v, alpha, beta, init_state, o, final_state, NULL}, C};
    run_tasks(gdn_chunk_task, &cc, (long)B * H, nthreads);
    return 0;
}

/* ========================================================================= */
/* Polar attention                                                             */
/* ========================================================================= */
/* Per-head parameters, each [Hq] except v_null [Hq, D]:
 *   temp_raw (alpha in Section 3.2), null_slope_raw (gamma in Section 3.2),
 *   null_bias (b in Section 3.2), mag_beta (beta in Appendix A.2), v_null (Appendix C.3). */
typedef struct {
    const double *temp_raw, *null_slope_raw, *null_bias, *mag_beta, *v_null;
    double eps;
} polar_par;

static double softplus(double x) { return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x)); }

/* One query row against n real keys (key j at K + j*kstride, value at V + j*vstride).
 * Materialised form of Appendix C.2: all n real logits plus the null logit, one softmax,
 * channels from the weights.  Outputs o[D], *mu, *meff, *neff.  w is scratch of n doubles. */
static void polar_row_materialised(const double* qi, const double* K, const double* V, size_t kstride,
                                   size_t vstride, long n, int D, int h, const polar_par* P,
                                   double* o, double* mu, double* meff, double* neff, double* w) {
    const double a = softplus(P->temp_raw[h]);
    const double s = softplus(P->null_slope_raw[h]);
    const double t = 1.0 + a * log((double)n);                          /* Section 3.2: t_i */
    const double nu = P->null_bias[h] + s * sqrt(log((double)n + 1.0)); /* Section 3.2: nu_i */
    const double lnull = t * nu;                                        /* virtual null logit */
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    double m = lnull;
    for (long j = 0; j < n; ++j) {
        double d = 0.0;
        for (int x = 0; x < D; ++x) d += qi[x] * K[j * kstride + x];
        w[j] = t * d * inv_sqrt_d;
        if (w[j] > m) m = w[j];
    }
    /* single softmax over {real logits} U {null logit} */
    double Z = exp(lnull - m);
    for (long j = 0; j < n; ++j) { w[j] = exp(w[j] - m); Z += w[j]; }
    const double wnull = exp(lnull - m) / Z;
    double R = 0.0, Q2 = 0.0;
    for (long j = 0; j < n; ++j) { w[j] /= Z; R += w[j]; Q2 += w[j] * w[j]; }
    /* magnitude channel: participation ratio of the real weights, scaled by real mass */
    const double ne = R * R / Q2;
    const double me = ne * R;
    const double muv = tanh(P->mag_beta[h] * log1p(me));
    /* direction channel: s_i = sum_j w_ij v_j + w_null v_null, c_i = s_i / max(||s_i||, eps) */
    double nrm2 = 0.0;
    for (int x = 0; x < D; ++x) {
        double acc = wnull * P->v_null[(size_t)h * D + x];
        for (long j = 0; j < n; ++j) acc += w[j] * V[j * vstride + x];
        o[x] = acc;
        nrm2 += acc * acc;
    }
    const double nrm = sqrt(nrm2);
    const double den = nrm > P->eps ? nrm : P->eps;
    for (int x = 0; x < D; ++x) o[x] = muv * (o[x] / den);
    *mu = muv; *meff = me; *neff = ne;
}

/* Streaming form of Appendix C.3 / Table 6, with the key range cut into `nsplit`
 * contiguous segments whose (M, L, Q2, S) states are combined afterwards.  Inside a
 * segment keys arrive in blocks of `block`: M <- max(M, max a); rho = exp(M_old - M_new);
 * L <- rho L + sum p; Q2 <- rho^2 Q2 + sum p^2; S <- rho S + sum p v.  M covers real keys
 * only; the null logit enters at finalisation with the common origin M* = max(M, l_null). */
static void polar_row_streaming(const double* qi, const double* K, const double* V, size_t kstride,
                                size_t vstride, long n, int D, int h, const polar_par* P, long block,
                                int nsplit, double* o, double* mu, double* meff, double* neff,
                                double* scratch /* (D+3)*nsplit + block */) {
    const double a = softplus(P->temp_raw[h]);
    const double s = softplus(P->null_slope_raw[h]);
    const double t = 1.0 + a * log((double)n);
    const double nu = P->null_bias[h] + s * sqrt(log((double)n + 1.0));
    const double lnull = t * nu;
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    double* st = scratch;                       /* per split: M, L, Q2, S[D] */
    double* blk = scratch + (size_t)(D + 3) * nsplit;
    for (int sp = 0; sp < nsplit; ++sp) {
        const long j0 = n * sp / nsplit, j1 = n * (sp + 1) / nsplit;
        double M = -INFINITY, L = 0.0, Q2 = 0.0;
        double* Sv = st + (size_t)sp * (D + 3) + 3;
        for (int x = 0; x < D; ++x) Sv[x] = 0.0;
        for (long jb = j0; jb < j1; jb += block) {
            const long je = (jb + block < j1) ? jb + block : j1;
            double bmax = -INFINITY;
            for (long j = jb; j < je; ++j) {
                double d = 0.0;
                for (int x = 0; x < D; ++x) d += qi[x] * K[j * kstride + x];
                blk[j - jb] = t * d * inv_sqrt_d;
                if (blk[j - jb] > bmax) bmax = blk[j - jb];
            }
            const double Mn = bmax > M ? bmax : M;
            const double rho = exp(M - Mn); /* exp(-inf) = 0 on the first block */
            L *= rho; Q2 *= rho * rho;
            for (int x = 0; x < D; ++x) Sv[x] *= rho;
            for (long j = jb; j < je; ++j) {
                const double p = exp(blk[j - jb] - Mn);
                L += p; Q2 += p * p;
                for (int x = 0; x < D; ++x) Sv[x] += p * V[j * vstride + x];
            }
            M = Mn;
        }
        st[(size_t)sp * (D + 3) + 0] = M;
        st[(size_t)sp * (D + 3) + 1] = L;
        st[(size_t)sp * (D + 3) + 2] = Q2;
    }
    /* combine segments: M = max M_x, r_x = exp(M_x - M), L = sum r_x L_x,
     * Q2 = sum r_x^2 Q2_x, S = sum r_x S_x (empty segments have M = -inf, r = 0) */
    double M = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) if (st[(size_t)sp * (D + 3)] > M) M = st[(size_t)sp * (D + 3)];
    double L = 0.0, Q2 = 0.0;
    for (int x = 0; x < D; ++x) o[x] = 0.0;
    for (int sp = 0; sp < nsplit; ++sp) {
        const double* e = st + (size_t)sp * (D + 3);
        if (e[0] == -INFINITY) continue;
        const double r = exp(e[0] - M);
        L += r * e[1]; Q2 += r * r * e[2];
        for (int x = 0; x < D; ++x) o[x] += r * e[3 + x];
    }
    /* finalise: merge the null with origin M* = max(M, l_null) */
    const double Ms = M > lnull ? M : lnull;
    const double pnull = exp(lnull - Ms);
    const double Ls = L * exp(M - Ms);
    const double Z = Ls + pnull;
    const double ne = L * L / Q2;          /* scale-free: the origin cancels */
    const double me = ne * Ls / Z;
    const double muv = tanh(P->mag_beta[h] * log1p(me));
    double nrm2 = 0.0;
    for (int x = 0; x < D; ++x) {
        o[x] = (o[x] * exp(M - Ms) + pnull * P->v_null[(size_t)h * D + x]) / Z;
        nrm2 += o[x] * o[x];
    }
    const double nrm = sqrt(nrm2);
    const double den = nrm > P->eps ? nrm : P->eps;
    for (int x = 0; x < D; ++x) o[x] = muv * (o[x] / den);
    *mu = muv; *meff = me; *neff = ne;
}

typedef struct {
    int B, T, Hq, Hkv, D;
    const double *q, *k, *v;
    polar_par P;
    const int64_t* rows; long nrows;
    int mode; long block; int nsplit;
    double *o, *mu, *meff, *neff;
} polar_ctx;

/* task = ((b * nrows) + r) * Hq + h */
static void polar_task(long task, void* p) {
    const polar_ctx* c = (const polar_ctx*)p;
    const int h = (int)(task % c->Hq);
    const long r = (task / c->Hq) % c->nrows;
    const int b = (int)(task / ((long)c->Hq * c->nrows));
    const long i = c->rows ? (long)c->rows[r] : r;
    const int hk = h / (c->Hq / c->Hkv);
    const int D = c->D;
    const double* qi = c->q + (((size_t)b * c->T + i) * c->Hq + h) * D;
    const double* K = c->k + ((size_t)b * c->T * c->Hkv + hk) * D;
    const double* V = c->v + ((size_t)b * c->T * c->Hkv + hk) * D;
    const size_t stride = (size_t)c->Hkv * D;
    const size_t out = ((size_t)b * c->nrows + r) * c->Hq + h;
    if (c->mode == 0) {
        double* w = (double*)malloc(sizeof(double) * (size_t)(i + 1));
        polar_row_materialised(qi, K, V, stride, stride, i + 1, D, h, &c->P, c->o + out * D, c->mu + out,
                               c->meff + out, c->neff + out, w);
        free(w);
    } else {
        double* sc = (double*)malloc(sizeof(double) * ((size_t)(D + 3) * c->nsplit + c->block));
        polar_row_streaming(qi, K, V, stride, stride, i + 1, D, h, &c->P, c->block, c->nsplit, c->o + out * D,
                            c->mu + out, c->meff + out, c->neff + out, sc);
        free(sc);
    }
}

/* Causal Polar attention for the query rows listed in `rows` (NULL = all T rows).
 *   q [B, T, Hq, D];  k, v [B, T, Hkv, D];  query head h reads kv head h / (Hq / Hkv).
 * Outputs (row-sampled layout): o [B, nrows, Hq, D]; mu, meff, neff [B, nrows, Hq].
 * mode 0 = materialised single softmax (Appendix C.2); mode 1 = streaming statistics
 * (Table 6) with key blocks of `block` and `nsplit` merged key segments. */
int oracle_polar_fwd(int B, int T, int Hq, int Hkv, int D,
                     const double* q, const double* k, const double* v,
                     const double* temp_raw, const double* null_slope_raw, const double* null_bias,
                     const double* mag_beta, const double* v_null, double eps,
                     const int64_t* rows, long nrows, int mode, long block, int nsplit,
                     double* o, double* mu, double* meff, double* neff, int nthreads) {
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv) return -1;
    if (!q || !k || !v || !temp_raw || !null_slope_raw || !null_bias || !mag_beta || !v_null) return -1;
    if (!o || !mu || !meff || !neff) return -1;
    if (mode != 0 && (block < 1 || nsplit < 1)) return -1;
    if (!rows) nrows = T;
    for (long r = 0; rows && r < nrows; ++r) if (rows[r] < 0 || rows[r] >= T) return -1;
    polar_ctx c = {B, T, Hq, Hkv, D, q, k, v,
                   {temp_raw, null_slope_raw, null_bias, mag_beta, v_null, eps},
                   rows, nrows, mode, block, nsplit, o, mu, meff, neff};
    run_tasks(polar_task, &c, (long)B * nrows * Hq, nthreads);
    return 0;
}

/* Decode: one query per (b, h) against cache slots 0..cache_len-1 (the newest token is
 * already in slot cache_len-1), i.e. the last row of the causal forward with n = cache_len.
 *   q [B, Hq, D];  k_cache, v_cache [B, Lmax, Hkv, D];  o [B, Hq, D];  mu, meff, neff [B, Hq]. */
typedef struct {
    int B, Hq, Hkv, D; long cache_len, Lmax;
    const double *q, *kc, *vc; polar_par P;
    double *o, *mu, *meff, *neff;
} polar_dec_ctx;

static void polar_dec_task(long task, void* p) {
    const polar_dec_ctx* c = (const polar_dec_ctx*)p;
    const int b = (int)(task / c->Hq), h = (int)(task % c->Hq);
    const int hk = h / (c->Hq / c->Hkv), D = c->D;
    const size_t stride = (size_t)c->Hkv * D;
    const double* K = c->kc + ((size_t)b * c->Lmax * c->Hkv + hk) * D;
    const double* V = c->vc + ((size_t)b * c->Lmax * c->Hkv + hk) * D;
    double* w = (double*)malloc(sizeof(double) * (size_t)c->cache_len);
    polar_row_materialised(c->q + ((size_t)b * c->Hq + h) * D, K, V, stride, stride, c->cache_len, D, h, &c->P,
                           c->o + ((size_t)b * c->Hq + h) * D, c->mu + task, c->meff + task, c->neff + task, w);
    free(w);
}

int oracle_polar_decode(int B, int Hq, int Hkv, int D, long cache_len, long Lmax,
                        const double* q, const double* k_cache, const double* v_cache,
                        const double* temp_raw, const double* null_slope_raw, const double* null_bias,
                        const double* mag_beta, const double* v_null, double eps,
                        double* o, double* mu, double* meff, double* neff, int nthreads) {
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv || cache_len < 1 || cache_len > Lmax) return -1;
    if (!q || !k_cache || !v_cache || !temp_raw || !null_slope_raw || !null_bias || !mag_beta || !v_null) return -1;
    if (!o || !mu || !meff || !neff) return -1;
    polar_dec_ctx c = {B, Hq, Hkv, D, cache_len, Lmax, q, k_cache, v_cache,
                       {temp_raw, null_slope_raw, null_bias, mag_beta, v_null, eps}, o, mu, meff, neff};
    run_tasks(polar_dec_task, &c, (long)B * Hq, nthreads);
    return 0;
}

/* ========================================================================= */
/* Baseline attention cores: NoPE and RoPE (the matched controls)            */
/* ========================================================================= */
/* The paper's matched models differ only in the attention core (Section 3.1: NoPE, RoPE
 * or Polar).  The pages name the two controls without restating them; these are their
 * textbook definitions (readings listed in the design notes):
 *   - NoPE: causal softmax attention, logit q_i . k_j / sqrt(D), output sum_j w_ij v_j;
 *   - RoPE: the same after rotating every adjacent pair (x[2p], x[2p+1]) of q_i and k_j by
 *     the angle pos * theta^(-2p/D), pos being the token's position (rotary position
 *     embedding of Su et al.; theta = 10000 in the usual setting). */

/* Round to the nearest bf16 value (ties to even), through fp32 as a bf16 pipeline rounds.
 * atma_rope writes bf16: its output is the exact rotation rounded once by this function. */
static double round_bf16(double x) {
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    u &= 0xFFFF0000u;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Rotate one D-vector in place to position `pos`. */
static void rope_vec(double* x, int D, double pos, double theta) {
    for (int p = 0; 2 * p + 1 < D; ++p) {
        const double ang = pos * pow(theta, -2.0 * p / D);
        const double c = cos(ang), s = sin(ang);
        const double a = x[2 * p], b = x[2 * p + 1];
        x[2 * p] = a * c - b * s;
        x[2 * p + 1] = a * s + b * c;
    }
}

/* x, y [B, T, H, D]; row t of every sequence is rotated to position pos0 + t (then rounded
 * to bf16 when quant is set). */
int oracle_rope(int B, int T, int H, int D, long pos0, double theta, int quant, const double* x, double* y) {
    if (B < 1 || T < 1 || H < 1 || D < 2 || D % 2 || theta <= 0.0 || !x || !y) return -1;
    for (long b = 0; b < B; ++b)
        for (long t = 0; t < T; ++t)
            for (long h = 0; h < H; ++h) {
                const size_t off = (((size_t)b * T + t) * H + h) * D;
                memcpy(y + off, x + off, sizeof(double) * D);
                rope_vec(y + off, D, (double)(pos0 + t), theta);
                for (int e = 0; quant && e < D; ++e) y[off + e] = round_bf16(y[off + e]);
            }
    return 0;
}

/* One softmax row: query qi (already rotated) against n keys (rows of K with stride ks,
 * already rotated), values V (stride vs); o [D]. */
static void softmax_row(const double* qi, const double* K, const double* V, size_t ks, size_t vs, long n, int D,
                        double* o, double* w) {
    const double scale = 1.0 / sqrt((double)D);
    double m = -INFINITY;
    for (long j = 0; j < n; ++j) {
        double d = 0.0;
        for (int e = 0; e < D; ++e) d += qi[e] * K[j * ks + e];
        w[j] = d * scale;
        if (w[j] > m) m = w[j];
    }
    double z = 0.0;
    for (long j = 0; j < n; ++j) {
        w[j] = exp(w[j] - m);
        z += w[j];
    }
    for (int e = 0; e < D; ++e) o[e] = 0.0;
    for (long j = 0; j < n; ++j)
        for (int e = 0; e < D; ++e) o[e] += w[j] / z * V[j * vs + e];
}

/* Rounding tolerance of one softmax row whose query and keys are rounded element by element to
 * the nearest bf16 value (what a bf16 attention kernel does to the rotated q and k of the RoPE
 * core), by probabilistic rounding error analysis (Higham and Mary, "A new approach to
 * probabilistic rounding error analysis", SIAM J. Sci. Comput. 41 (2019)): the relative rounding
 * errors eta of the elements are modelled as independent, mean zero, |eta| <= u = 2^-8 (the unit
 * roundoff of bf16, which keeps 8 significant bits).
 *   To first order, q_e -> q_e (1 + eta_e) and k_je -> k_je (1 + eta'_je) move logit j by
 *       d_j = sum_e (eta_e + eta'_je) q_e k_je / sqrt(D),
 *   the weights by w_j (d_j - sum_k w_k d_k), and output element x by
 *       dO_x = sum_j w_j d_j c_jx,   c_jx = v_jx - o_x   (the sum_k w_k d_k part cancels),
 *            = (1/sqrt(D)) [ sum_e eta_e A_ex + sum_{j,e} eta'_je B_jex ],
 *   A_ex = q_e sum_j w_j k_je c_jx,   B_jex = q_e k_je w_j c_jx.
 *   Hoeffding's inequality for a sum of independent terms a_i eta_i, |eta_i| <= u, gives
 *       P(|dO_x| >= lambda u sqrt(sum a_i^2) / sqrt(D)) <= 2 exp(-lambda^2 / 2),
 *   so tol_x = lambda u sqrt(sum_e A_ex^2 + sum_j w_j^2 c_jx^2 sum_e (q_e k_je)^2) / sqrt(D).
 * qi, K (stride ks), V (stride vs) as softmax_row; w the row's weights from softmax_row
 * (renormalised here); tol [D] receives the tolerance for the given lambda. */
static void rounding_tolerance(const double* qi, const double* K, const double* V, size_t ks, size_t vs, long n,
                               int D, const double* o, const double* w, double lambda, double* tol) {
    const double u = 1.0 / 256.0;
    double z = 0.0;
    for (long j = 0; j < n; ++j) z += w[j];
    double* M = (double*)calloc((size_t)D * D, sizeof(double));  /* M[x][e] = sum_j w_j k_je c_jx */
    double* sb = (double*)calloc((size_t)D, sizeof(double));     /* sum_j w_j^2 c_jx^2 sum_e (q_e k_je)^2 */
    for (long j = 0; j < n; ++j) {
        const double wj = w[j] / z;
        double a2 = 0.0;
        for (int e = 0; e < D; ++e) a2 += (qi[e] * K[j * ks + e]) * (qi[e] * K[j * ks + e]);
        for (int x = 0; x < D; ++x) {
            const double c = V[j * vs + x] - o[x];
            sb[x] += wj * wj * c * c * a2;
            double* Mx = M + (size_t)x * D;
            for (int e = 0; e < D; ++e) Mx[e] += wj * c * K[j * ks + e];
        }
    }
    for (int x = 0; x < D; ++x) {
        double sa = 0.0;
        for (int e = 0; e < D; ++e) sa += (qi[e] * M[(size_t)x * D + e]) * (qi[e] * M[(size_t)x * D + e]);
        tol[x] = lambda * u * sqrt((sa + sb[x]) / (double)D);
    }
    free(M);
    free(sb);
}

typedef struct {
    int B, T, Hq, Hkv, D;
    const double *q, *k, *v;
    double theta;
    double* o;
    double* tol;    /* NULL, or the rounding tolerance of every output element (see above) */
    double lambda;
} softmax_ctx;

/* task = b * Hq + h: every query row of one (batch, query head) */
static void softmax_task(long task, void* p) {
    const softmax_ctx* c = (const softmax_ctx*)p;
    const int b = (int)(task / c->Hq), h = (int)(task % c->Hq), hk = h / (c->Hq / c->Hkv), D = c->D;
    const size_t T = (size_t)c->T;
    double* K = (double*)malloc(sizeof(double) * T * D);
    double* w = (double*)malloc(sizeof(double) * T);
    double* qi = (double*)malloc(sizeof(double) * D);
    for (size_t j = 0; j < T; ++j) {
        memcpy(K + j * D, c->k + ((b * T + j) * c->Hkv + hk) * D, sizeof(double) * D);
        if (c->theta > 0.0) rope_vec(K + j * D, D, (double)j, c->theta);
    }
    const double* V = c->v + ((size_t)b * T * c->Hkv + hk) * D;
    for (size_t i = 0; i < T; ++i) {
        memcpy(qi, c->q + ((b * T + i) * c->Hq + h) * D, sizeof(double) * D);
        if (c->theta > 0.0) rope_vec(qi, D, (double)i, c->theta);
        double* oi = c->o + ((b * T + i) * c->Hq + h) * D;
        softmax_row(qi, K, V, D, (size_t)c->Hkv * D, (long)i + 1, D, oi, w);
        if (c->tol) rounding_tolerance(qi, K, V, D, (size_t)c->Hkv * D, (long)i + 1, D, oi, w, c->lambda,
                                       c->tol + ((b * T + i) * c->Hq + h) * D);
    }
    free(K);
    free(w);
    free(qi);
}

/* Causal softmax attention, NoPE (theta <= 0) or RoPE (theta > 0, exact rotation), all rows.
 *   q [B, T, Hq, D];  k, v [B, T, Hkv, D];  o [B, T, Hq, D];
 *   tol [B, T, Hq, D] or NULL: for every output element, the tolerance (rounding_tolerance, with
 *   the given lambda) for rounding each element of the rotated q and k to the nearest bf16 value. */
int oracle_softmax_attn(int B, int T, int Hq, int Hkv, int D, double theta, const double* q,
                        const double* k, const double* v, double* o, double* tol, double lambda, int nthreads) {
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || D < 2 || D % 2 || Hq % Hkv || !q || !k || !v || !o) return -1;
    softmax_ctx c = {B, T, Hq, Hkv, D, q, k, v, theta, o, tol, lambda};
    run_tasks(softmax_task, &c, (long)B * Hq, nthreads);
    return 0;
}

/* Decode row of the same cores: the query at position cache_len - 1 against cache slots
 * 0..cache_len-1, used as given.  For RoPE (theta > 0) the cache holds keys already rotated to
 * their slot positions (a RoPE KV cache is filled with rotated keys), and only the query is
 * rotated here.
 *   q [B, Hq, D];  k_cache, v_cache [B, Lmax, Hkv, D];  o [B, Hq, D]. */
int oracle_softmax_decode(int B, int Hq, int Hkv, int D, long cache_len, long Lmax, double theta,
                          const double* q, const double* kc, const double* vc, double* o) {
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 2 || D % 2 || Hq % Hkv || cache_len < 1 || cache_len > Lmax) return -1;
    if (!q || !kc || !vc || !o) return -1;
    double* w = (double*)malloc(sizeof(double) * (size_t)cache_len);
    double* qi = (double*)malloc(sizeof(double) * D);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            const int hk = h / (Hq / Hkv);
            memcpy(qi, q + ((size_t)b * Hq + h) * D, sizeof(double) * D);
            if (theta > 0.0) rope_vec(qi, D, (double)(cache_len - 1), theta);
            softmax_row(qi, kc + ((size_t)b * Lmax * Hkv + hk) * D, vc + ((size_t)b * Lmax * Hkv + hk) * D,
                        (size_t)Hkv * D, (size_t)Hkv * D, cache_len, D, o + ((size_t)b * Hq + h) * D, w);
        }
    free(w);
    free(qi);
    return 0;
}

/* ========================================================================= */
/* Canon prologue: depthwise causal convolution, optional per-head L2 norm    */
/* ========================================================================= */
/* Section 3.1 of the paper applies Canon depthwise causal convolutions to q, k and v before
 * attention; the pages fix neither the width nor a bias or residual.  Reading (listed in the
 * design notes): per channel c, y_t = sum_{j<K} w[j][c] x_{t-j} (+ x_t with `residual`), the
 * inputs before the first token taken from `state` (the K-1 previous inputs, oldest first;
 * zeros when NULL); then, when H > 0, each of the H groups of C/H channels is scaled to unit
 * L2 norm, y / max(||y||, eps) (the memory path's unit-norm keys and queries).
 *   x [B, T, C];  w [K, C];  state [B, K-1, C] or NULL;  y [B, T, C]. */
int oracle_canon(int B, int T, int C, int K, int residual, int H, double eps, const double* x, const double* w,
                 const double* state, double* y) {
    if (B < 1 || T < 1 || C < 1 || K < 1 || H < 0 || (H > 0 && C % H) || !x || !w || !y) return -1;
    for (long b = 0; b < B; ++b) {
        for (long t = 0; t < T; ++t) {
            double* yt = y + ((size_t)b * T + t) * C;
            for (int c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int j = 0; j < K; ++j) {
                    const long s = t - j;
                    double xv = 0.0;
                    if (s >= 0) xv = x[((size_t)b * T + s) * C + c];
                    else if (state && K - 1 + s >= 0) xv = state[((size_t)b * (K - 1) + (K - 1 + s)) * C + c];
                    acc += w[(size_t)j * C + c] * xv;
                }
                yt[c] = acc + (residual ? x[((size_t)b * T + t) * C + c] : 0.0);
            }
            for (int h = 0; h < H; ++h) {
                const int D = C / H;
                double n2 = 0.0;
                for (int e = 0; e < D; ++e) n2 += yt[h * D + e] * yt[h * D + e];
                const double den = sqrt(n2) > eps ? sqrt(n2) : eps;
                for (int e = 0; e < D; ++e) yt[h * D + e] /= den;
            }
        }
    }
    return 0;
}

/* ========================================================================= */
/* Backward: gradients of a scalar loss through the two definitions above     */
/* ========================================================================= */
/* The layer is trained end to end, and the paper's materialised path serves as the reference
 * for its gradients as well as its outputs (Appendix C.2).  The gradients here are the chain
 * rule applied to the forward definitions exactly as written above, one intermediate at a time,
 * in reverse order.  Given the upstream
 * gradient dO of the outputs (and optionally of the final memory state), every function returns
 * the gradient of every input and parameter. */

/* Gated-delta memory (Section 3.3 equation), reverse pass over the token-by-token recurrence.
 * With u_t = S_{t-1} k_t and S_t = alpha_t (S_{t-1} - beta_t u_t k_t^T) + beta_t v_t k_t^T,
 * o_t = S_t q_t, and G the gradient on S_t (dO_t q_t^T plus what flows back from S_{t+1}):
 *   dq_t     = S_t^T dO_t
 *   dv_t     = beta_t G k_t
 *   dbeta_t  = (G k_t) . (v_t - alpha_t u_t)
 *   dalpha_t = <G, S_{t-1}> - beta_t (G k_t) . u_t
 *   dk_t     = beta_t G^T v_t - alpha_t beta_t (S_{t-1}^T (G k_t) + G^T u_t)
 *   G_{t-1}  = alpha_t (G - beta_t (G k_t) k_t^T)
 * Layouts as the forward; dS_final [B, H, Dv, Dk] or NULL (zero); d_init [B, H, Dv, Dk] or
 * NULL (the gradient on the initial state, G_{-1}). */
typedef struct {
    gdn_ctx g;
    const double *dO, *dSfin;
    double *dq, *dk, *dv, *dalpha, *dbeta, *dinit;
} gdn_bwd_ctx;

static void gdn_bwd_task(long task, void* p) {
    const gdn_bwd_ctx* bc = (const gdn_bwd_ctx*)p;
    const gdn_ctx* c = &bc->g;
    const int b = (int)(task / c->H), h = (int)(task % c->H);
    const int Dk = c->Dk, Dv = c->Dv, H = c->H, T = c->T;
    const size_t SS = (size_t)Dv * Dk;
    /* forward, keeping every state: hist[t + 1] = S_t, hist[0] = initial state */
    double* hist = (double*)calloc((size_t)(T + 1) * SS, sizeof(double));
    double* G = (double*)calloc(SS, sizeof(double));
    double* u = (double*)malloc(sizeof(double) * Dv);
    double* Gk = (double*)malloc(sizeof(double) * Dv);
    if (c->init) memcpy(hist, c->init + ((size_t)b * H + h) * SS, sizeof(double) * SS);
#define TOKB(t) (((size_t)b * T + (t)) * H + h)
    for (int t = 0; t < T; ++t) {
        const double* Sp = hist + (size_t)t * SS;
        double* Sn = hist + (size_t)(t + 1) * SS;
        const double* kt = c->k + TOKB(t) * Dk;
        const double* vt = c->v + TOKB(t) * Dv;
        const double a = c->alpha[TOKB(t)], be = c->beta[TOKB(t)];
        for (int r = 0; r < Dv; ++r) {
            double s = 0.0;
            for (int j = 0; j < Dk; ++j) s += Sp[r * Dk + j] * kt[j];
            u[r] = s;
        }
        for (int r = 0; r < Dv; ++r)
            for (int j = 0; j < Dk; ++j) Sn[r * Dk + j] = a * (Sp[r * Dk + j] - be * u[r] * kt[j]) + be * vt[r] * kt[j];
    }
    if (bc->dSfin) memcpy(G, bc->dSfin + ((size_t)b * H + h) * SS, sizeof(double) * SS);
    for (int t = T - 1; t >= 0; --t) {
        const double* Sp = hist + (size_t)t * SS;
        const double* St = hist + (size_t)(t + 1) * SS;
        const double* qt = c->q + TOKB(t) * Dk;
        const double* kt = c->k + TOKB(t) * Dk;
        const double* vt = c->v + TOKB(t) * Dv;
        const double* gt = bc->dO + TOKB(t) * Dv;
        const double a = c->alpha[TOKB(t)], be = c->beta[TOKB(t)];
        /* o_t = S_t q_t */
        for (int r = 0; r < Dv; ++r)
            for (int j = 0; j < Dk; ++j) G[r * Dk + j] += gt[r] * qt[j];
        double* dqt = bc->dq + TOKB(t) * Dk;
        for (int j = 0; j < Dk; ++j) {
            double s = 0.0;
            for (int r = 0; r < Dv; ++r) s += St[r * Dk + j] * gt[r];
            dqt[j] = s;
        }
        /* the update S_t = alpha (S_{t-1} - beta u k^T) + beta v k^T */
        for (int r = 0; r < Dv; ++r) {
            double s = 0.0, s2 = 0.0;
            for (int j = 0; j < Dk; ++j) { s += Sp[r * Dk + j] * kt[j]; s2 += G[r * Dk + j] * kt[j]; }
            u[r] = s;
            Gk[r] = s2;
        }
        double db = 0.0, da = 0.0, gku = 0.0;
        for (int r = 0; r < Dv; ++r) {
            db += Gk[r] * (vt[r] - a * u[r]);
            gku += Gk[r] * u[r];
            for (int j = 0; j < Dk; ++j) da += G[r * Dk + j] * Sp[r * Dk + j];
        }
        bc->dbeta[TOKB(t)] = db;
        bc->dalpha[TOKB(t)] = da - be * gku;
        double* dvt = bc->dv + TOKB(t) * Dv;
        for (int r = 0; r < Dv; ++r) dvt[r] = be * Gk[r];
        double* dkt = bc->dk + TOKB(t) * Dk;
        for (int j = 0; j < Dk; ++j) {
            double gv = 0.0, sg = 0.0, gu = 0.0;
            for (int r = 0; r < Dv; ++r) {
                gv += G[r * Dk + j] * vt[r];
                sg += Sp[r * Dk + j] * Gk[r];
                gu += G[r * Dk + j] * u[r];
            }
            dkt[j] = be * gv - a * be * (sg + gu);
        }
        /* G_{t-1} = alpha (G - beta (G k) k^T) */
        for (int r = 0; r < Dv; ++r)
            for (int j = 0; j < Dk; ++j) G[r * Dk + j] = a * (G[r * Dk + j] - be * Gk[r] * kt[j]);
    }
    if (bc->dinit) memcpy(bc->dinit + ((size_t)b * H + h) * SS, G, sizeof(double) * SS);
#undef TOKB
    free(hist); free(G); free(u); free(Gk);
}

int oracle_gdn_bwd(int B, int T, int H, int Dk, int Dv,
                   const double* q, const double* k, const double* v,
                   const double* alpha, const double* beta, const double* init_state,
                   const double* dO, const double* dS_final,
                   double* dq, double* dk, double* dv, double* dalpha, double* dbeta, double* d_init,
                   int nthreads) {
    if (B < 1 || T < 0 || H < 1 || Dk < 1 || Dv < 1 || !q || !k || !v || !alpha || !beta || !dO) return -1;
    if (!dq || !dk || !dv || !dalpha || !dbeta) return -1;
    gdn_bwd_ctx bc = {{B, T, H, Dk, Dv, q, k, v, alpha, beta, init_state, NULL, NULL, NULL},
                      dO, dS_final, dq, dk, dv, dalpha, dbeta, d_init};
    run_tasks(gdn_bwd_task, &bc, (long)B * H, nthreads);
    return 0;
}

/* Polar attention (Section 3.2 equation, Appendix C.2 single softmax, Appendix A.2 channels),
 * one query row in reverse, with g = dO_i and the forward quantities recomputed as in
 * polar_row_materialised (weights w_j, null weight w_0, real mass R, squared mass Q2 = sum w_j^2,
 * m_eff = R^3 / Q2, mu, s, den = max(||s||, eps), c = s / den):
 *   dmu = g . c,   dc = mu g
 *   ds  = (dc - c (c . dc)) / den   when ||s|| > eps, else dc / eps
 *   dm_eff = dmu (1 - mu^2) beta / (1 + m_eff);   dbeta += dmu (1 - mu^2) ln(1 + m_eff)
 *   dR = dm_eff 3 R^2 / Q2;   dQ2 = -dm_eff R^3 / Q2^2
 *   dw_j = dR + 2 w_j dQ2 + ds . v_j;   dw_0 = ds . v_null;   dv_j += w_j ds;   dv_null += w_0 ds
 *   softmax: Sigma = sum_j w_j dw_j + w_0 dw_0;  dl_j = w_j (dw_j - Sigma);  dl_0 = w_0 (dw_0 - Sigma)
 *   logits l_j = t (q . k_j) / sqrt(D):  dq += sum_j dl_j t k_j / sqrt(D);  dk_j += dl_j t q / sqrt(D)
 *   dt = sum_j dl_j (q . k_j) / sqrt(D) + dl_0 nu;   dnu = dl_0 t      (null logit l_0 = t nu)
 *   t = 1 + softplus(temp_raw) ln n:             dtemp_raw += dt ln(n) sigmoid(temp_raw)
 *   nu = b + softplus(slope_raw) sqrt(ln(n+1)):  dnull_bias += dnu;  dslope_raw += dnu sqrt(ln(n+1)) sigmoid(slope_raw)
 * dpar[0..3] accumulate dtemp_raw, dslope_raw, dnull_bias, dbeta of head h; dpar[4..4+D) dv_null.
 * dabs[0..3] accumulate the magnitudes of the same four per-row contributions: the scale of those
 * sums, against which their rounding error is judged (the terms of a row sum can cancel).  The
 * temperature's row term is itself a sum over keys (dl_j q.k_j / sqrt(D), plus the null's), so its
 * magnitude is taken term by term. */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static void polar_row_backward(const double* qi, const double* K, const double* V, size_t kstride, long n, int D,
                               int h, const polar_par* P, const double* g, double* dqi, double* dK, double* dV,
                               double* dpar, double* dabs, double* w, double* qk) {
    const double a = softplus(P->temp_raw[h]);
    const double sl = softplus(P->null_slope_raw[h]);
    const double t = 1.0 + a * log((double)n);
    const double nu = P->null_bias[h] + sl * sqrt(log((double)n + 1.0));
    const double lnull = t * nu;
    const double isd = 1.0 / sqrt((double)D);
    const double* vn = P->v_null + (size_t)h * D;
    /* forward recomputation */
    double m = lnull;
    for (long j = 0; j < n; ++j) {
        double d = 0.0;
        for (int x = 0; x < D; ++x) d += qi[x] * K[j * kstride + x];
        qk[j] = d * isd;
        w[j] = t * qk[j];
        if (w[j] > m) m = w[j];
    }
    double Z = exp(lnull - m);
    for (long j = 0; j < n; ++j) { w[j] = exp(w[j] - m); Z += w[j]; }
    const double w0 = exp(lnull - m) / Z;
    double R = 0.0, Q2 = 0.0;
    for (long j = 0; j < n; ++j) { w[j] /= Z; R += w[j]; Q2 += w[j] * w[j]; }
    const double me = R * R * R / Q2;
    const double be = P->mag_beta[h];
    const double mu = tanh(be * log1p(me));
    double* s = (double*)malloc(sizeof(double) * D * 2);
    double* ds = s + D;
    double nrm2 = 0.0;
    for (int x = 0; x < D; ++x) {
        double acc = w0 * vn[x];
        for (long j = 0; j < n; ++j) acc += w[j] * V[j * kstride + x];
        s[x] = acc;
        nrm2 += acc * acc;
    }
    const double nrm = sqrt(nrm2);
    const int clamped = !(nrm > P->eps);
    const double den = clamped ? P->eps : nrm;
    /* channels */
    double dmu = 0.0, cdc = 0.0;
    for (int x = 0; x < D; ++x) dmu += g[x] * s[x] / den;
    for (int x = 0; x < D; ++x) cdc += (s[x] / den) * (mu * g[x]);
    for (int x = 0; x < D; ++x) ds[x] = (mu * g[x] - (clamped ? 0.0 : (s[x] / den) * cdc)) / den;
    const double dme = dmu * (1.0 - mu * mu) * be / (1.0 + me);
    dpar[3] += dmu * (1.0 - mu * mu) * log1p(me);
    dabs[3] += fabs(dmu * (1.0 - mu * mu) * log1p(me));
    const double dR = dme * 3.0 * R * R / Q2;
    const double dQ2 = -dme * R * R * R / (Q2 * Q2);
    /* weights: dw_j kept in w's place after Sigma is formed */
    double dw0 = 0.0;
    for (int x = 0; x < D; ++x) dw0 += ds[x] * vn[x];
    double Sig = w0 * dw0;
    for (long j = 0; j < n; ++j) {
        double dv = 0.0;
        for (int x = 0; x < D; ++x) dv += ds[x] * V[j * kstride + x];
        const double dwj = dR + 2.0 * w[j] * dQ2 + dv;
        Sig += w[j] * dwj;
        for (int x = 0; x < D; ++x) dV[j * kstride + x] += w[j] * ds[x];
        qk[j + n] = dwj; /* second half of the scratch holds dw_j */
    }
    for (int x = 0; x < D; ++x) dpar[4 + x] += w0 * ds[x];
    /* softmax and logits */
    double dt = 0.0, dt_mag = 0.0;
    for (long j = 0; j < n; ++j) {
        const double dl = w[j] * (qk[j + n] - Sig);
        dt += dl * qk[j];
        dt_mag += fabs(dl * qk[j]);
        for (int x = 0; x < D; ++x) {
            dqi[x] += dl * t * isd * K[j * kstride + x];
            dK[j * kstride + x] += dl * t * isd * qi[x];
        }
    }
    const double dl0 = w0 * (dw0 - Sig);
    dt += dl0 * nu;
    const double dnu = dl0 * t;
    dpar[0] += dt * log((double)n) * sigmoid(P->temp_raw[h]);
    dpar[1] += dnu * sqrt(log((double)n + 1.0)) * sigmoid(P->null_slope_raw[h]);
    dpar[2] += dnu;
    dabs[0] += (dt_mag + fabs(dl0 * nu)) * log((double)n) * sigmoid(P->temp_raw[h]);
    dabs[1] += fabs(dnu * sqrt(log((double)n + 1.0)) * sigmoid(P->null_slope_raw[h]));
    dabs[2] += fabs(dnu);
    free(s);
}

typedef struct {
    int B, T, Hq, Hkv, D;
    const double *q, *k, *v, *dO;
    polar_par P;
    double *dq, *dk, *dv, *dpar; /* dpar [B, Hq, 4 + D] partials, summed over b afterwards */
    double* dabs;                /* [B, Hq, 4] magnitudes of the scalar parameter contributions */
} polar_bwd_ctx;

/* task = b * Hkv + hk: every query head of the group and every row, so that the task alone
 * accumulates the key and value gradients of its (b, hk) */
static void polar_bwd_task(long task, void* p) {
    const polar_bwd_ctx* c = (const polar_bwd_ctx*)p;
    const int b = (int)(task / c->Hkv), hk = (int)(task % c->Hkv);
    const int D = c->D, G = c->Hq / c->Hkv;
    const size_t stride = (size_t)c->Hkv * D;
    const double* K = c->k + ((size_t)b * c->T * c->Hkv + hk) * D;
    const double* V = c->v + ((size_t)b * c->T * c->Hkv + hk) * D;
    double* dK = c->dk + ((size_t)b * c->T * c->Hkv + hk) * D;
    double* dV = c->dv + ((size_t)b * c->T * c->Hkv + hk) * D;
    double* w = (double*)malloc(sizeof(double) * (size_t)c->T);
    double* qk = (double*)malloc(sizeof(double) * (size_t)c->T * 2);
    for (long i = 0; i < c->T; ++i)
        for (int x = 0; x < D; ++x) dK[i * stride + x] = dV[i * stride + x] = 0.0;
    for (int h = hk * G; h < (hk + 1) * G; ++h)
        for (long i = 0; i < c->T; ++i) {
            const size_t row = ((size_t)b * c->T + i) * c->Hq + h;
            double* dqi = c->dq + row * D;
            for (int x = 0; x < D; ++x) dqi[x] = 0.0;
            polar_row_backward(c->q + row * D, K, V, stride, i + 1, D, h, &c->P, c->dO + row * D, dqi, dK, dV,
                               c->dpar + ((size_t)b * c->Hq + h) * (4 + D), c->dabs + ((size_t)b * c->Hq + h) * 4,
                               w, qk);
        }
    free(w);
    free(qk);
}

/* Gradients of causal Polar attention (materialised form) given dO [B, T, Hq, D].
 * Outputs dq [B, T, Hq, D]; dk, dv [B, T, Hkv, D]; d_temp_raw, d_null_slope_raw, d_null_bias,
 * d_mag_beta [Hq]; d_v_null [Hq, D]; d_abs [4, Hq] or NULL: the sums of the magnitudes of the
 * per-row contributions to the four scalar parameter gradients (tolerance scale for tests). */
int oracle_polar_bwd(int B, int T, int Hq, int Hkv, int D, const double* q, const double* k, const double* v,
                     const double* temp_raw, const double* null_slope_raw, const double* null_bias,
                     const double* mag_beta, const double* v_null, double eps, const double* dO,
                     double* dq, double* dk, double* dv, double* d_temp_raw, double* d_null_slope_raw,
                     double* d_null_bias, double* d_mag_beta, double* d_v_null, double* d_abs, int nthreads) {
    if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv) return -1;
    if (!q || !k || !v || !temp_raw || !null_slope_raw || !null_bias || !mag_beta || !v_null || !dO) return -1;
    if (!dq || !dk || !dv || !d_temp_raw || !d_null_slope_raw || !d_null_bias || !d_mag_beta || !d_v_null) return -1;
    double* dpar = (double*)calloc((size_t)B * Hq * (4 + D), sizeof(double));
    double* dabs = (double*)calloc((size_t)B * Hq * 4, sizeof(double));
    polar_bwd_ctx c = {B, T, Hq, Hkv, D, q, k, v, dO, {temp_raw, null_slope_raw, null_bias, mag_beta, v_null, eps},
                       dq, dk, dv, dpar, dabs};
    run_tasks(polar_bwd_task, &c, (long)B * Hkv, nthreads);
    for (int h = 0; h < Hq; ++h) {
        double acc[4] = {0.0, 0.0, 0.0, 0.0};
        for (int x = 0; x < D; ++x) d_v_null[(size_t)h * D + x] = 0.0;
        for (int b = 0; b < B; ++b) {
            const double* pp = dpar + ((size_t)b * Hq + h) * (4 + D);
            for (int e = 0; e < 4; ++e) acc[e] += pp[e];
            for (int x = 0; x < D; ++x) d_v_null[(size_t)h * D + x] += pp[4 + x];
        }
        d_temp_raw[h] = acc[0];
        d_null_slope_raw[h] = acc[1];
        d_null_bias[h] = acc[2];
        d_mag_beta[h] = acc[3];
        for (int e = 0; d_abs && e < 4; ++e) {
            double m = 0.0;
            for (int b = 0; b < B; ++b) m += dabs[((size_t)b * Hq + h) * 4 + e];
            d_abs[(size_t)e * Hq + h] = m;
        }
    }
    free(dpar);
    free(dabs);
    return 0;
}
