/*
 * rodimus_oracle.c -- plain, slow, sequential fp64 CPU oracle for the Rodimus*
 * token mixer.  TEST INFRASTRUCTURE ONLY: it is loaded by the tests, by the
 * smoke check and by the CPU-baseline leg of the benchmark, never by the
 * product path.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (sources):
 *  - The recurrence and its output: the Rodimus block paragraph of
 *    "ICLR 2025 | Rodimus*: ..." (CodeFuse article): at inference the block
 *    keeps a fixed-size hidden state updated once per token through a
 *    selection gate, a temperature gate and an input gate; q, k, v are the
 *    current token's query/key/value.  The formula itself is not printed on
 *    the page; the form used here is
 *        S_t = diag(a_t) S_{t-1} + (beta_t * k_t)^T v_t,   o_t = q_t S_t
 *    with S in R^{dk x dv} (rows = key channels).
 *  - The gate map (not printed on any page; our reading, see the gate section
 *    below): selection s = sigmoid(g), temperature tau = sigmoid(theta),
 *        a = s^tau,   beta = (1 - s)^tau,
 *    evaluated in log space:
 *        log a    = -tau * softplus(-g),
 *        log beta = -tau * softplus(g).
 *    tau_init = sigmoid(0) = 0.5 matches the "tempered_gate_init 0.5" entry of
 *    the module configuration in section 3 of the Rodimus* deployment blog
 *    (m.nxbn.cn/news/205411).
 *  - Sliding-window shared-key attention: the SKA and Rodimus+ paragraphs
 *    (Fig. 4) of the CodeFuse article (one key matrix shared by all heads,
 *    one value matrix per head, inside sliding-window attention), with
 *    softmax(q k^T / sqrt(d)) v from section 1.1 and "each query only sees
 *    the previous w keys" from section 2.1 of the MiniCPM-SALA blog
 *    (wzjinhao.cn/news/68323).
 *
 * Everything is fp64, one token at a time, no blocking or reordering.
 * The only concession to speed is that independent (batch, head) pairs (or
 * query rows, for attention) may be split over POSIX threads; each thread runs
 * exactly the same sequential loop on its own pairs.
 */
#include "rodimus_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ gates */

/* Logistic sigmoid, evaluated without overflow for either sign.
 * sigmoid(-inf) = 0 exactly, sigmoid(+inf) = 1 exactly. */
static double sigmoid(double x) {
    if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/* softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^{-|x|}). */
static double softplus(double x) {
    return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

void oracle_gates(const double *g, const double *theta, size_t n,
                  double *log_a, double *log_beta) {
    for (size_t i = 0; i < n; ++i) {
        double tau = sigmoid(theta[i]);
        /* tau == 0 (theta = -inf) gives a = beta = 1 exactly. */
        log_a[i] = (tau == 0.0) ? 0.0 : -tau * softplus(-g[i]);
        log_beta[i] = (tau == 0.0) ? 0.0 : -tau * softplus(g[i]);
    }
}

/* ---------------------------------------------------- low-rank gate logits */

/* silu(x) = x * sigmoid(x) */
static double silu(double x) { return x * sigmoid(x); }

/* The gate logits from rank-R factors (our reading: the Rodimus block
 * paragraph of the CodeFuse article computes the selection and temperature
 * gates from the token through learnable weights, and section 3 of the
 * Rodimus* deployment blog names SiLU as the selection gate's activation; the
 * projection itself is not printed).  Each token's hidden state has been
 * projected to two factor rows z_g, z_tau in R^R shared by all heads; per head
 * h and key channel c:
 *     g[b,h,t,c]     = sum_r silu(z_g[b,t,r]) U_g[h,c,r]   + b_g[h,c]
 *     theta[b,h,t,c] = sum_r      z_tau[b,t,r] U_tau[h,c,r] + b_tau[h,c]
 * Layouts: zg, zt [B,T,R]; Ug, Ut [H,dk,R]; bg, bt [H,dk]; g, theta
 * [B,H,T,dk]. */
int oracle_lowrank_gate_logits(int B, int H, int T, int dk, int R,
                               const double *zg, const double *zt,
                               const double *Ug, const double *bg,
                               const double *Ut, const double *bt,
                               double *g, double *theta) {
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || R <= 0) return -1;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int t = 0; t < T; ++t) {
                const double *zgt = zg + ((size_t)b * T + t) * R;
                const double *ztt = zt + ((size_t)b * T + t) * R;
                double *gt = g + (((size_t)b * H + h) * T + t) * dk;
                double *tht = theta + (((size_t)b * H + h) * T + t) * dk;
                for (int c = 0; c < dk; ++c) {
                    const double *ug = Ug + ((size_t)h * dk + c) * R;
                    const double *ut = Ut + ((size_t)h * dk + c) * R;
                    double sg = bg[(size_t)h * dk + c], st = bt[(size_t)h * dk + c];
                    for (int r = 0; r < R; ++r) {
                        sg += silu(zgt[r]) * ug[r];
                        st += ztt[r] * ut[r];
                    }
                    gt[c] = sg;
                    tht[c] = st;
                }
            }
    return 0;
}

/* --------------------------------------------------------------- the scan */

typedef struct {
    int B, H, T, dk, dv;
    const double *q, *k, *v, *g, *theta, *S0;
    double *o, *ST;
    int next; /* next (b,h) pair to take */
    pthread_mutex_t lock;
} scan_job;

/* One (b,h) pair: the definition, token by token. */
static void scan_one(const scan_job *J, int bh, double *S, double *a, double *bk) {
    const int T = J->T, dk = J->dk, dv = J->dv;
    const size_t xoff = (size_t)bh * T * dk, voff = (size_t)bh * T * dv;
    const size_t soff = (size_t)bh * dk * dv;
    if (J->S0) memcpy(S, J->S0 + soff, sizeof(double) * dk * dv);
    else memset(S, 0, sizeof(double) * dk * dv);
    for (int t = 0; t < T; ++t) {
        const double *qt = J->q + xoff + (size_t)t * dk;
        const double *kt = J->k + xoff + (size_t)t * dk;
        const double *gt = J->g + xoff + (size_t)t * dk;
        const double *ht = J->theta + xoff + (size_t)t * dk;
        const double *vt = J->v + voff + (size_t)t * dv;
        double *ot = J->o + voff + (size_t)t * dv;
        for (int i = 0; i < dk; ++i) {
            double la, lb;
            oracle_gates(gt + i, ht + i, 1, &la, &lb);
            a[i] = exp(la);
            bk[i] = exp(lb) * kt[i];
        }
        /* S <- diag(a) S + (beta*k)^T v */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[i * dv + j] = a[i] * S[i * dv + j] + bk[i] * vt[j];
        /* o_t = q_t S_t (the state after the update) */
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += qt[i] * S[i * dv + j];
            ot[j] = acc;
        }
    }
    if (J->ST) memcpy(J->ST + soff, S, sizeof(double) * dk * dv);
}

static void *scan_worker(void *arg) {
    scan_job *J = (scan_job *)arg;
    double *S = (double *)malloc(sizeof(double) * J->dk * J->dv);
    double *a = (double *)malloc(sizeof(double) * J->dk);
    double *bk = (double *)malloc(sizeof(double) * J->dk);
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int bh = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (bh >= J->B * J->H) break;
        scan_one(J, bh, S, a, bk);
    }
    free(S); free(a); free(bk);
    return NULL;
}

int oracle_scan(int B, int H, int T, int dk, int dv,
                const double *q, const double *k, const double *v,
                const double *g, const double *theta, const double *S0,
                double *o, double *ST, int nthreads) {
    if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
    scan_job J = {B, H, T, dk, dv, q, k, v, g, theta, S0, o, ST, 0,
                  PTHREAD_MUTEX_INITIALIZER};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > B * H) nthreads = B * H;
    if (nthreads == 1) { scan_worker(&J); return 0; }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, scan_worker, &J);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    return 0;
}

/* --------------------------------------------------- the scan, backward */

/* Gradients of L = sum(dO * o) + sum(dST * S_T) with respect to every input
 * of the scan, by reverse-mode differentiation of the definition above:
 *   S_t = diag(a_t) S_{t-1} + (beta_t * k_t)^T v_t,   o_t = q_t S_t.
 * With G_t the gradient of L with respect to S_t (G_T = dST, or 0):
 *   G_t    += q_t^T dO_t                       (o_t reads S_t)
 *   dq_t    = dO_t S_t^T
 *   da_t    = rowsum(G_t * S_{t-1}),   d(beta*k)_t = G_t v_t^T,   dv_t = (beta_t*k_t) G_t
 *   G_{t-1} = diag(a_t) G_t,           dS0 = G_0.
 * Gate chain rule (a = exp(-sigmoid(theta) softplus(-g)),
 * beta = exp(-sigmoid(theta) softplus(g)); sigmoid' = sigmoid(x) sigmoid(-x),
 * softplus' = sigmoid):
 *   da/dg     =  a    * sigmoid(theta) sigmoid(-g)
 *   dbeta/dg  = -beta * sigmoid(theta) sigmoid(g)
 *   da/dth    = -a    * sigmoid(theta) sigmoid(-theta) softplus(-g)
 *   dbeta/dth = -beta * sigmoid(theta) sigmoid(-theta) softplus(g)
 * All states S_0 .. S_T of a pair are kept (fp64), so memory is
 * (T + 1) * dk * dv doubles per thread. */
typedef struct {
    int B, H, T, dk, dv;
    const double *q, *k, *v, *g, *theta, *S0, *dO, *dST;
    double *dq, *dk_, *dv_, *dg, *dtheta, *dS0;
    int next;
    pthread_mutex_t lock;
} bwd_job;

static void bwd_one(const bwd_job *J, int bh, double *Sall, double *a, double *beta, double *G,
                    double *dbk) {
    const int T = J->T, dk = J->dk, dv = J->dv;
    const size_t xoff = (size_t)bh * T * dk, voff = (size_t)bh * T * dv;
    const size_t soff = (size_t)bh * dk * dv, ss = (size_t)dk * dv;
    /* forward, keeping every state: Sall[t] = S_t, S_0 = S0 */
    if (J->S0) memcpy(Sall, J->S0 + soff, sizeof(double) * ss);
    else memset(Sall, 0, sizeof(double) * ss);
    for (int t = 0; t < T; ++t) {
        const double *kt = J->k + xoff + (size_t)t * dk;
        const double *gt = J->g + xoff + (size_t)t * dk, *ht = J->theta + xoff + (size_t)t * dk;
        const double *vt = J->v + voff + (size_t)t * dv;
        double *at = a + (size_t)t * dk, *bt = beta + (size_t)t * dk;
        for (int i = 0; i < dk; ++i) {
            double la, lb;
            oracle_gates(gt + i, ht + i, 1, &la, &lb);
            at[i] = exp(la);
            bt[i] = exp(lb);
        }
        const double *Sp = Sall + (size_t)t * ss;
        double *Sn = Sall + (size_t)(t + 1) * ss;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                Sn[i * dv + j] = at[i] * Sp[i * dv + j] + bt[i] * kt[i] * vt[j];
    }
    /* reverse */
    if (J->dST) memcpy(G, J->dST + soff, sizeof(double) * ss);
    else memset(G, 0, sizeof(double) * ss);
    for (int t = T - 1; t >= 0; --t) {
        const double *qt = J->q + xoff + (size_t)t * dk, *kt = J->k + xoff + (size_t)t * dk;
        const double *gt = J->g + xoff + (size_t)t * dk, *ht = J->theta + xoff + (size_t)t * dk;
        const double *vt = J->v + voff + (size_t)t * dv, *dOt = J->dO + voff + (size_t)t * dv;
        const double *St = Sall + (size_t)(t + 1) * ss, *Sp = Sall + (size_t)t * ss;
        const double *at = a + (size_t)t * dk, *bt = beta + (size_t)t * dk;
        double *dqt = J->dq + xoff + (size_t)t * dk, *dkt = J->dk_ + xoff + (size_t)t * dk;
        double *dgt = J->dg + xoff + (size_t)t * dk, *dht = J->dtheta + xoff + (size_t)t * dk;
        double *dvt = J->dv_ + voff + (size_t)t * dv;
        /* o_t = q_t S_t */
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) acc += dOt[j] * St[i * dv + j];
            dqt[i] = acc;
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) G[i * dv + j] += qt[i] * dOt[j];
        /* S_t = diag(a_t) S_{t-1} + (beta_t k_t)^T v_t */
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += bt[i] * kt[i] * G[i * dv + j];
            dvt[j] = acc;
        }
        for (int i = 0; i < dk; ++i) {
            double da = 0.0, d_bk = 0.0;
            for (int j = 0; j < dv; ++j) {
                da += G[i * dv + j] * Sp[i * dv + j];
                d_bk += G[i * dv + j] * vt[j];
            }
            dbk[i] = d_bk;
            dkt[i] = bt[i] * d_bk;
            const double dbeta = kt[i] * d_bk;
            const double st = sigmoid(ht[i]), sg = sigmoid(gt[i]), sgm = sigmoid(-gt[i]);
            const double stm = sigmoid(-ht[i]);
            dgt[i] = da * at[i] * st * sgm - dbeta * bt[i] * st * sg;
            dht[i] = -st * stm * (da * at[i] * softplus(-gt[i]) + dbeta * bt[i] * softplus(gt[i]));
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) G[i * dv + j] *= at[i];
    }
    if (J->dS0) memcpy(J->dS0 + soff, G, sizeof(double) * ss);
}

static void *bwd_worker(void *arg) {
    bwd_job *J = (bwd_job *)arg;
    const size_t ss = (size_t)J->dk * J->dv;
    double *Sall = (double *)malloc(sizeof(double) * ss * (J->T + 1));
    double *a = (double *)malloc(sizeof(double) * ((size_t)J->T * J->dk + 1));
    double *beta = (double *)malloc(sizeof(double) * ((size_t)J->T * J->dk + 1));
    double *G = (double *)malloc(sizeof(double) * ss);
    double *dbk = (double *)malloc(sizeof(double) * J->dk);
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int bh = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (bh >= J->B * J->H) break;
        bwd_one(J, bh, Sall, a, beta, G, dbk);
    }
    free(Sall); free(a); free(beta); free(G); free(dbk);
    return NULL;
}

int oracle_scan_backward(int B, int H, int T, int dk, int dv,
                         const double *q, const double *k, const double *v,
                         const double *g, const double *theta, const double *S0,
                         const double *dO, const double *dST,
                         double *dq, double *dk_, double *dv_, double *dg, double *dtheta,
                         double *dS0, int nthreads) {
    if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
    bwd_job J = {B, H, T, dk, dv, q, k, v, g, theta, S0, dO, dST,
                 dq, dk_, dv_, dg, dtheta, dS0, 0, PTHREAD_MUTEX_INITIALIZER};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > B * H) nthreads = B * H;
    if (nthreads == 1) { bwd_worker(&J); return 0; }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, bwd_worker, &J);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    return 0;
}

/* ------------------------------------------------------------- the decode */

/* One recurrent step for N independent sequences: the same update as one
 * iteration of the scan, on a state that persists between calls.
 * S_out may alias S_in. */
int oracle_decode(int N, int H, int dk, int dv,
                  const double *q, const double *k, const double *v,
                  const double *g, const double *theta,
                  const double *S_in, double *o, double *S_out) {
    if (N <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    double *a = (double *)malloc(sizeof(double) * dk);
    double *bk = (double *)malloc(sizeof(double) * dk);
    for (int nh = 0; nh < N * H; ++nh) {
        const double *qt = q + (size_t)nh * dk, *kt = k + (size_t)nh * dk;
        const double *gt = g + (size_t)nh * dk, *ht = theta + (size_t)nh * dk;
        const double *vt = v + (size_t)nh * dv;
        const double *Si = S_in + (size_t)nh * dk * dv;
        double *So = S_out + (size_t)nh * dk * dv;
        double *ot = o + (size_t)nh * dv;
        for (int i = 0; i < dk; ++i) {
            double la, lb;
            oracle_gates(gt + i, ht + i, 1, &la, &lb);
            a[i] = exp(la);
            bk[i] = exp(lb) * kt[i];
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                So[i * dv + j] = a[i] * Si[i * dv + j] + bk[i] * vt[j];
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += qt[i] * So[i * dv + j];
            ot[j] = acc;
        }
    }
    free(a); free(bk);
    return 0;
}

/* ------------------------------------------------------------ SW-SKA */

typedef struct {
    int B, H, T, dk, dv, window;
    double scale;
    const double *q, *k, *v;
    double *o;
    const long long *rows; /* flat (b*H + h)*T + t indices, or NULL = all */
    long long nrows;
    long long next;
    pthread_mutex_t lock;
} ska_job;

/* One query row: dense softmax over the keys s in [max(0, t-w+1), t]. */
static void ska_row(const ska_job *J, long long r, double *p) {
    const int T = J->T, dk = J->dk, dv = J->dv, H = J->H;
    long long bh = r / T;
    int t = (int)(r % T);
    int b = (int)(bh / H);
    const double *qt = J->q + (size_t)r * dk;
    const double *kb = J->k + (size_t)b * T * dk; /* the one shared key matrix */
    const double *vb = J->v + (size_t)bh * T * dv; /* this head's values */
    double *ot = J->o + (size_t)r * dv;
    int s0 = t - J->window + 1;
    if (s0 < 0) s0 = 0;
    double m = -INFINITY;
    for (int s = s0; s <= t; ++s) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += qt[i] * kb[(size_t)s * dk + i];
        p[s - s0] = J->scale * acc;
        if (p[s - s0] > m) m = p[s - s0];
    }
    double den = 0.0;
    for (int s = s0; s <= t; ++s) {
        p[s - s0] = exp(p[s - s0] - m);
        den += p[s - s0];
    }
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int s = s0; s <= t; ++s) acc += p[s - s0] * vb[(size_t)s * dv + j];
        ot[j] = acc / den;
    }
}

static void *ska_worker(void *arg) {
    ska_job *J = (ska_job *)arg;
    double *p = (double *)malloc(sizeof(double) * (size_t)(J->window < J->T ? J->window : J->T));
    for (;;) {
        pthread_mutex_lock(&J->lock);
        long long i = J->next;
        J->next += 16;
        pthread_mutex_unlock(&J->lock);
        if (i >= J->nrows) break;
        long long e = i + 16 < J->nrows ? i + 16 : J->nrows;
        for (; i < e; ++i) ska_row(J, J->rows ? J->rows[i] : i, p);
    }
    free(p);
    return NULL;
}

int oracle_swska(int B, int H, int T, int dk, int dv, int window, double scale,
                 const double *q, const double *k_shared, const double *v,
                 double *o, const long long *rows, long long nrows, int nthreads) {
    if (B <= 0 || H <= 0 || T <= 0 || dk <= 0 || dv <= 0 || window <= 0) return -1;
    ska_job J = {B, H, T, dk, dv, window, scale, q, k_shared, v, o, rows,
                 rows ? nrows : (long long)B * H * T, 0, PTHREAD_MUTEX_INITIALIZER};
    if (nthreads < 1) nthreads = 1;
    if (nthreads == 1) { ska_worker(&J); return 0; }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, ska_worker, &J);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    return 0;
}
