/*
 * rodimus_oracle.h -- fp64 CPU oracle for the Rodimus* token mixer.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU baseline of the bench).
 * All arrays are contiguous, row-major fp64:
 *   q, k, g, theta : [B, H, T, dk]     v, o : [B, H, T, dv]
 *   S0, ST          : [B, H, dk, dv]   (S0 may be NULL = zeros, ST may be NULL)
 *   decode tensors  : [N, H, .],  S [N, H, dk, dv]
 *   SW-SKA          : q [B,H,T,dk], k_shared [B,T,dk], v/o [B,H,T,dv]
 * Functions return 0, or -1 on a non-positive size.
 */
#ifndef RODIMUS_ORACLE_H
#define RODIMUS_ORACLE_H
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* log a = -sigmoid(theta) softplus(-g),  log beta = -sigmoid(theta) softplus(g) */
void oracle_gates(const double *g, const double *theta, size_t n,
                  double *log_a, double *log_beta);

/* Gate logits from rank-R factors shared by the heads:
 *   g = silu(zg) Ug^T + bg,  theta = zt Ut^T + bt   (per head h, channel c)
 * zg, zt [B,T,R]; Ug, Ut [H,dk,R]; bg, bt [H,dk]; g, theta [B,H,T,dk]. */
int oracle_lowrank_gate_logits(int B, int H, int T, int dk, int R,
                               const double *zg, const double *zt,
                               const double *Ug, const double *bg,
                               const double *Ut, const double *bt,
                               double *g, double *theta);

/* Sequential recurrence over T tokens for every (b,h); nthreads splits (b,h). */
int oracle_scan(int B, int H, int T, int dk, int dv,
                const double *q, const double *k, const double *v,
                const double *g, const double *theta, const double *S0,
                double *o, double *ST, int nthreads);

/* Gradients of sum(dO * o) + sum(dST * S_T) with respect to q, k, v, g, theta
 * and S0 (reverse-mode through the definition).  S0, dST may be NULL (zeros);
 * dS0 may be NULL (not returned).  dO: [B,H,T,dv]; outputs shaped like the
 * inputs. */
int oracle_scan_backward(int B, int H, int T, int dk, int dv,
                         const double *q, const double *k, const double *v,
                         const double *g, const double *theta, const double *S0,
                         const double *dO, const double *dST,
                         double *dq, double *dk_, double *dv_, double *dg, double *dtheta,
                         double *dS0, int nthreads);

/* One recurrent step on N x H states; S_out may alias S_in. */
int oracle_decode(int N, int H, int dk, int dv,
                  const double *q, const double *k, const double *v,
                  const double *g, const double *theta,
                  const double *S_in, double *o, double *S_out);

/* Sliding-window shared-key attention.  rows: optional list of flat query
 * indices (b*H + h)*T + t to compute (others in o are left untouched);
 * NULL computes every row. */
int oracle_swska(int B, int H, int T, int dk, int dv, int window, double scale,
                 const double *q, const double *k_shared, const double *v,
                 double *o, const long long *rows, long long nrows, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
