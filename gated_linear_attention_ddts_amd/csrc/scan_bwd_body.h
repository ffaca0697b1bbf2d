// scan_bwd_body.h -- exact per-chunk backward of the DDTS-gated scan on the
// vector ALUs (fp32 arithmetic, pairwise decay weights).  Used by the generic
// backward for every chunk and by the matrix-core backward for the chunks
// whose decay span is too wide for its factored operands.
//
// The forward recurrence (CodeFuse article, Rodimus block paragraph; the gate
// map is in device_common.h):
//     S_t = diag(a_t) S_{t-1} + (beta_t * k_t)^T v_t,     o_t = q_t S_t.
// In natural-log units, with lam = log a, mu = log beta, Lam_t the inclusive
// in-chunk cumulative sum of lam, Gam = Lam_{C-1}, S the state entering the
// chunk and G the gradient of the state leaving it (from later tokens):
//
//   intra-chunk pairs j <= i, weight w_ij = exp(Lam_i - Lam_j + mu_j) <= 1:
//     dP_ij = dO_i . v_j,    A_ij = sum_r q_i[r] k_j[r] w_ij[r]
//     dq_i += sum_j dP_ij k_j w_ij,   dk_j += sum_i dP_ij q_i w_ij,
//     dv_j += sum_i A_ij dO_i
//   through the entering state:    dq_i += exp(Lam_i) * (S dO_i^T)
//   through the leaving state, with Kb_j = k_j exp(Gam - Lam_j + mu_j):
//     dk_j += exp(Gam - Lam_j + mu_j) * (G v_j^T),   dv_j += Kb_j G
//   exponent gradients (d/dx of c * exp(x) is the term itself):
//     dLam_i = q_i dq_i - k_i dk_i(intra) - Kb_i (G v_i^T),
//     dmu_j  = k_j dk_j(intra) + Kb_j (G v_j^T),
//     dGam   = sum_j Kb_j (G v_j^T) + exp(Gam) * rowsum(G * S),
//     dlam_t = sum_{t' >= t} dLam_t' + dGam,
// then the chain rule through the gate map gives dg and dtau.  The weights
// w_ij are evaluated pairwise, so no exponent ever exceeds 0.
#pragma once
#include "device_common.h"

namespace rodimus {

constexpr int kBC = 32;      // tokens per backward chunk
constexpr int kBD = 128;     // largest dk / dv

// Gradients of the natural-log gates (dla = dL/dlog a, dlb = dL/dlog beta)
// through log a = -sigmoid(th) softplus(-g), log beta = -sigmoid(th) softplus(g):
//   dg  = dla sigmoid(th) sigmoid(-g) - dlb sigmoid(th) sigmoid(g)
//   dth = -sigmoid(th) sigmoid(-th) (dla softplus(-g) + dlb softplus(g))
__device__ __forceinline__ void ddts_gate_grads(float g, float th, float dla, float dlb, float &dg,
                                                float &dth) {
    const float xt = exp2_fast(-fabsf(th) * kLog2e);                 // e^{-|th|}
    const float rt = __builtin_amdgcn_rcpf(1.f + xt);
    const float tau = (th >= 0.f ? 1.f : xt) * rt;                  // sigmoid(th)
    const float dtau = xt * rt * rt;                                // sigmoid(th) sigmoid(-th)
    const float x = exp2_fast(-fabsf(g) * kLog2e);                  // e^{-|g|}
    const float u = 1.f + x, ru = __builtin_amdgcn_rcpf(u);
    // log1p(x) as log(u) * x / (u - 1) (exact when u == 1); the hardware
    // reciprocal's 1-ulp error is far below the gradients' tolerance
    const float L = (u == 1.f) ? x : log2_fast(u) * kLn2 * (x * __builtin_amdgcn_rcpf(u - 1.f));
    const float spn = fmaxf(-g, 0.f) + L, spp = fmaxf(g, 0.f) + L;  // softplus(-g), softplus(g)
    const float sp_ = (g >= 0.f) ? ru : x * ru;                     // sigmoid(g)
    const float sn_ = (g >= 0.f) ? x * ru : ru;                     // sigmoid(-g)
    dg = tau * (dla * sn_ - dlb * sp_);
    dth = -dtau * (dla * spn + dlb * spp);
}

// Rows of sequence-head bh = s * H + h.  cu == nullptr: the batched layout,
// rows bh * T .. bh * T + T - 1.  Otherwise the packed layout: sequence s takes
// rows cu[s] .. cu[s+1] - 1 of head h's [total] rows, the span clamped to
// [0, total] and to T (the longest length), so that a malformed table cannot
// address memory outside the tensors.  bh must be wave-uniform; so are the
// results.
__device__ __forceinline__ void seq_rows(const int *cu, int H, int total, int T, int bh, size_t &row0,
                                         int &len) {
    if (cu == nullptr) {
        row0 = (size_t)bh * T;
        len = T;
        return;
    }
    const int s = bh / H, h = bh - s * H;
    const int a = min(max(__builtin_amdgcn_readfirstlane(cu[s]), 0), total);
    const int b = min(max(__builtin_amdgcn_readfirstlane(cu[s + 1]), a), total);
    row0 = (size_t)h * total + a;
    len = min(b - a, T);
}

// Cooperative: natural-log gates of chunk tokens [t0, t0 + L) of one (b,h)
// into lam / mu ([kBC][dk]); lam becomes the inclusive cumulative sum over the
// chunk.  Tokens past L get lam = 0, mu = -inf.  256 threads.
template <typename Tin>
__device__ __forceinline__ void chunk_gates(const Tin *g, const Tin *th, size_t xbase, int t0, int L, int dk,
                                            float *lam, float *mu) {
    for (int e = threadIdx.x; e < kBC * dk; e += blockDim.x) {
        const int t = e / dk, r = e % dk;
        float la = 0.f, lb = -INFINITY;
        if (t < L) {
            const size_t x = xbase + (size_t)(t0 + t) * dk + r;
            ddts_log_gates(Elem<Tin>::ld(g, x), Elem<Tin>::ld(th, x), la, lb);
        }
        lam[t * kBD + r] = la;
        mu[t * kBD + r] = lb;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < dk; r += blockDim.x) {
        float run = 0.f;
        for (int t = 0; t < kBC; ++t) {
            run += lam[t * kBD + r];
            lam[t * kBD + r] = run;
        }
    }
    __syncthreads();
}

// The gradients of one chunk of kBC tokens (t0 = c * kBC) of one sequence
// whose len tokens occupy rows row0 .. row0+len-1 of the [rows][dk] / [rows][dv]
// tensors, given S, the state entering the chunk, and G, the gradient of the
// state leaving it (both fp32 [dk][dv], row-major).  256 threads; per-element
// work maps thread -> channel r = tid % 128 and tokens tid / 128 + 2m.  smem
// holds kBodyFloats floats; the caller synchronises before reusing it.
constexpr int kBodyFloats = 8 * kBC * kBD + 2 * kBC * kBC + 2 * kBD;

template <typename Tin>
__device__ __forceinline__ void chunk_grads_body(
    const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v, const Tin *__restrict__ g,
    const Tin *__restrict__ th, const Tin *__restrict__ dO, const float *__restrict__ S,
    const float *__restrict__ G, float *__restrict__ dq, float *__restrict__ dk_, float *__restrict__ dv_,
    float *__restrict__ dg, float *__restrict__ dth, size_t row0, int len, int dk, int dv, int c, float *smem) {
    float *Q = smem, *K = Q + kBC * kBD, *V = K + kBC * kBD, *DO = V + kBC * kBD;
    float *lam = DO + kBC * kBD, *mu = lam + kBC * kBD, *X1 = mu + kBC * kBD, *X2 = X1 + kBC * kBD;
    float *dP = X2 + kBC * kBD, *A = dP + kBC * kBC, *dGam = A + kBC * kBC, *dGam2 = dGam + kBD;
    const int tid = threadIdx.x;
    const int t0 = c * kBC, L = min(kBC, len - t0);
    const size_t xbase = row0 * dk, vbase = row0 * dv;

    // P1: inputs (zero past L) and gates
    for (int e = tid; e < kBC * dk; e += 256) {
        const int t = e / dk, r = e % dk;
        const size_t x = xbase + (size_t)(t0 + t) * dk + r;
        Q[t * kBD + r] = t < L ? Elem<Tin>::ld(q, x) : 0.f;
        K[t * kBD + r] = t < L ? Elem<Tin>::ld(k, x) : 0.f;
    }
    for (int e = tid; e < kBC * dv; e += 256) {
        const int t = e / dv, n = e % dv;
        const size_t x = vbase + (size_t)(t0 + t) * dv + n;
        V[t * kBD + n] = t < L ? Elem<Tin>::ld(v, x) : 0.f;
        DO[t * kBD + n] = t < L ? Elem<Tin>::ld(dO, x) : 0.f;
    }
    chunk_gates<Tin>(g, th, xbase, t0, L, dk, lam, mu);   // ends with a barrier

    // P2: dP_ij = dO_i . v_j and A_ij = sum_r q_i k_j w_ij, for j <= i (else 0)
    for (int e = tid; e < kBC * kBC; e += 256) {
        const int i = e / kBC, jj = e % kBC;
        float p = 0.f, a = 0.f;
        if (jj <= i && i < L) {
            for (int n = 0; n < dv; ++n) p = fmaf(DO[i * kBD + n], V[jj * kBD + n], p);
            for (int r = 0; r < dk; ++r)
                a = fmaf(Q[i * kBD + r] * K[jj * kBD + r],
                         __expf(lam[i * kBD + r] - lam[jj * kBD + r] + mu[jj * kBD + r]), a);
        }
        dP[e] = p;
        A[e] = a;
    }
    // P3: through the states: X1[t][r] = (S dO_t^T)[r], X2[t][r] = (G v_t^T)[r];
    // decay term exp(Gam_r) sum_n G[r][n] S[r][n]
    {
        const int r = tid & 127, half = tid >> 7;
        if (r < dk) {
            float x1[16], x2[16], dec = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) { x1[m] = 0.f; x2[m] = 0.f; }
            for (int n = 0; n < dv; n += 4) {
                const float4 s4 = *reinterpret_cast<const float4 *>(S + (size_t)r * dv + n);
                const float4 g4 = *reinterpret_cast<const float4 *>(G + (size_t)r * dv + n);
                if (half == 0) dec += g4.x * s4.x + g4.y * s4.y + g4.z * s4.z + g4.w * s4.w;
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    const int t = half + 2 * m;
                    const float4 d4 = *reinterpret_cast<const float4 *>(DO + t * kBD + n);
                    const float4 v4 = *reinterpret_cast<const float4 *>(V + t * kBD + n);
                    x1[m] += d4.x * s4.x + d4.y * s4.y + d4.z * s4.z + d4.w * s4.w;
                    x2[m] += v4.x * g4.x + v4.y * g4.y + v4.z * g4.z + v4.w * g4.w;
                }
            }
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int t = half + 2 * m;
                X1[t * kBD + r] = x1[m];
                X2[t * kBD + r] = x2[m];
            }
            if (half == 0) dGam2[r] = dec;
        }
    }
    __syncthreads();

    // P4: per element (t, r): dq, dk, exponent gradients
    const int r = tid & 127, half = tid >> 7;
    float kbar[16], ebs = 0.f;
    if (r < dk) {
        const float Gam = lam[(kBC - 1) * kBD + r];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int t = half + 2 * m;
            kbar[m] = 0.f;
            if (t >= L) continue;
            const float lt = lam[t * kBD + r], mt = mu[t * kBD + r];
            float dqi = 0.f, dki = 0.f;
            for (int jj = 0; jj <= t; ++jj)
                dqi = fmaf(dP[t * kBC + jj] * K[jj * kBD + r], __expf(lt - lam[jj * kBD + r] + mu[jj * kBD + r]), dqi);
            for (int i = t; i < L; ++i)
                dki = fmaf(dP[i * kBC + t] * Q[i * kBD + r], __expf(lam[i * kBD + r] - lt + mt), dki);
            const float eq = __expf(lt), kbs = __expf(Gam - lt + mt);
            const float dqt = dqi + X1[t * kBD + r] * eq;
            const float dkt = dki + X2[t * kBD + r] * kbs;
            const size_t x = xbase + (size_t)(t0 + t) * dk + r;
            dq[x] = dqt;
            dk_[x] = dkt;
            const float kb = K[t * kBD + r] * kbs;
            const float eb = X2[t * kBD + r] * kb;
            const float ek = K[t * kBD + r] * dki;
            kbar[m] = kb;
            ebs += eb;
            X1[t * kBD + r] = Q[t * kBD + r] * dqt - ek - eb;   // dLam_t
            X2[t * kBD + r] = ek + eb;                           // dmu_t
        }
    }
    if (half == 1 && r < dk) dGam[r] = ebs;
    __syncthreads();
    // P5: Kb into K; dGam; reverse cumulative sum dlam_t = sum_{t'>=t} dLam_t' + dGam
    if (r < dk) {
#pragma unroll
        for (int m = 0; m < 16; ++m) K[(half + 2 * m) * kBD + r] = kbar[m];
        if (half == 0) {
            const float Gam = lam[(kBC - 1) * kBD + r];
            const float dG = ebs + dGam[r] + __expf(Gam) * dGam2[r];
            float run = 0.f;
            for (int t = L - 1; t >= 0; --t) {
                run += X1[t * kBD + r];
                X1[t * kBD + r] = run + dG;
            }
        }
    }
    __syncthreads();
    // P6: gate chain rule; dv
    if (r < dk) {
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int t = half + 2 * m;
            if (t >= L) continue;
            const size_t x = xbase + (size_t)(t0 + t) * dk + r;
            float dgx, dthx;
            ddts_gate_grads(Elem<Tin>::ld(g, x), Elem<Tin>::ld(th, x), X1[t * kBD + r], X2[t * kBD + r], dgx, dthx);
            dg[x] = dgx;
            dth[x] = dthx;
        }
    }
    {
        const int n = tid & 127;
        if (n < dv) {
            float acc[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) acc[m] = 0.f;
            for (int rr = 0; rr < dk; ++rr) {
                const float gn = G[(size_t)rr * dv + n];
#pragma unroll
                for (int m = 0; m < 16; ++m) acc[m] = fmaf(K[(half + 2 * m) * kBD + rr], gn, acc[m]);
            }
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int t = half + 2 * m;
                if (t >= L) continue;
                float a = acc[m];
                for (int i = t; i < L; ++i) a = fmaf(A[i * kBC + t], DO[i * kBD + n], a);
                dv_[vbase + (size_t)(t0 + t) * dv + n] = a;
            }
        }
    }
}

}  // namespace rodimus
