// scan_bwd.hip -- generic backward of the chunked DDTS-gated scan (fp32
// arithmetic, any dk, dv that are multiples of 16 up to 128, fp32 or bf16
// inputs).  The per-chunk mathematics is in scan_bwd_body.h.
//
// Three kernels over chunks of kBC = 32 tokens:
//   bwd_states_fwd: the state entering every chunk (checkpoints), a forward
//       pass over chunks with S <- diag(exp Gam) S + Kb^T V;
//   bwd_states_rev: the gradient of the state leaving every chunk, a reverse
//       pass with G <- diag(exp Gam) G + Qt^T dO (Qt_i = q_i exp(Lam_i)); its
//       final value is dS0;
//   bwd_chunk_grads: every chunk independently, from its checkpoint pair.
// Both state passes: one workgroup per (b,h, 64 state columns); wave w owns
// state rows 32w .. 32w+31, lane = column.  In the packed layout (cu non-null)
// every sequence runs over its own rows and chunks only (seq_rows).
#include "launch.h"
#include "scan_bwd_body.h"

namespace rodimus {

namespace {

constexpr int kCols = 64;    // state columns per state-pass workgroup

// Forward state pass: Sck[bh][c] = state entering chunk c.
template <typename Tin>
__global__ __launch_bounds__(256)
void bwd_states_fwd(const Tin *__restrict__ k, const Tin *__restrict__ v, const Tin *__restrict__ g,
                    const Tin *__restrict__ th, const float *__restrict__ S0, float *__restrict__ Sck,
                    int T, int dk, int dv, int nck, const int *cu, int H, int total) {
    __shared__ float lam[kBC * kBD], mu[kBC * kBD], kb[kBC * kBD], vs[kBC * kCols];
    const int bh = blockIdx.x, w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int j = blockIdx.y * kCols + l;          // state column
    const bool col = j < dv;
    size_t row0;
    int len;
    seq_rows(cu, H, total, T, bh, row0, len);
    const size_t xbase = row0 * dk, vbase = row0 * dv;
    const int ncl = (len + kBC - 1) / kBC;         // this sequence's chunks
    float S[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const int r = 32 * w + i;
        S[i] = (S0 && col && r < dk) ? S0[((size_t)bh * dk + r) * dv + j] : 0.f;
    }
    for (int c = 0; c < ncl; ++c) {
        const int t0 = c * kBC, L = min(kBC, len - t0);
        float *ck = Sck + ((size_t)bh * nck + c) * dk * dv;
        if (col) {
#pragma unroll
            for (int i = 0; i < 32; ++i)
                if (32 * w + i < dk) ck[(size_t)(32 * w + i) * dv + j] = S[i];
        }
        chunk_gates<Tin>(g, th, xbase, t0, L, dk, lam, mu);
        // Kb[t][r] = k exp(Gam - Lam_t + mu_t) (<= |k|), v tile of this block's columns
        for (int e = threadIdx.x; e < kBC * dk; e += 256) {
            const int t = e / dk, r = e % dk;
            kb[t * kBD + r] = t < L ? Elem<Tin>::ld(k, xbase + (size_t)(t0 + t) * dk + r) *
                                          __expf(lam[(kBC - 1) * kBD + r] - lam[t * kBD + r] + mu[t * kBD + r])
                                    : 0.f;
        }
        for (int e = threadIdx.x; e < kBC * kCols; e += 256) {
            const int t = e / kCols, jj = blockIdx.y * kCols + e % kCols;
            vs[e] = (t < L && jj < dv) ? Elem<Tin>::ld(v, vbase + (size_t)(t0 + t) * dv + jj) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int r = min(32 * w + i, dk - 1);
            float x = S[i] * __expf(lam[(kBC - 1) * kBD + r]);
            for (int t = 0; t < L; ++t) x = fmaf(kb[t * kBD + r], vs[t * kCols + l], x);
            S[i] = x;
        }
        __syncthreads();
    }
}

// Reverse state pass: Gck[bh][c] = gradient of the state leaving chunk c from
// the tokens after it; dS0 = the gradient entering chunk 0.
template <typename Tin>
__global__ __launch_bounds__(256)
void bwd_states_rev(const Tin *__restrict__ q, const Tin *__restrict__ g, const Tin *__restrict__ th,
                    const Tin *__restrict__ dO, const float *__restrict__ dST, float *__restrict__ Gck,
                    float *__restrict__ dS0, int T, int dk, int dv, int nck, const int *cu, int H, int total) {
    __shared__ float lam[kBC * kBD], mu[kBC * kBD], qt[kBC * kBD], ds[kBC * kCols];
    const int bh = blockIdx.x, w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int j = blockIdx.y * kCols + l;
    const bool col = j < dv;
    size_t row0;
    int len;
    seq_rows(cu, H, total, T, bh, row0, len);
    const size_t xbase = row0 * dk, vbase = row0 * dv;
    const int ncl = (len + kBC - 1) / kBC;
    float G[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const int r = 32 * w + i;
        G[i] = (dST && col && r < dk) ? dST[((size_t)bh * dk + r) * dv + j] : 0.f;
    }
    for (int c = ncl - 1; c >= 0; --c) {
        const int t0 = c * kBC, L = min(kBC, len - t0);
        float *ck = Gck + ((size_t)bh * nck + c) * dk * dv;
        if (col) {
#pragma unroll
            for (int i = 0; i < 32; ++i)
                if (32 * w + i < dk) ck[(size_t)(32 * w + i) * dv + j] = G[i];
        }
        chunk_gates<Tin>(g, th, xbase, t0, L, dk, lam, mu);
        for (int e = threadIdx.x; e < kBC * dk; e += 256) {
            const int t = e / dk, r = e % dk;
            qt[t * kBD + r] = t < L ? Elem<Tin>::ld(q, xbase + (size_t)(t0 + t) * dk + r) * __expf(lam[t * kBD + r])
                                    : 0.f;
        }
        for (int e = threadIdx.x; e < kBC * kCols; e += 256) {
            const int t = e / kCols, jj = blockIdx.y * kCols + e % kCols;
            ds[e] = (t < L && jj < dv) ? Elem<Tin>::ld(dO, vbase + (size_t)(t0 + t) * dv + jj) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int r = min(32 * w + i, dk - 1);
            float x = G[i] * __expf(lam[(kBC - 1) * kBD + r]);
            for (int t = 0; t < L; ++t) x = fmaf(qt[t * kBD + r], ds[t * kCols + l], x);
            G[i] = x;
        }
        __syncthreads();
    }
    if (dS0 && col) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
            if (32 * w + i < dk) dS0[((size_t)bh * dk + 32 * w + i) * dv + j] = G[i];
    }
}

// Every chunk independently, from its checkpoint pair.
template <typename Tin>
__global__ __launch_bounds__(256)
void bwd_chunk_grads(const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ v,
                     const Tin *__restrict__ g, const Tin *__restrict__ th, const Tin *__restrict__ dO,
                     const float *__restrict__ Sck, const float *__restrict__ Gck,
                     float *__restrict__ dq, float *__restrict__ dk_, float *__restrict__ dv_,
                     float *__restrict__ dg, float *__restrict__ dth, int T, int dk, int dv, int nck,
                     const int *cu, int H, int total) {
    __shared__ float smem[kBodyFloats];
    const int bh = blockIdx.x / nck, c = blockIdx.x % nck;
    size_t row0;
    int len;
    seq_rows(cu, H, total, T, bh, row0, len);
    if (c * kBC >= len) return;
    const size_t off = ((size_t)bh * nck + c) * dk * dv;
    chunk_grads_body<Tin>(q, k, v, g, th, dO, Sck + off, Gck + off, dq, dk_, dv_, dg, dth, row0, len, dk, dv, c,
                          smem);
}

}  // namespace

int scan_bwd_chunks(int T) { return (T + kBC - 1) / kBC; }

size_t scan_bwd_workspace(int B, int H, int T, int dk, int dv) {
    return 2 * (size_t)B * H * scan_bwd_chunks(T) * dk * dv * sizeof(float);
}

uint64_t scan_bwd_launch_items(long long BH, int T) {
    const uint64_t a = (uint64_t)BH * 256, b = (uint64_t)BH * scan_bwd_chunks(T) * 256;
    return a > b ? a : b;
}

template <typename Tin>
static void launch_bwd_t(const ScanBwdArgs &a, hipStream_t st) {
    const int BH = a.B * a.H, nck = scan_bwd_chunks(a.T);
    float *Sck = reinterpret_cast<float *>(a.workspace);
    float *Gck = Sck + (size_t)BH * nck * a.dk * a.dv;
    const dim3 gs((unsigned)BH, (unsigned)((a.dv + kCols - 1) / kCols));
    hipLaunchKernelGGL(bwd_states_fwd<Tin>, gs, dim3(256), 0, st, (const Tin *)a.k, (const Tin *)a.v,
                       (const Tin *)a.g, (const Tin *)a.tau, a.S0, Sck, a.T, a.dk, a.dv, nck, a.cu, a.H, a.total);
    hipLaunchKernelGGL(bwd_states_rev<Tin>, gs, dim3(256), 0, st, (const Tin *)a.q, (const Tin *)a.g,
                       (const Tin *)a.tau, (const Tin *)a.dO, a.dS_T, Gck, a.dS0, a.T, a.dk, a.dv, nck, a.cu,
                       a.H, a.total);
    hipLaunchKernelGGL(bwd_chunk_grads<Tin>, dim3((unsigned)((size_t)BH * nck)), dim3(256), 0, st,
                       (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v, (const Tin *)a.g,
                       (const Tin *)a.tau, (const Tin *)a.dO, Sck, Gck, a.dq, a.dk_, a.dv_, a.dg, a.dtau,
                       a.T, a.dk, a.dv, nck, a.cu, a.H, a.total);
}

void launch_scan_bwd(const ScanBwdArgs &a, hipStream_t st) {
    if (a.dtype == 1) launch_bwd_t<bf16_t>(a, st);
    else launch_bwd_t<float>(a, st);
}

}  // namespace rodimus
