// scan_generic.hip -- chunkwise-parallel prefill, fp32 VALU arithmetic, any
// dk, dv (multiples of 16 up to 128), fp32 or bf16 inputs.
//
// This is the fp32 path and the path for shapes outside the MFMA kernel.  It
// computes the same chunk algebra as the MFMA kernel, entirely in fp32:
// per chunk of L <= C tokens entering with state S, with Lam[t] the inclusive
// in-chunk cumulative sum of log2 a (base-2 units throughout),
//     Qt[t] = q[t] * 2^{Lam[t]}            Kh[t] = k[t] * 2^{log2 beta[t] - Lam[t]}
//     o[t]  = Qt[t] S + sum_{s<=t} (Qt[t] . Kh[s]) v[s]
//     S'    = diag(2^{Lam[L-1]}) S + Kb^T V,   Kb[t] = Kh[t] * 2^{Lam[L-1]}
// (the chunkwise-parallel form of the recurrence, CodeFuse article, Rodimus
// block paragraph).  The factorisation needs 2^{-Lam} to stay finite; a chunk
// whose decay span max_i(-Lam[L-1, i]) exceeds kSpanLimit2 is instead run
// token by token, which gives the same result without overflow.
//
// Grid: (B*H, ceil(dv/64)); one 64-lane wave per workgroup, lane = state
// column.  Each lane holds its column of S (DK floats) in registers for the
// whole sequence; the chunk operands live in LDS.
#include "device_common.h"
#include "launch.h"

namespace rodimus {

constexpr float kSpanLimit2 = 112.f;  // log2 units: 2^112 ~ 5e33 stays finite in fp32/bf16
constexpr int kGenCols = 64;
constexpr int kGenMaxC = 64;

template <typename Tin, int DK>
__global__ __launch_bounds__(64)
void scan_generic_kernel(const Tin *__restrict__ q, const Tin *__restrict__ k,
                         const Tin *__restrict__ v, const Tin *__restrict__ g,
                         const Tin *__restrict__ th, const float *__restrict__ S0,
                         Tin *__restrict__ o, float *__restrict__ S_T,
                         int Tmax, int dv, int C, const int *__restrict__ cu, int H, int total) {
    __shared__ float bufQ[kGenMaxC * DK];       // log2 a, then Lam, then Qt
    __shared__ float bufK[kGenMaxC * DK];       // log2 beta, then Kh, then Kb
    __shared__ float bufV[kGenMaxC * kGenCols];  // v tile (this block's columns)
    __shared__ float bufA[kGenMaxC * kGenMaxC];  // masked Qt Kh^T
    __shared__ float gam[DK];                   // Lam[L-1] (log2), then 2^{Lam[L-1]}
    __shared__ int fallback;

    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int j = blockIdx.y * kGenCols + tid;
    const bool active = j < dv;
    // rows of (b,h): batched [B][H][T], or a packed sequence (bh = s * H + h,
    // rows cu[s] .. cu[s+1]-1 of head h, clamped to [0, total] and Tmax)
    size_t row0 = (size_t)bh * Tmax;
    int T = Tmax;
    if (cu) {
        const int s = bh / H, h = bh - s * H;
        const int a = min(max(cu[s], 0), total), b = min(max(cu[s + 1], a), total);
        row0 = (size_t)h * total + a;
        T = min(b - a, Tmax);
    }
    const size_t xbase = row0 * DK;
    const size_t vbase = row0 * dv;

    float S[DK];
#pragma unroll
    for (int i = 0; i < DK; ++i)
        S[i] = (S0 && active) ? S0[(size_t)bh * DK * dv + (size_t)i * dv + j] : 0.f;

    for (int c0 = 0; c0 < T; c0 += C) {
        const int L = min(C, T - c0);
        if (tid == 0) fallback = 0;
        // 1. gates (log2 units) and the v tile
        for (int e = tid; e < L * DK; e += 64) {
            size_t x = xbase + (size_t)c0 * DK + e;
            float l2a, l2b;
            ddts_log2_gates(Elem<Tin>::ld(g, x), Elem<Tin>::ld(th, x), l2a, l2b);
            bufQ[e] = l2a;
            bufK[e] = l2b;
        }
        for (int e = tid; e < L * kGenCols; e += 64) {
            int t = e / kGenCols, jj = blockIdx.y * kGenCols + e % kGenCols;
            bufV[e] = jj < dv ? Elem<Tin>::ld(v, vbase + (size_t)(c0 + t) * dv + jj) : 0.f;
        }
        __syncthreads();
        // 2. in-chunk inclusive cumulative sum per key channel
        for (int i = tid; i < DK; i += 64) {
            float run = 0.f;
            for (int t = 0; t < L; ++t) {
                run += bufQ[t * DK + i];
                bufQ[t * DK + i] = run;
            }
            gam[i] = run;
            if (run < -kSpanLimit2) fallback = 1;
        }
        __syncthreads();
        if (!fallback) {
            // 3. operands
            for (int e = tid; e < L * DK; e += 64) {
                size_t x = xbase + (size_t)c0 * DK + e;
                float lam = bufQ[e];
                bufQ[e] = Elem<Tin>::ld(q, x) * exp2_fast(lam);
                bufK[e] = Elem<Tin>::ld(k, x) * exp2_fast(bufK[e] - lam);
            }
            __syncthreads();
            for (int i = tid; i < DK; i += 64) gam[i] = exp2_fast(gam[i]);
            // 4. A = tril(Qt Kh^T)
            for (int p = tid; p < L * L; p += 64) {
                int t = p / L, s = p % L;
                float acc = 0.f;
                if (s <= t) {
#pragma unroll 8
                    for (int i = 0; i < DK; ++i) acc = fmaf(bufQ[t * DK + i], bufK[s * DK + i], acc);
                }
                bufA[t * kGenMaxC + s] = acc;
            }
            __syncthreads();
            // 5. outputs o[t] = Qt[t] S + sum_{s<=t} A[t,s] v[s]
            if (active) {
                for (int t = 0; t < L; ++t) {
                    float acc = 0.f;
#pragma unroll
                    for (int i = 0; i < DK; ++i) acc = fmaf(bufQ[t * DK + i], S[i], acc);
                    for (int s = 0; s <= t; ++s) acc = fmaf(bufA[t * kGenMaxC + s], bufV[s * kGenCols + tid], acc);
                    Elem<Tin>::st(o, vbase + (size_t)(c0 + t) * dv + j, acc);
                }
            }
            // 6. S <- diag(gamma) S + Kb^T V with Kb = Kh * gamma
#pragma unroll
            for (int i = 0; i < DK; ++i) S[i] *= gam[i];
            for (int t = 0; t < L; ++t) {
                const float vt = bufV[t * kGenCols + tid];
#pragma unroll
                for (int i = 0; i < DK; ++i) S[i] = fmaf(bufK[t * DK + i] * gam[i], vt, S[i]);
            }
        } else {
            // Token-by-token fallback: recompute log2 a / log2 beta (the cumsum
            // overwrote log2 a) and run the recurrence directly.
            __syncthreads();
            for (int e = tid; e < L * DK; e += 64) {
                size_t x = xbase + (size_t)c0 * DK + e;
                float l2a, l2b;
                ddts_log2_gates(Elem<Tin>::ld(g, x), Elem<Tin>::ld(th, x), l2a, l2b);
                bufQ[e] = exp2_fast(l2a);
                bufK[e] = exp2_fast(l2b) * Elem<Tin>::ld(k, x);
            }
            __syncthreads();
            for (int t = 0; t < L; ++t) {
                const float vt = bufV[t * kGenCols + tid];
                const size_t x = xbase + (size_t)(c0 + t) * DK;
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < DK; ++i) {
                    S[i] = fmaf(bufQ[t * DK + i], S[i], bufK[t * DK + i] * vt);
                    acc = fmaf(Elem<Tin>::ld(q, x + i), S[i], acc);
                }
                if (active) Elem<Tin>::st(o, vbase + (size_t)(c0 + t) * dv + j, acc);
            }
        }
        __syncthreads();
    }
    if (S_T && active) {
#pragma unroll
        for (int i = 0; i < DK; ++i) S_T[(size_t)bh * DK * dv + (size_t)i * dv + j] = S[i];
    }
}

template <typename Tin, int DK>
static void launch_dk(const ScanArgs &a, hipStream_t st) {
    dim3 grid(a.B * a.H, (a.dv + kGenCols - 1) / kGenCols);
    hipLaunchKernelGGL((scan_generic_kernel<Tin, DK>), grid, dim3(64), 0, st,
                       (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v, (const Tin *)a.g,
                       (const Tin *)a.tau, a.S0, (Tin *)a.o, a.S_T, a.T, a.dv, a.chunk, a.cu, a.H,
                       a.total);
}

template <typename Tin>
static void launch_typed(const ScanArgs &a, hipStream_t st) {
    switch (a.dk) {
        case 16: return launch_dk<Tin, 16>(a, st);
        case 32: return launch_dk<Tin, 32>(a, st);
        case 48: return launch_dk<Tin, 48>(a, st);
        case 64: return launch_dk<Tin, 64>(a, st);
        case 80: return launch_dk<Tin, 80>(a, st);
        case 96: return launch_dk<Tin, 96>(a, st);
        case 112: return launch_dk<Tin, 112>(a, st);
        default: return launch_dk<Tin, 128>(a, st);
    }
}

uint64_t scan_generic_launch_items(long long BH) { return (uint64_t)BH * 64; }

void launch_scan_generic(const ScanArgs &a, hipStream_t st) {
    if (a.dtype == 0) launch_typed<float>(a, st);
    else launch_typed<bf16_t>(a, st);
}

}  // namespace rodimus
