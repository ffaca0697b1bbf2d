// scan_mfma.hip -- chunkwise-parallel prefill on gfx950 matrix cores
// (bf16 inputs, dk = dv = 128, chunk C in {32, 64}, fp32 state).
//
// Method: the Rodimus block runs training/prefill in chunkwise-parallel form
// and inference as a recurrence on a fixed-size state (CodeFuse article,
// "ICLR 2025 | Rodimus*: ...", Rodimus block paragraph).  Per chunk of C
// tokens entering with state S (Lam = inclusive in-chunk cumulative sum of
// log2 a, base-2 units; the gate map is in device_common.h):
//
//     Qt = q * 2^{Lam}                      (bf16 MFMA operand)
//     Kh = k * 2^{log2 beta - Lam}          (bf16)
//     Kb = Kh * 2^{Lam[C-1]}                (bf16)
//     o  = Qt S  +  tril(Qt Kh^T) V         (two MFMA contractions, fp32 acc)
//     S' = diag(2^{Lam[C-1]}) S + Kb^T V    (MFMA, fp32 acc, state in registers)
//
// A chunk whose decay span max_i(-Lam[C-1, i]) exceeds kSpan2 (where 2^{-Lam}
// would leave the fp32/bf16 range) is instead processed token by token on the
// VALU, which gives the same result.
//
// Work decomposition.  One workgroup of 4 waves runs one (b, h) pair over one
// segment of the sequence.  Each wave owns 32 of the 128 state columns: the
// fp32 state tile 128x32 stays in MFMA accumulator registers for the whole
// segment and never goes through memory between chunks.  Per chunk:
//   producer (all 256 lanes, VALU): gates, in-chunk scan of log2 a (DPP scan
//     inside 16-lane rows), the operands Qt, Kh, Kb^T, V^T written to LDS;
//   consumer (MFMA): wave w < C/32 + 1 builds one 32x32 tile of the masked
//     score matrix; then every wave computes its o columns and its state slice.
// The next chunk's raw inputs are loaded into registers while the current
// chunk's contractions run.
//
// Long sequences with few (b, h) pairs are split into G segments so that the
// grid fills the GPU (segment-parallel form of the same recurrence):
//   phase 1 (STATE_ONLY): each segment but the last computes its local end
//            state from zero and its total log2 decay;
//   phase 2 (combine):   S_in[j+1] = diag(2^{A_j}) S_in[j] + S_loc[j], left to right;
//   phase 3 (FULL):      each segment reruns from its S_in and writes o.
//
// MFMA: v_mfma_f32_32x32x16_bf16.  Operand A[m][k] sits in lane m + 32*(k/8),
// element k%8; B[k][n] in lane n + 32*(k/8), element k%8; the accumulator
// C[m][n] in lane n + 32*((m/4)%2), register 4*(m/8) + m%4.  The state kept in
// accumulator layout feeds the o = Qt S contraction directly as operand B with
// a permuted k order (rows 4h..4h+3 and 8+4h..8+4h+3 of each 16-row step); Qt
// is read from LDS with the same permutation.
#include "device_common.h"
#include "launch.h"

namespace rodimus {

namespace {

constexpr int kD = 128;        // dk = dv
constexpr int kThreads = 256;  // 4 waves
constexpr float kSpan2 = 112.f;
constexpr int kTargetBlocks = 256;  // one workgroup on each of the 256 CUs

// LDS layout (bytes).  Rows are padded by 16 bytes so that the 32 rows read by
// one MFMA operand load fall in distinct banks.
constexpr int kQRow = kD + 8;       // bf16 elements per row of sQ / sK  [C][128]
constexpr int kTRow = 64 + 8;       // bf16 elements per row of sKbT / sVT [128][C]
constexpr int kARow = 64 + 8;       // bf16 elements per row of sA [C][C]
constexpr int kOffQ = 0;
constexpr int kOffK = kOffQ + 64 * kQRow * 2;
constexpr int kOffKbT = kOffK + 64 * kQRow * 2;
constexpr int kOffVT = kOffKbT + kD * kTRow * 2;
constexpr int kOffA = kOffVT + kD * kTRow * 2;
constexpr int kOffGam = kOffA + 64 * kARow * 2;
constexpr int kOffFlag = kOffGam + kD * 4;
constexpr int kSmemBytes = kOffFlag + 16;
static_assert(kSmemBytes <= 81920, "two workgroups per CU must fit in 160 KiB of LDS");

struct Params {
    const bf16_t *q, *k, *v, *g, *th;
    const float *S0;  // [BH][128][128] or null (zeros)
    bf16_t *o;
    float *S_T;       // [BH][128][128] or null
    float *wsS;       // [G-1][BH][128][128]: local end states, then incoming states
    float *wsA;       // [G-1][BH][128]: total log2 decay of each segment
    int BH, T, G, seg_len;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    f32x2_t f = {a, b};
    bf16x2_t h = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float lo_bf(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4 &x, float *f) {
    f[0] = lo_bf(x.x); f[1] = hi_bf(x.x);
    f[2] = lo_bf(x.y); f[3] = hi_bf(x.y);
    f[4] = lo_bf(x.z); f[5] = hi_bf(x.z);
    f[6] = lo_bf(x.w); f[7] = hi_bf(x.w);
}

// Shift right by k lanes inside each 16-lane row; lanes with no source get 0.
template <int K>
__device__ __forceinline__ float row_shr(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x110 + K, 0xf, 0xf, false));
}

__device__ __forceinline__ float bcast_lane(float x, int src_lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src_lane << 2, __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ f32x16_t mfma(const bf16x8_t &a, const bf16x8_t &b, const f32x16_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t lds_b128(const char *smem, int byte_off) {
    return *reinterpret_cast<const bf16x8_t *>(smem + byte_off);
}

__device__ __forceinline__ bf16x8_t lds_2x_b64(const char *smem, int off0, int off1) {
    bf16x4_t a = *reinterpret_cast<const bf16x4_t *>(smem + off0);
    bf16x4_t b = *reinterpret_cast<const bf16x4_t *>(smem + off1);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8_t cvt8(const f32x16_t &s, int base) {
    uint4 u;
    u.x = pack2(s[base + 0], s[base + 1]);
    u.y = pack2(s[base + 2], s[base + 3]);
    u.z = pack2(s[base + 4], s[base + 5]);
    u.w = pack2(s[base + 6], s[base + 7]);
    return __builtin_bit_cast(bf16x8_t, u);
}

// One chunk of raw inputs held in registers by a producer lane: TPR tokens x 8
// channels of each tensor (16-byte vectors).
template <int TPR, bool FULL>
struct Raw {
    uint4 q[FULL ? TPR : 1], k[TPR], g[TPR], th[TPR], v[TPR];
};

template <int C, bool FULL>
__device__ __forceinline__ void load_raw(Raw<C / 16, FULL> &R, const Params &p, size_t rowbase,
                                         int t0, int tend, int r, int cg) {
    constexpr int TPR = C / 16;
#pragma unroll
    for (int tt = 0; tt < TPR; ++tt) {
        const int t = t0 + TPR * r + tt;
        const uint4 z = make_uint4(0, 0, 0, 0);
        if (t < tend) {
            const size_t e = (rowbase + t) * kD + 8 * cg;
            if (FULL) R.q[tt] = *reinterpret_cast<const uint4 *>(p.q + e);
            R.k[tt] = *reinterpret_cast<const uint4 *>(p.k + e);
            R.g[tt] = *reinterpret_cast<const uint4 *>(p.g + e);
            R.th[tt] = *reinterpret_cast<const uint4 *>(p.th + e);
            R.v[tt] = *reinterpret_cast<const uint4 *>(p.v + e);
        } else {
            if (FULL) R.q[tt] = z;
            R.k[tt] = z; R.g[tt] = z; R.th[tt] = z; R.v[tt] = z;
        }
    }
}

// Token-by-token processing of one chunk (decay span too large for the
// factorised form).  Uses the operand area of LDS as fp32 scratch.
template <int C, bool FULL>
__device__ void chunk_fallback(char *smem, const Params &p, size_t rowbase, int t0, int tend,
                               f32x16_t (&S)[4], int bh) {
    float *fa = reinterpret_cast<float *>(smem);   // [16][128] a
    float *fb = fa + 16 * kD;                      // [16][128] beta*k
    float *fq = fb + 16 * kD;                      // [16][128] q
    float *fv = fq + 16 * kD;                      // [16][128] v
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, n = 32 * w + (l & 31);
    for (int sb = 0; sb < C; sb += 16) {
        __syncthreads();
        for (int e = tid; e < 16 * kD; e += kThreads) {
            const int tt = e / kD, i = e % kD, t = t0 + sb + tt;
            float a = 1.f, bk = 0.f, qq = 0.f, vv = 0.f;
            if (t < tend) {
                const size_t x = (rowbase + t) * kD + i;
                float l2a, l2b;
                ddts_log2_gates(bf2f(p.g[x]), bf2f(p.th[x]), l2a, l2b);
                a = exp2_fast(l2a);
                bk = exp2_fast(l2b) * bf2f(p.k[x]);
                if (FULL) qq = bf2f(p.q[x]);
                vv = bf2f(p.v[x]);
            }
            fa[e] = a; fb[e] = bk; fq[e] = qq; fv[e] = vv;
        }
        __syncthreads();
        for (int tt = 0; tt < 16; ++tt) {
            const int t = t0 + sb + tt;
            if (t >= tend) break;
            const float vn = fv[tt * kD + n];
            float part = 0.f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int i0 = 32 * mt + 8 * a4 + 4 * h;
                    const float4 av = *reinterpret_cast<const float4 *>(fa + tt * kD + i0);
                    const float4 bv = *reinterpret_cast<const float4 *>(fb + tt * kD + i0);
                    const float4 qv = *reinterpret_cast<const float4 *>(fq + tt * kD + i0);
                    float x;
                    x = fmaf(av.x, S[mt][4 * a4 + 0], bv.x * vn); S[mt][4 * a4 + 0] = x; part = fmaf(qv.x, x, part);
                    x = fmaf(av.y, S[mt][4 * a4 + 1], bv.y * vn); S[mt][4 * a4 + 1] = x; part = fmaf(qv.y, x, part);
                    x = fmaf(av.z, S[mt][4 * a4 + 2], bv.z * vn); S[mt][4 * a4 + 2] = x; part = fmaf(qv.z, x, part);
                    x = fmaf(av.w, S[mt][4 * a4 + 3], bv.w * vn); S[mt][4 * a4 + 3] = x; part = fmaf(qv.w, x, part);
                }
            }
            if (FULL) {
                part += __shfl_xor(part, 32);
                if (h == 0) p.o[((size_t)bh * p.T + t) * kD + n] = f2bf(part);
            }
        }
    }
}

template <int C, bool FULL>
__global__ __launch_bounds__(kThreads, 1)
void scan_mfma_kernel(Params p) {
    constexpr int TPR = C / 16;   // tokens per producer lane
    constexpr int NT = C / 32;    // 32-token tiles per chunk
    __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
    int *sFlag = reinterpret_cast<int *>(smem + kOffFlag);
    float *sGam = reinterpret_cast<float *>(smem + kOffGam);

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, l32 = l & 31;
    // producer coordinates: token group r (TPR consecutive tokens), channel group cg (8 channels)
    const int r = l & 15, cg = (w << 2) | (l >> 4);

    const int nseg = FULL ? p.G : p.G - 1;
    const int bh = blockIdx.x % p.BH, seg = blockIdx.x / p.BH;
    if (seg >= nseg) return;
    const int t_begin = seg * p.seg_len;
    const int t_end = min(p.T, t_begin + p.seg_len);
    const size_t rowbase = (size_t)bh * p.T;
    const size_t sstride = (size_t)kD * kD;

    // ---- initial state (accumulator layout): rows 32mt + 8a + 4h + r4, column 32w + l32
    f32x16_t S[4];
    const float *Sin = nullptr;
    if (FULL) Sin = (seg == 0) ? (p.S0 ? p.S0 + bh * sstride : nullptr)
                               : p.wsS + ((size_t)(seg - 1) * p.BH + bh) * sstride;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
            S[mt][i] = Sin ? Sin[row * kD + 32 * w + l32] : 0.f;
        }

    float logdecay[8];  // running sum of this lane's 8 channels' Lam_end (STATE_ONLY)
#pragma unroll
    for (int e = 0; e < 8; ++e) logdecay[e] = 0.f;

    if (tid < 2) sFlag[tid] = 0;
    __syncthreads();

    Raw<TPR, FULL> R;
    load_raw<C, FULL>(R, p, rowbase, t_begin, t_end, r, cg);

    int parity = 0;
    for (int t0 = t_begin; t0 < t_end; t0 += C, parity ^= 1) {
        // ================= producer: gates, scan, operands -> LDS =================
        {
            float l2a[TPR][8], l2b[TPR][8];
#pragma unroll
            for (int tt = 0; tt < TPR; ++tt) {
                float gf[8], tf[8];
                unpack8(R.g[tt], gf);
                unpack8(R.th[tt], tf);
                const bool valid = (t0 + TPR * r + tt) < t_end;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ddts_log2_gates_fast(gf[e], tf[e], l2a[tt][e], l2b[tt][e]);
                    if (!valid) { l2a[tt][e] = 0.f; l2b[tt][e] = -INFINITY; }
                }
            }
            // in-lane inclusive scan over the TPR tokens
#pragma unroll
            for (int tt = 1; tt < TPR; ++tt)
#pragma unroll
                for (int e = 0; e < 8; ++e) l2a[tt][e] += l2a[tt - 1][e];
            // scan of the per-lane totals across the 16 lanes of the row
            float excl[8], lend[8];
            bool bad = false;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = l2a[TPR - 1][e];
                x += row_shr<1>(x);
                x += row_shr<2>(x);
                x += row_shr<4>(x);
                x += row_shr<8>(x);
                excl[e] = row_shr<1>(x);
                lend[e] = bcast_lane(x, (l & 48) | 15);
                bad |= lend[e] < -kSpan2;
                logdecay[e] += lend[e];
            }
            float gam[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) gam[e] = exp2_fast(lend[e]);
            if (r == 0) {
                *reinterpret_cast<float4 *>(sGam + 8 * cg) = make_float4(gam[0], gam[1], gam[2], gam[3]);
                *reinterpret_cast<float4 *>(sGam + 8 * cg + 4) = make_float4(gam[4], gam[5], gam[6], gam[7]);
            }
            if (bad) sFlag[parity] = 1;

            float kb[TPR][8], vf[TPR][8];
#pragma unroll
            for (int tt = 0; tt < TPR; ++tt) {
                const int t = TPR * r + tt;  // token index inside the chunk
                float kf[8];
                unpack8(R.k[tt], kf);
                unpack8(R.v[tt], vf[tt]);
                float kh[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float lam = l2a[tt][e] + excl[e];
                    kh[e] = kf[e] * exp2_fast(l2b[tt][e] - lam);
                    kb[tt][e] = kh[e] * gam[e];
                    l2a[tt][e] = lam;
                }
                if (FULL) {
                    float qf[8], qt[8];
                    unpack8(R.q[tt], qf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) qt[e] = qf[e] * exp2_fast(l2a[tt][e]);
                    uint4 uq = make_uint4(pack2(qt[0], qt[1]), pack2(qt[2], qt[3]),
                                          pack2(qt[4], qt[5]), pack2(qt[6], qt[7]));
                    uint4 uk = make_uint4(pack2(kh[0], kh[1]), pack2(kh[2], kh[3]),
                                          pack2(kh[4], kh[5]), pack2(kh[6], kh[7]));
                    *reinterpret_cast<uint4 *>(smem + kOffQ + (t * kQRow + 8 * cg) * 2) = uq;
                    *reinterpret_cast<uint4 *>(smem + kOffK + (t * kQRow + 8 * cg) * 2) = uk;
                }
            }
            // transposed Kb and V: row = channel, TPR consecutive tokens per write
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = 8 * cg + e;
                if (TPR == 4) {
                    uint2 ukb = make_uint2(pack2(kb[0][e], kb[1 % TPR][e]), pack2(kb[2 % TPR][e], kb[3 % TPR][e]));
                    uint2 uvv = make_uint2(pack2(vf[0][e], vf[1 % TPR][e]), pack2(vf[2 % TPR][e], vf[3 % TPR][e]));
                    *reinterpret_cast<uint2 *>(smem + kOffKbT + (c * kTRow + TPR * r) * 2) = ukb;
                    *reinterpret_cast<uint2 *>(smem + kOffVT + (c * kTRow + TPR * r) * 2) = uvv;
                } else {
                    *reinterpret_cast<uint32_t *>(smem + kOffKbT + (c * kTRow + TPR * r) * 2) = pack2(kb[0][e], kb[1 % TPR][e]);
                    *reinterpret_cast<uint32_t *>(smem + kOffVT + (c * kTRow + TPR * r) * 2) = pack2(vf[0][e], vf[1 % TPR][e]);
                }
            }
        }
        __syncthreads();  // operands of this chunk are in LDS

        // prefetch the next chunk's raw inputs while the contractions run
        if (t0 + C < t_end) load_raw<C, FULL>(R, p, rowbase, t0 + C, t_end, r, cg);
        if (tid == 0) sFlag[parity ^ 1] = 0;

        if (sFlag[parity]) {
            chunk_fallback<C, FULL>(smem, p, rowbase, t0, t_end, S, bh);
            __syncthreads();
            continue;
        }

        // ================= consumer: MFMA contractions =================
        // V^T operand fragments (B operand, k = token): reused by o and by the state update
        bf16x8_t vB[C / 16];
#pragma unroll
        for (int s = 0; s < C / 16; ++s)
            vB[s] = lds_b128(smem, kOffVT + ((32 * w + l32) * kTRow + 16 * s + 8 * h) * 2);

        if (FULL) {
            // (1) masked score tiles A^T[j][i] = Kh[j] . Qt[i], j <= i; wave w builds tile w
            //     (Jt, It) in {(0,0), (0,1), (1,1)} for C = 64, {(0,0)} for C = 32.
            if (w < (NT == 2 ? 3 : 1)) {
                const int Jt = (w == 2) ? 1 : 0;
                const int It = (w == 0) ? 0 : 1;
                f32x16_t acc = {};
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    bf16x8_t a = lds_b128(smem, kOffK + ((32 * Jt + l32) * kQRow + 16 * s + 8 * h) * 2);
                    bf16x8_t b = lds_b128(smem, kOffQ + ((32 * It + l32) * kQRow + 16 * s + 8 * h) * 2);
                    acc = mfma(a, b, acc);
                }
                const int i = 32 * It + l32;
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    float x[4];
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int j = 32 * Jt + 8 * a4 + 4 * h + r4;
                        x[r4] = (j <= i) ? acc[4 * a4 + r4] : 0.f;
                    }
                    *reinterpret_cast<uint2 *>(smem + kOffA + (i * kARow + 32 * Jt + 8 * a4 + 4 * h) * 2) =
                        make_uint2(pack2(x[0], x[1]), pack2(x[2], x[3]));
                }
            }
            // bf16 copy of the state for o = Qt S (operand B, permuted k order)
            bf16x8_t Sb[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) Sb[s] = cvt8(S[s >> 1], 8 * (s & 1));
            __syncthreads();  // score tiles ready

            // (2) o tiles for this wave's 32 columns
#pragma unroll
            for (int It = 0; It < NT; ++It) {
                f32x16_t acc = {};
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const int rowoff = (32 * It + l32) * kQRow + 16 * s + 4 * h;
                    bf16x8_t a = lds_2x_b64(smem, kOffQ + rowoff * 2, kOffQ + (rowoff + 8) * 2);
                    acc = mfma(a, Sb[s], acc);
                }
#pragma unroll
                for (int s = 0; s < 2 * It + 2; ++s) {
                    bf16x8_t a = lds_b128(smem, kOffA + ((32 * It + l32) * kARow + 16 * s + 8 * h) * 2);
                    acc = mfma(a, vB[s], acc);
                }
                const int n = 32 * w + l32;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int t = t0 + 32 * It + 8 * (i >> 2) + 4 * h + (i & 3);
                    if (t < t_end) p.o[(rowbase + t) * kD + n] = f2bf(acc[i]);
                }
            }
        }

        // (3) state: S <- diag(gamma) S + Kb^T V  (this wave's 32 columns)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const float4 gm = *reinterpret_cast<const float4 *>(sGam + 32 * mt + 8 * a4 + 4 * h);
                S[mt][4 * a4 + 0] *= gm.x;
                S[mt][4 * a4 + 1] *= gm.y;
                S[mt][4 * a4 + 2] *= gm.z;
                S[mt][4 * a4 + 3] *= gm.w;
            }
#pragma unroll
            for (int s = 0; s < C / 16; ++s) {
                bf16x8_t a = lds_b128(smem, kOffKbT + ((32 * mt + l32) * kTRow + 16 * s + 8 * h) * 2);
                S[mt] = mfma(a, vB[s], S[mt]);
            }
        }
        __syncthreads();  // LDS operands free for the next chunk
    }

    // ---- outputs of the segment
    float *Sout = nullptr;
    if (FULL) {
        if (seg == p.G - 1) Sout = p.S_T ? p.S_T + bh * sstride : nullptr;
    } else {
        Sout = p.wsS + ((size_t)seg * p.BH + bh) * sstride;
        if (r == 0) {
            float *A = p.wsA + ((size_t)seg * p.BH + bh) * kD + 8 * cg;
#pragma unroll
            for (int e = 0; e < 8; ++e) A[e] = logdecay[e];
        }
    }
    if (Sout) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
                Sout[row * kD + 32 * w + l32] = S[mt][i];
            }
    }
}

// Phase 2: S_in of segment j+1 = diag(2^{A_j}) S_in of segment j + S_loc[j], in place
// over the local states.  One thread per (b,h, state element).
__global__ __launch_bounds__(256)
void scan_combine_kernel(const float *__restrict__ S0, float *wsS, const float *__restrict__ wsA,
                         int BH, int nseg) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t per = (size_t)kD * kD;
    if (idx >= (size_t)BH * per) return;
    const size_t bh = idx / per, e = idx % per;
    const int i = (int)(e / kD);
    float s = S0 ? S0[idx] : 0.f;
    for (int j = 0; j < nseg; ++j) {
        const size_t base = (size_t)j * BH * per;
        s = exp2_fast(wsA[((size_t)j * BH + bh) * kD + i]) * s + wsS[base + idx];
        wsS[base + idx] = s;
    }
}

}  // namespace

ScanPlan plan_scan(int B, int H, int T, int dk, int dv, int chunk, int dtype) {
    ScanPlan pl{false, 1, 0};
    if (!(dtype == 1 && dk == kD && dv == kD && (chunk == 32 || chunk == 64))) return pl;
    pl.mfma = true;
    const long long BH = (long long)B * H;
    const long long nchunks = (T + chunk - 1) / chunk;
    if (nchunks == 0 || BH == 0) return pl;  // nothing to scan: one segment, no workspace
    long long G = (kTargetBlocks + BH - 1) / BH;
    if (G > nchunks) G = nchunks;
    if (G < 1) G = 1;
    const long long per_seg = (nchunks + G - 1) / G;  // chunks per segment
    G = (nchunks + per_seg - 1) / per_seg;
    pl.segments = (int)G;
    pl.workspace_bytes = (size_t)(G - 1) * BH * (kD * kD + kD) * sizeof(float);
    return pl;
}

void launch_scan_mfma(const ScanArgs &a, const ScanPlan &pl, hipStream_t st) {
    const int BH = a.B * a.H;
    const int G = pl.segments;
    const int nchunks = (a.T + a.chunk - 1) / a.chunk;
    const int per_seg = (nchunks + G - 1) / G;
    Params p;
    p.q = (const bf16_t *)a.q; p.k = (const bf16_t *)a.k; p.v = (const bf16_t *)a.v;
    p.g = (const bf16_t *)a.g; p.th = (const bf16_t *)a.tau;
    p.S0 = a.S0; p.o = (bf16_t *)a.o; p.S_T = a.S_T;
    p.wsS = (float *)a.workspace;
    p.wsA = p.wsS ? p.wsS + (size_t)(G > 1 ? G - 1 : 0) * BH * kD * kD : nullptr;
    p.BH = BH; p.T = a.T; p.G = G; p.seg_len = per_seg * a.chunk;
    if (G > 1) {
        if (a.chunk == 64) hipLaunchKernelGGL((scan_mfma_kernel<64, false>), dim3((G - 1) * BH), dim3(kThreads), 0, st, p);
        else hipLaunchKernelGGL((scan_mfma_kernel<32, false>), dim3((G - 1) * BH), dim3(kThreads), 0, st, p);
        const size_t n = (size_t)BH * kD * kD;
        hipLaunchKernelGGL(scan_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           a.S0, p.wsS, p.wsA, BH, G - 1);
    }
    if (a.chunk == 64) hipLaunchKernelGGL((scan_mfma_kernel<64, true>), dim3(G * BH), dim3(kThreads), 0, st, p);
    else hipLaunchKernelGGL((scan_mfma_kernel<32, true>), dim3(G * BH), dim3(kThreads), 0, st, p);
}

}  // namespace rodimus
