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
//     o  = Qt S  +  tril(Qt Kh^T) V         (MFMA, fp32 accumulation)
//     S' = diag(2^{Lam[C-1]}) S + Kb^T V    (MFMA, fp32 accumulation)
//
// Kh needs 2^{-Lam} to stay inside the fp32/bf16 range: a chunk whose decay
// span max_i(-Lam[C-1, i]) exceeds kSpan2 is processed token by token on the
// VALU instead (same result).  Kb never overflows (its exponent is <= 0).
//
// Segment-parallel form.  So that the grid fills the GPU when B*H is small, the
// sequence of each (b, h) is cut into G segments (each a whole number of
// chunks), and every segment but the last into P sub-segments:
//   phase 1 (scan_state_kernel): each sub-segment's local end state (from zero)
//            and its total log2 decay, in 32-token chunks with two chunks of
//            inputs in flight.  Chunks are visited last to first, so the
//            decay of the later chunks folds into the operand exponent:
//            S_loc = sum_c (Kb_c * 2^{rho_c})^T V_c, rho_c = sum of Lam_end after c;
//            there is no state rescaling and nothing can overflow;
//   phase 2 (scan_combine_kernel): S_in of every segment, left to right;
//   phase 3 (scan_full_kernel): every segment from its S_in, writing o.
//
// scan_full_kernel: 8 waves.  Waves 0-3 (producers) turn chunk k's raw inputs
// into LDS operands (gates, DPP scan of log2 a inside 16-lane rows, Qt, Kh,
// Kb^T, V^T) while waves 4-7 (consumers) contract chunk k-1 on the matrix cores
// from the other LDS buffer; one barrier per chunk.  Each consumer wave owns 32
// of the 128 state columns: its fp32 128x32 state slice lives in MFMA
// accumulator registers for the whole segment, and the consumer waves issue at
// a higher priority than the producers.  The masked score tiles A^T = Kh Qt^T
// are built once per chunk (the three 32x32 tiles on or below the diagonal for
// C = 64, one for C = 32, each by one consumer wave) and exchanged through LDS
// behind a barrier of the four consumer waves only.  o is produced transposed
// (o^T = S^T Qt^T + V^T A^T) so that each lane stores 8-byte runs.
//
// MFMA: v_mfma_f32_32x32x16_bf16.  Operand A[m][k] sits in lane m + 32*(k/8),
// element k%8; B[k][n] in lane n + 32*(k/8), element k%8; the accumulator
// C[m][n] in lane n + 32*((m/4)%2), register 4*(m/8) + m%4.  An accumulator
// therefore holds, per lane half h, the rows {4h..4h+3, 8+4h..8+4h+3} of every
// 16-row step; used as an operand it contracts k in that order.  LDS stores
// the channels of Qt/Kh and the tokens of Kb^T/V^T in the matching order
// (blocks of 4 permuted as 0,2,1,3 inside each 16), so every operand read is
// one 16-byte ds_read.
#include "launch.h"
#include "mfma_common.h"

namespace rodimus {

namespace {

constexpr int kCUs = 256;
constexpr int kMaxT = 1 << 23;     // 32-bit buffer offsets (T * 256 bytes)

// LDS buffer layout (bytes); rows padded by 16 bytes (conflict-free 16-byte reads)
constexpr int kQRow = kD + 8;      // bf16 per row of sQ / sK       [C][128]
constexpr int kTRow = 64 + 8;      // bf16 per row of sKbT / sVT    [128][C]
constexpr int kOffQ = 0;
constexpr int kOffK = kOffQ + 64 * kQRow * 2;
constexpr int kOffKbT = kOffK + 64 * kQRow * 2;
constexpr int kOffVT = kOffKbT + kD * kTRow * 2;
constexpr int kOffGam = kOffVT + kD * kTRow * 2;
constexpr int kBufBytes = kOffGam + kD * 4;
constexpr int kARow = 64 + 8;      // bf16 per row of sA [C][C] (token i, token j permuted)
constexpr int kSABytes = 64 * kARow * 2;

struct Params {
    const bf16_t *q, *k, *v, *g, *th;
    const float *S0;  // [BH][128][128] or null (zeros)
    bf16_t *o;
    float *S_T;       // [BH][128][128] or null
    float *wsS;       // [(G-1)*P][BH][128][128] sub-segment states / incoming states
    float *wsA;       // [(G-1)*P][BH][128] total log2 decay of each sub-segment
    int BH, T, G, seg_len, P, sub_len;
    // packed variable-length batch: sequence s = bh / H occupies rows
    // cu[s] .. cu[s+1]-1 of head h = bh % H's [total][128] rows; T is then the
    // longest length (the segment plan)
    const int *cu;
    int H, total;
    const int *order;  // packed batch: longest-first order of the sequences, or null
};

// Rows of (b,h): first row and length.  The packed form clamps each span to
// [0, total] and to T, so a malformed offset table cannot address memory
// outside the inputs and outputs.
template <bool VL>
__device__ __forceinline__ void seq_span(const Params &p, int bh, size_t &rowbase, int &len) {
    if (!VL) {
        rowbase = (size_t)bh * p.T;
        len = p.T;
        return;
    }
    const int s = bh / p.H, h = bh - s * p.H;
    const int a = min(max(uni(p.cu[s]), 0), p.total);
    const int b = min(max(uni(p.cu[s + 1]), a), p.total);
    rowbase = (size_t)h * p.total + a;
    len = min(b - a, p.T);
}

// ------------------------------------------------------------- phase 3 (full)
template <int C, bool VL>
__global__ __launch_bounds__(512, 1)
void scan_full_kernel(Params p) {
    constexpr int TPR = C / 16, NT = C / 32;
    __shared__ __attribute__((aligned(16))) char smem[2 * kBufBytes + kSABytes + 16];
    char *sA = smem + 2 * kBufBytes;                                        // score tiles of one chunk
    int *sFlag = reinterpret_cast<int *>(smem + 2 * kBufBytes + kSABytes);  // chunk k -> slot k % 3
    int *sCBar = sFlag + 3;                                                 // consumer-wave barrier

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, l32 = l & 31;
    const int seg = uni(blockIdx.x / p.BH);
    if (seg >= p.G) return;
    const int bh = VL ? seq_head(p.order, p.H, uni(blockIdx.x % p.BH)) : uni(blockIdx.x % p.BH);
    size_t rowbase;
    int Tb;
    seq_span<VL>(p, bh, rowbase, Tb);
    const int t_begin = seg * p.seg_len;
    const int t_end = min(Tb, t_begin + p.seg_len);
    const int nch = max(0, (t_end - t_begin + C - 1) / C);

    if (tid < 4) sFlag[tid] = 0;
    __syncthreads();

    if (w < 4) {
        // ======================= producers =======================
        const int r = l & 15, cg = (w << 2) | (l >> 4);
        Rsrc rs;
        rs.q = rsrc(p.q + rowbase * kD, Tb); rs.k = rsrc(p.k + rowbase * kD, Tb);
        rs.v = rsrc(p.v + rowbase * kD, Tb); rs.g = rsrc(p.g + rowbase * kD, Tb);
        rs.th = rsrc(p.th + rowbase * kD, Tb);
        Raw<C, true> R;
        load_raw<C, true>(R, rs, t_begin, r, cg);
        for (int kk = 0; kk <= nch; ++kk) {
            if (kk < nch) {
                const int t0 = t_begin + kk * C;
                char *buf = smem + (kk & 1) * kBufBytes;
                const bool more = kk + 1 < nch;
                store_vt<TPR, kTRow>(buf + kOffVT, cg, r, R.v);
                if (more) load_one<TPR>(R.v, rs.v, t0 + C, r, cg);
                float l2a[TPR][8], l2b[TPR][8], lend[8];
                gates_scan<C, true>(R, t0, t_end, r, l, l2a, l2b, lend);
                if (more) {
                    load_one<TPR>(R.g, rs.g, t0 + C, r, cg);
                    load_one<TPR>(R.th, rs.th, t0 + C, r, cg);
                }
                bool bad = false;
                float gam[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    bad |= lend[e] < -kSpan2;
                    gam[e] = exp2_fast(lend[e]);
                }
                if (r == 0) {
                    float *sg = reinterpret_cast<float *>(buf + kOffGam) + 8 * cg;
                    *reinterpret_cast<float4 *>(sg) = make_float4(gam[0], gam[1], gam[2], gam[3]);
                    *reinterpret_cast<float4 *>(sg + 4) = make_float4(gam[4], gam[5], gam[6], gam[7]);
                }
                if (bad) sFlag[kk % 3] = 1;
                if (tid == 0) sFlag[(kk + 1) % 3] = 0;
                float kbT[8][TPR];
#pragma unroll
                for (int tt = 0; tt < TPR; ++tt) {
                    float qf[8], kf[8], qt[8], kh[8];
                    unpack8(R.q[tt], qf);
                    unpack8(R.k[tt], kf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        qt[e] = qf[e] * exp2_fast(l2a[tt][e]);
                        kh[e] = kf[e] * exp2_fast(l2b[tt][e] - l2a[tt][e]);
                        kbT[e][tt] = kh[e] * gam[e];
                    }
                    const int t = TPR * r + tt;
                    store_q_row<kQRow>(buf + kOffQ, t, cg, qt);
                    store_q_row<kQRow>(buf + kOffK, t, cg, kh);
                }
                if (more) {
                    load_one<TPR>(R.q, rs.q, t0 + C, r, cg);
                    load_one<TPR>(R.k, rs.k, t0 + C, r, cg);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) store_t_rows<TPR, kTRow>(buf + kOffKbT, 8 * cg + e, r, kbT[e]);
            }
            __syncthreads();
        }
        return;
    }

    // ======================= consumers =======================
    // The consumer waves' MFMA chain is the shorter critical path of an interval:
    // issue it first and let the producer waves fill the VALU around it.
    __builtin_amdgcn_s_setprio(3);
    const int cw = w - 4;                 // state columns 32cw .. 32cw+31
    int cbar_target = 0;
    const int n = 32 * cw + l32;
    f32x16_t S[4];                        // rows 32mt + 8a + 4h + r4, column n
    {
        const float *Sin = (seg == 0) ? (p.S0 ? p.S0 + (size_t)bh * kD * kD : nullptr)
                                      : p.wsS + ((size_t)(seg * p.P - 1) * p.BH + bh) * kD * kD;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                S[mt][i] = Sin ? Sin[(32 * mt + 8 * (i >> 2) + 4 * h + (i & 3)) * kD + n] : 0.f;
    }
    for (int kk = 0; kk <= nch; ++kk) {
        if (kk >= 1) {
            const int c = kk - 1;
            const int t0 = t_begin + c * C;
            char *buf = smem + (c & 1) * kBufBytes;
            if (sFlag[c % 3]) {
                // Token-by-token fallback.  Each consumer wave works alone in a
                // private 6 KiB slice of this chunk's (no longer needed) buffer.
                float *fa = reinterpret_cast<float *>(buf) + cw * 1536;  // [4][128] a
                float *fb = fa + 512;                                    // [4][128] beta*k
                float *fq = fb + 512;                                    // [4][128] q
                for (int sb = 0; sb < C; sb += 4) {
                    for (int e = l; e < 512; e += 64) {
                        const int tt = e >> 7, i = e & 127, t = t0 + sb + tt;
                        float a = 1.f, bk = 0.f, qq = 0.f;
                        if (t < t_end) {
                            const size_t x = (rowbase + t) * kD + i;
                            float l2a, l2b;
                            ddts_log2_gates(bf2f(p.g[x]), bf2f(p.th[x]), l2a, l2b);
                            a = exp2_fast(l2a);
                            bk = exp2_fast(l2b) * bf2f(p.k[x]);
                            qq = bf2f(p.q[x]);
                        }
                        fa[e] = a; fb[e] = bk; fq[e] = qq;
                    }
                    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    for (int tt = 0; tt < 4; ++tt) {
                        const int t = t0 + sb + tt;
                        if (t >= t_end) break;
                        const float vn = bf2f(p.v[(rowbase + t) * kD + n]);
                        float part = 0.f;
#pragma unroll
                        for (int mt = 0; mt < 4; ++mt) {
                            // one accumulator block at a time, as a whole: the state keeps
                            // its MFMA registers, and this rarely taken branch does not
                            // raise the register count of the kernel
                            f32x16_t av, bv, qv;
#pragma unroll
                            for (int a4 = 0; a4 < 4; ++a4) {
                                const int i0 = tt * 128 + 32 * mt + 8 * a4 + 4 * h;
                                const float4 x = *reinterpret_cast<const float4 *>(fa + i0);
                                const float4 y = *reinterpret_cast<const float4 *>(fb + i0);
                                const float4 z = *reinterpret_cast<const float4 *>(fq + i0);
                                av[4 * a4 + 0] = x.x; av[4 * a4 + 1] = x.y; av[4 * a4 + 2] = x.z; av[4 * a4 + 3] = x.w;
                                bv[4 * a4 + 0] = y.x; bv[4 * a4 + 1] = y.y; bv[4 * a4 + 2] = y.z; bv[4 * a4 + 3] = y.w;
                                qv[4 * a4 + 0] = z.x; qv[4 * a4 + 1] = z.y; qv[4 * a4 + 2] = z.z; qv[4 * a4 + 3] = z.w;
                            }
#pragma unroll
                            for (int i = 0; i < 16; ++i) {
                                const float x = fmaf(av[i], S[mt][i], bv[i] * vn);
                                S[mt][i] = x;
                                part = fmaf(qv[i], x, part);
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        part += __shfl_xor(part, 32);
                        if (h == 0) p.o[(rowbase + t) * kD + n] = f2bf(part);
                    }
                    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                }
            } else {
                // V^T fragments: B operand (k = token, permuted order) of both
                // o += A V and S += Kb^T V
                bf16x8_t vB[C / 16];
#pragma unroll
                for (int s = 0; s < C / 16; ++s)
                    vB[s] = lds16(buf, kOffVT + (n * kTRow + 16 * s + 8 * h) * 2);
                // bf16 state as the B operand of o += Qt S (k = channel, permuted order)
                bf16x8_t Sb[8];
#pragma unroll
                for (int s = 0; s < 8; ++s) Sb[s] = cvt8(S[s >> 1], 8 * (s & 1));
                // masked score tiles A^T[j][i] = Kh[j] . Qt[i] (j <= i); consumer wave ti
                // builds tile (Jt, It) = (0,0), (0,1), (1,1) (only (0,0) for C = 32) and
                // stores it as A[i][j] (j in permuted order) for all four waves
                if (cw < (NT == 2 ? 3 : 1)) {
                    const int Jt = (cw == 2) ? 1 : 0, It = (cw == 0) ? 0 : 1;
                    f32x16_t at = {};
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        const bf16x8_t a = lds16(buf, kOffK + ((32 * Jt + l32) * kQRow + 16 * s + 8 * h) * 2);
                        const bf16x8_t b = lds16(buf, kOffQ + ((32 * It + l32) * kQRow + 16 * s + 8 * h) * 2);
                        at = mfma(a, b, at);
                    }
                    const int i = 32 * It + l32;
#pragma unroll
                    for (int a4 = 0; a4 < 4; ++a4) {
                        float x[4];
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4) {
                            const int j = 32 * Jt + 8 * a4 + 4 * h + r4;
                            x[r4] = (j <= i) ? at[4 * a4 + r4] : 0.f;
                        }
                        *reinterpret_cast<uint2 *>(sA + (i * kARow + perm16(32 * Jt + 8 * a4 + 4 * h)) * 2) =
                            make_uint2(pack2(x[0], x[1]), pack2(x[2], x[3]));
                    }
                }
                // the four consumer waves meet (LDS counter; the producer waves are
                // not involved); bounded wait
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
                if (l == 0) __hip_atomic_fetch_add(sCBar, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                cbar_target += 4;
                for (int spin = 0; spin < (1 << 24); ++spin) {
                    if (__hip_atomic_load(sCBar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= cbar_target) break;
                    __builtin_amdgcn_s_sleep(1);
                }
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
                // o^T tiles: 32 value channels (this wave's) x 32 tokens (32It..).  Same
                // fragments as o = Qt S + A V with the operands swapped, so that a
                // lane holds one token and 4 consecutive channels per register group.
#pragma unroll
                for (int It = 0; It < NT; ++It) {
                    f32x16_t acc = {};
#pragma unroll
                    for (int s = 0; s < 8; ++s)
                        acc = mfma(Sb[s], lds16(buf, kOffQ + ((32 * It + l32) * kQRow + 16 * s + 8 * h) * 2), acc);
#pragma unroll
                    for (int s = 0; s < 2 * It + 2; ++s)
                        acc = mfma(vB[s], lds16(sA, ((32 * It + l32) * kARow + 16 * s + 8 * h) * 2), acc);
                    const int t = t0 + 32 * It + l32;
                    if (t < t_end) {
                        bf16_t *op = p.o + (rowbase + t) * kD + 32 * cw + 4 * h;
#pragma unroll
                        for (int a4 = 0; a4 < 4; ++a4)
                            *reinterpret_cast<uint2 *>(op + 8 * a4) =
                                make_uint2(pack2(acc[4 * a4 + 0], acc[4 * a4 + 1]),
                                           pack2(acc[4 * a4 + 2], acc[4 * a4 + 3]));
                    }
                }
                // state: S <- diag(gamma) S + Kb^T V
                const float *gam = reinterpret_cast<const float *>(buf + kOffGam);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                    for (int a4 = 0; a4 < 4; ++a4) {
                        const float4 gm = *reinterpret_cast<const float4 *>(gam + 32 * mt + 8 * a4 + 4 * h);
                        S[mt][4 * a4 + 0] *= gm.x; S[mt][4 * a4 + 1] *= gm.y;
                        S[mt][4 * a4 + 2] *= gm.z; S[mt][4 * a4 + 3] *= gm.w;
                    }
#pragma unroll
                    for (int s = 0; s < C / 16; ++s)
                        S[mt] = mfma(lds16(buf, kOffKbT + ((32 * mt + l32) * kTRow + 16 * s + 8 * h) * 2), vB[s], S[mt]);
                }
            }
        }
        __syncthreads();
    }
    if (seg == p.G - 1 && p.S_T) {
        float *So = p.S_T + (size_t)bh * kD * kD;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) So[(32 * mt + 8 * (i >> 2) + 4 * h + (i & 3)) * kD + n] = S[mt][i];
    }
}

// ----------------------------------------------------------- phase 1 (state)
// One sub-segment's local end state.  Processed in chunks of 32 tokens whatever
// the caller's C (the result does not depend on the chunking), which leaves
// room in the registers for two chunks of raw inputs in flight.
template <int TPR>
__device__ __forceinline__ void state_chunk(Raw<16 * TPR, false> &R, const Rsrc &rs, int t0, int tnext,
                                            char *sKbT, char *sVT, f32x16_t (&S)[4], float (&rho)[8],
                                            int r, int cg, int l, int w, int h, int l32, int T) {
    store_vt<TPR, kTRow>(sVT, cg, r, R.v);
    if (tnext >= 0) load_one<TPR>(R.v, rs.v, tnext, r, cg);
    float l2a[TPR][8], l2b[TPR][8], lend[8];
    gates_scan<16 * TPR, false>(R, t0, T, r, l, l2a, l2b, lend);
    if (tnext >= 0) {
        load_one<TPR>(R.g, rs.g, tnext, r, cg);
        load_one<TPR>(R.th, rs.th, tnext, r, cg);
    }
    float kbT[8][TPR];
#pragma unroll
    for (int tt = 0; tt < TPR; ++tt) {
        float kf[8];
        unpack8(R.k[tt], kf);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            kbT[e][tt] = kf[e] * exp2_fast(l2b[tt][e] + lend[e] - l2a[tt][e] + rho[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) rho[e] += lend[e];
    if (tnext >= 0) load_one<TPR>(R.k, rs.k, tnext, r, cg);
#pragma unroll
    for (int e = 0; e < 8; ++e) store_t_rows<TPR, kTRow>(sKbT, 8 * cg + e, r, kbT[e]);
    __syncthreads();
    bf16x8_t vB[TPR];
#pragma unroll
    for (int s = 0; s < TPR; ++s) vB[s] = lds16(sVT, ((32 * w + l32) * kTRow + 16 * s + 8 * h) * 2);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int s = 0; s < TPR; ++s)
            S[mt] = mfma(lds16(sKbT, ((32 * mt + l32) * kTRow + 16 * s + 8 * h) * 2), vB[s], S[mt]);
    __syncthreads();
}

template <bool VL>
__global__ __launch_bounds__(256, 2)
void scan_state_kernel(Params p) {
    constexpr int CS = 32, TPR = CS / 16;
    __shared__ __attribute__((aligned(16))) char smem[2 * kD * kTRow * 2];
    char *sKbT = smem, *sVT = smem + kD * kTRow * 2;

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, l32 = l & 31;
    const int nsub = (p.G - 1) * p.P;
    const int sub = uni(blockIdx.x / p.BH);
    if (sub >= nsub) return;
    const int bh = VL ? seq_head(p.order, p.H, uni(blockIdx.x % p.BH)) : uni(blockIdx.x % p.BH);
    const int seg = sub / p.P, part = sub % p.P;
    const int seg_begin = seg * p.seg_len;
    const int t_begin = seg_begin + part * p.sub_len;
    const int t_end = min(seg_begin + p.seg_len, t_begin + p.sub_len);  // whole chunks
    size_t rowbase;
    int Tb;
    seq_span<VL>(p, bh, rowbase, Tb);
    // chunks of this sub-segment that hold tokens (all of them unless packed)
    const int nch = VL ? max(0, min((t_end - t_begin) / CS, (Tb - t_begin + CS - 1) / CS)) : (t_end - t_begin) / CS;
    const int r = l & 15, cg = (w << 2) | (l >> 4);

    Rsrc rs;
    rs.k = rsrc(p.k + rowbase * kD, Tb); rs.v = rsrc(p.v + rowbase * kD, Tb);
    rs.g = rsrc(p.g + rowbase * kD, Tb); rs.th = rsrc(p.th + rowbase * kD, Tb);
    rs.q = rs.k;

    f32x16_t S[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) S[mt] = f32x16_t{};
    float rho[8];  // log2 decay of the chunks after the current one, per channel
#pragma unroll
    for (int e = 0; e < 8; ++e) rho[e] = 0.f;

    // chunks are visited last to first; two chunks of raw inputs are in flight
    Raw<CS, false> Ra, Rb;
    const int c0 = nch - 1;
    if (c0 >= 0) load_raw<CS, false>(Ra, rs, t_begin + c0 * CS, r, cg);
    if (c0 >= 1) load_raw<CS, false>(Rb, rs, t_begin + (c0 - 1) * CS, r, cg);
    for (int c = c0; c >= 0; c -= 2) {
        state_chunk<TPR>(Ra, rs, t_begin + c * CS, c >= 2 ? t_begin + (c - 2) * CS : -1, sKbT, sVT,
                         S, rho, r, cg, l, w, h, l32, Tb);
        if (c >= 1)
            state_chunk<TPR>(Rb, rs, t_begin + (c - 1) * CS, c >= 3 ? t_begin + (c - 3) * CS : -1,
                             sKbT, sVT, S, rho, r, cg, l, w, h, l32, Tb);
    }
    float *So = p.wsS + ((size_t)sub * p.BH + bh) * kD * kD;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) So[(32 * mt + 8 * (i >> 2) + 4 * h + (i & 3)) * kD + 32 * w + l32] = S[mt][i];
    if (r == 0) {
        float *A = p.wsA + ((size_t)sub * p.BH + bh) * kD + 8 * cg;
#pragma unroll
        for (int e = 0; e < 8; ++e) A[e] = rho[e];
    }
}

// Phase 2: run the sub-segment states left to right,
//   S <- diag(2^{A_j}) S + S_loc[j],
// storing S into the slot of the last sub-segment of every segment (the
// incoming state of the next segment).  One thread per (b,h, 4 consecutive
// state elements of one row); all loads of a thread are independent and issued
// up front.
__global__ __launch_bounds__(256)
void scan_combine_kernel(const float *__restrict__ S0, float *wsS, const float *__restrict__ wsA,
                         int BH, int nsub, int P) {
    const size_t idx4 = (size_t)blockIdx.x * 256 + threadIdx.x;  // float4 index
    const size_t per4 = (size_t)kD * kD / 4;
    if (idx4 >= (size_t)BH * per4) return;
    const size_t bh = idx4 / per4;
    const int i = (int)((idx4 % per4) / (kD / 4));
    float4 s = S0 ? reinterpret_cast<const float4 *>(S0)[idx4] : make_float4(0.f, 0.f, 0.f, 0.f);
    constexpr int kBatch = 8;
    for (int j0 = 0; j0 < nsub; j0 += kBatch) {
        float4 x[kBatch];
        float a[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = j0 + u;
            if (j < nsub) {
                x[u] = reinterpret_cast<const float4 *>(wsS)[(size_t)j * BH * per4 + idx4];
                a[u] = wsA[((size_t)j * BH + bh) * kD + i];
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = j0 + u;
            if (j < nsub) {
                const float d = exp2_fast(a[u]);
                s.x = fmaf(d, s.x, x[u].x); s.y = fmaf(d, s.y, x[u].y);
                s.z = fmaf(d, s.z, x[u].z); s.w = fmaf(d, s.w, x[u].w);
                if ((j + 1) % P == 0) reinterpret_cast<float4 *>(wsS)[(size_t)j * BH * per4 + idx4] = s;
            }
        }
    }
}

struct Plan3 {
    int G, per_seg, P, sub;  // segments, chunks per segment, sub-segments, chunks per sub-segment
};

Plan3 plan3(long long BH, long long nchunks) {
    Plan3 q{1, (int)nchunks, 1, (int)nchunks};
    long long G = (kCUs + BH - 1) / BH;  // phase 3: one 8-wave workgroup per CU
    if (G > nchunks) G = nchunks;
    if (G < 1) G = 1;
    const long long per_seg = (nchunks + G - 1) / G;
    G = (nchunks + per_seg - 1) / per_seg;
    q.G = (int)G;
    q.per_seg = (int)per_seg;
    if (G > 1) {
        // phase 1: ~1.5 workgroups per CU (it is bandwidth-bound; more sub-segments
        // only add state traffic to the combine)
        long long P = (3 * kCUs + (G - 1) * BH) / (2 * (G - 1) * BH);
        if (P < 1) P = 1;
        if (P > per_seg) P = per_seg;
        const long long sub = (per_seg + P - 1) / P;
        q.P = (int)((per_seg + sub - 1) / sub);
        q.sub = (int)sub;
    }
    return q;
}

}  // namespace

ScanPlan plan_scan(int B, int H, int T, int dk, int dv, int chunk, int dtype) {
    ScanPlan pl{false, 1, 0};
    if (!(dtype == 1 && dk == kD && dv == kD && (chunk == 32 || chunk == 64) && T < kMaxT)) return pl;
    pl.mfma = true;
    const long long BH = (long long)B * H;
    const long long nchunks = (T + chunk - 1) / chunk;
    if (nchunks == 0 || BH == 0) return pl;
    const Plan3 q = plan3(BH, nchunks);
    pl.segments = q.G;
    if (q.G > 1) pl.workspace_bytes = (size_t)(q.G - 1) * q.P * BH * (kD * kD + kD) * sizeof(float);
    return pl;
}

void launch_scan_mfma(const ScanArgs &a, const ScanPlan &pl, hipStream_t st) {
    (void)pl;
    const int BH = a.B * a.H;
    const int nchunks = (a.T + a.chunk - 1) / a.chunk;
    const Plan3 q = plan3(BH, nchunks);
    Params p;
    p.q = (const bf16_t *)a.q; p.k = (const bf16_t *)a.k; p.v = (const bf16_t *)a.v;
    p.g = (const bf16_t *)a.g; p.th = (const bf16_t *)a.tau;
    p.S0 = a.S0; p.o = (bf16_t *)a.o; p.S_T = a.S_T;
    const int nsub = (q.G - 1) * q.P;
    p.wsS = (float *)a.workspace;
    p.wsA = p.wsS ? p.wsS + (size_t)nsub * BH * kD * kD : nullptr;
    p.BH = BH; p.T = a.T; p.G = q.G; p.seg_len = q.per_seg * a.chunk; p.P = q.P;
    p.sub_len = q.sub * a.chunk;
    p.cu = a.cu; p.H = a.H; p.total = a.total;
    p.order = a.cu ? a.order : nullptr;
    const bool vl = a.cu != nullptr;
    if (q.G > 1) {
        if (vl) hipLaunchKernelGGL(scan_state_kernel<true>, dim3(nsub * BH), dim3(256), 0, st, p);
        else hipLaunchKernelGGL(scan_state_kernel<false>, dim3(nsub * BH), dim3(256), 0, st, p);
        const size_t n4 = (size_t)BH * kD * kD / 4;
        hipLaunchKernelGGL(scan_combine_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st,
                           a.S0, p.wsS, p.wsA, BH, nsub, q.P);
    }
    const dim3 grid(q.G * BH), blk(512);
    if (a.chunk == 64) {
        if (vl) hipLaunchKernelGGL((scan_full_kernel<64, true>), grid, blk, 0, st, p);
        else hipLaunchKernelGGL((scan_full_kernel<64, false>), grid, blk, 0, st, p);
    } else {
        if (vl) hipLaunchKernelGGL((scan_full_kernel<32, true>), grid, blk, 0, st, p);
        else hipLaunchKernelGGL((scan_full_kernel<32, false>), grid, blk, 0, st, p);
    }
}

}  // namespace rodimus
