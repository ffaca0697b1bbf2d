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
// Kh needs 2^{-Lam} to stay inside the fp32/bf16 range.  A 64-token chunk is
// therefore contracted as two 32-token halves, each with its own reference
// (Lam restarts at the half's first token; Kb of the first half is taken to
// the half's end): the first half's outputs, the state carried through the
// first half, then the second half's outputs from that state, so that no
// score tile spans both halves.  A chunk in which a half's decay span
// max_i(-Lam[31, i]) exceeds kSpan2 is processed token by token on the VALU
// instead (same result).  Kb never overflows (its exponent is <= 0).
//
// Segment-parallel form.  So that the grid fills the GPU when B*H is small, the
// sequence of each (b, h) is cut into G segments (each a whole number of
// chunks), and every segment but the last into P sub-segments:
//   phase 1 (scan_state_kernel, scan_state.hip): each sub-segment's local end state (from zero)
//            and its total log2 decay, in 32-token chunks with two chunks of
//            inputs in flight.  Chunks are visited last to first, so the
//            decay of the later chunks folds into the operand exponent:
//            S_loc = sum_c (Kb_c * 2^{rho_c})^T V_c, rho_c = sum of Lam_end after c;
//            there is no state rescaling and nothing can overflow;
//   phase 2: S_in of every segment, left to right: folded by the output
//            pass's consumer waves from the sub-segment states before their
//            first chunk when a segment has at most kFoldMax of them before
//            it, else by scan_combine_kernel;
//   phase 3 (scan_full_kernel): every segment from its S_in, writing o.
// The sub-segment states are stored lane-major: float4 k (0..15) of lane
// (wave w, lane l) of a 4-wave MFMA layout at [k][64 w + l], i.e. the 4
// accumulator registers 4k..4k+3 of the lane that owns them in both kernels,
// so each lane reads its 64 values as 16 coalesced 16-byte loads.
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
#include <algorithm>

#include "launch.h"
#include "scan_mfma.h"

namespace rodimus {

namespace {

using namespace prefill;

constexpr int kCUs = 256;
constexpr int kFoldMax = 8;        // sub-segment states a consumer wave folds itself

// LDS buffer layout (bytes); rows padded by 16 bytes (conflict-free 16-byte reads)
constexpr int kQRow = kD + 8;      // bf16 per row of sQ / sK       [C][128]
constexpr int kOffQ = 0;
constexpr int kOffK = kOffQ + 64 * kQRow * 2;
constexpr int kOffKbT = kOffK + 64 * kQRow * 2;
constexpr int kOffVT = kOffKbT + kD * kTRow * 2;
constexpr int kOffGam = kOffVT + kD * kTRow * 2;   // 2^{decay} of each half: [2][128] fp32
constexpr int kBufBytes = kOffGam + 2 * kD * 4;
constexpr int kARow = 64 + 8;      // bf16 per row of sA [C][C] (token i, token j permuted)
constexpr int kSABytes = 64 * kARow * 2;

// The four consumer waves meet (an LDS counter; the producer waves are not
// involved), with a bounded wait.  Returns true if the wait gave up: what the
// other waves wrote may then be stale, and the caller poisons its outputs.
__device__ __forceinline__ bool consumer_barrier(int *sCBar, int &target, int l) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (l == 0) __hip_atomic_fetch_add(sCBar, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    target += 4;
    for (int spin = 0; spin < (1 << 24); ++spin) {
        if (__hip_atomic_load(sCBar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    const bool stale = __hip_atomic_load(sCBar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    return stale;
}

// ------------------------------------------------------------- phase 3 (full)
template <int C, bool VL, bool LR>
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
        // Lane (r, cg) holds tokens TPR r .. TPR r + TPR - 1 of the chunk for
        // channels 8 cg .. 8 cg + 7.  For the full-rank 64-token chunks the
        // wave pairs take the halves (r = 8 (w >> 1) + (l >> 3), cg = 8 (w & 1) +
        // (l & 7)), so that each load instruction reads 8 rows of 128 bytes, and
        // each half is scanned inside its waves; otherwise the 16 lanes of a row
        // hold the whole chunk of one channel group (16 rows of 64 bytes).
        constexpr bool kHalves = C == 64 && !LR;
        const int r = kHalves ? 8 * (w >> 1) + (l >> 3) : l & 15;
        const int cg = kHalves ? 8 * (w & 1) + (l & 7) : (w << 2) | (l >> 4);
        Rsrc rs;
        rs.q = rsrc(p.q + rowbase * kD, Tb); rs.k = rsrc(p.k + rowbase * kD, Tb);
        rs.v = rsrc(p.v + rowbase * kD, Tb);
        // low-rank gates: factor-row descriptors, the head's factors (B
        // operands) and the first chunk's factor rows
        __amdgpu_buffer_rsrc_t rzg, rzt;
        LrOps ops;
        Zops<NT> Z;
        if constexpr (LR) {
            const size_t zrow = (size_t)(bh / p.H) * p.T;
            rzg = rsrc_bytes(p.zg + zrow * kRank, Tb * (int)kZRow);
            rzt = rsrc_bytes(p.zt + zrow * kRank, Tb * (int)kZRow);
            lr_load_ops(ops, p.Ug, p.bg, p.Ut, p.bt, bh % p.H, w, l);
        } else {
            rs.g = rsrc(p.g + rowbase * kD, Tb);
            rs.th = rsrc(p.th + rowbase * kD, Tb);
        }
        Raw<C, true, LR> R;
        if constexpr (LR) {
            // Low rank: the first chunk in the order of the loop's prefetches
            // (v, the factor rows, then q and k), and the prefetches always
            // issued (from past the rows' end after the last chunk), so that
            // each wait of the in-order load counter is exact: the factor rows
            // are waited for without q and k, which are needed only after the
            // gate map.
            load_one<TPR>(R.v, rs.v, t_begin, r, cg);
            load_zops<NT>(Z, rzg, rzt, t_begin, l);
            load_one<TPR>(R.q, rs.q, t_begin, r, cg);
            load_one<TPR>(R.k, rs.k, t_begin, r, cg);
        } else {
            load_raw<C, true>(R, rs, t_begin, r, cg);
        }
        for (int kk = 0; kk <= nch; ++kk) {
            if (kk < nch) {
                const int t0 = t_begin + kk * C;
                char *buf = smem + (kk & 1) * kBufBytes;
                const bool more = kk + 1 < nch;
                float l2a[TPR][8], l2b[TPR][8], lend[8];
                const int tn = more ? t0 + C : kNoRow;  // low rank: the next chunk's loads
                if constexpr (LR) {
                    // logits on the matrix cores, staged in this wave's rows of
                    // the K-bar^T (g) and V^T (tau) areas, read back per lane
                    lr_stage<NT, kTRow>(Z, ops, buf + kOffKbT, buf + kOffVT, w, l);
                    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    uint32_t gw[8][TPR / 2], tw[8][TPR / 2];
                    lr_read<TPR, kTRow>(buf + kOffKbT, buf + kOffVT, r, cg, gw, tw);
                    store_vt<TPR, kTRow>(buf + kOffVT, cg, r, R.v);   // after the reads, in LDS order
                    load_one<TPR>(R.v, rs.v, tn, r, cg);
                    load_zops<NT>(Z, rzg, rzt, tn, l);
                    gates_scan_cols<C>(gw, tw, t0, t_end, r, l, l2a, l2b, lend);
                } else {
                    store_vt<TPR, kTRow>(buf + kOffVT, cg, r, R.v);
                    if (more) load_one<TPR>(R.v, rs.v, t0 + C, r, cg);
                    if constexpr (kHalves) gates_scan_half<C>(R.g, R.th, t0, t_end, r, l, l2a, l2b, lend);
                    else gates_scan_gt<C>(R.g, R.th, t0, t_end, r, l, l2a, l2b, lend);
                    if (more) load_gates<C, true>(R, rs, t0 + C, r, cg);
                }
                bool bad = false;
                float gam[8], gam1[8];  // 2^{decay} of the (first) half and of the second half
                bool second = false;    // this lane's tokens are in the second half
                if constexpr (kHalves) {
                    // lend is this wave pair's half total, Lam already from the half's start
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        bad |= lend[e] < -kSpan2;
                        gam[e] = exp2_fast(lend[e]);
                    }
                    second = r >= 8;
                } else if constexpr (NT == 2) {
                    // each half against its own reference: Lam at the first half's
                    // end (token 31, lane row 7) is taken off the second half's
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float lmid = bcast_lane(l2a[TPR - 1][e], (l & 48) | 7);
                        bad |= lmid < -kSpan2 || lend[e] - lmid < -kSpan2;
                        gam[e] = exp2_fast(lmid);
                        gam1[e] = exp2_fast(lend[e] - lmid);
                        if (r >= 8) {
#pragma unroll
                            for (int tt = 0; tt < TPR; ++tt) l2a[tt][e] -= lmid;
                        }
                    }
                    second = r >= 8;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        bad |= lend[e] < -kSpan2;
                        gam[e] = exp2_fast(lend[e]);
                        gam1[e] = 1.f;
                    }
                }
                if (kHalves ? (r & 7) == 0 : r == 0) {
                    // by halves: each wave pair writes its own half's factor
                    float *sg = reinterpret_cast<float *>(buf + kOffGam) + 8 * cg + (kHalves && second ? kD : 0);
                    *reinterpret_cast<float4 *>(sg) = make_float4(gam[0], gam[1], gam[2], gam[3]);
                    *reinterpret_cast<float4 *>(sg + 4) = make_float4(gam[4], gam[5], gam[6], gam[7]);
                    if (!kHalves && NT == 2) {
                        *reinterpret_cast<float4 *>(sg + kD) = make_float4(gam1[0], gam1[1], gam1[2], gam1[3]);
                        *reinterpret_cast<float4 *>(sg + kD + 4) = make_float4(gam1[4], gam1[5], gam1[6], gam1[7]);
                    }
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
                        kbT[e][tt] = kh[e] * (!kHalves && second ? gam1[e] : gam[e]);
                    }
                    const int t = TPR * r + tt;
                    store_q_row<kQRow>(buf + kOffQ, t, cg, qt);
                    store_q_row<kQRow>(buf + kOffK, t, cg, kh);
                }
                if (LR || more) {
                    load_one<TPR>(R.q, rs.q, LR ? tn : t0 + C, r, cg);
                    load_one<TPR>(R.k, rs.k, LR ? tn : t0 + C, r, cg);
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
    if (seg == 0 || p.fold) {
        // S0 (row-major), then, for a later segment, every earlier sub-segment
        // state folded in: S <- diag(2^{A_j}) S + S_j
        const float *S0 = p.S0 ? p.S0 + (size_t)bh * kD * kD : nullptr;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                S[mt][i] = S0 ? S0[(32 * mt + 8 * (i >> 2) + 4 * h + (i & 3)) * kD + n] : 0.f;
        const int nj = seg * p.P;
        for (int j = 0; j < nj; ++j) {
            const float4 *Sj = reinterpret_cast<const float4 *>(p.wsS + ((size_t)j * p.BH + bh) * kD * kD) + 64 * cw + l;
            const float4 *Dj = reinterpret_cast<const float4 *>(p.wsA + ((size_t)j * p.BH + bh) * kD);
            float4 x[16], d[16];
#pragma unroll
            for (int k4 = 0; k4 < 16; ++k4) {
                x[k4] = Sj[256 * k4];
                d[k4] = Dj[(32 * (k4 >> 2) + 8 * (k4 & 3) + 4 * h) >> 2];
            }
#pragma unroll
            for (int k4 = 0; k4 < 16; ++k4) {
                f32x16_t &A = S[k4 >> 2];
                const int i = 4 * (k4 & 3);
                A[i + 0] = fmaf(d[k4].x, A[i + 0], x[k4].x); A[i + 1] = fmaf(d[k4].y, A[i + 1], x[k4].y);
                A[i + 2] = fmaf(d[k4].z, A[i + 2], x[k4].z); A[i + 3] = fmaf(d[k4].w, A[i + 3], x[k4].w);
            }
        }
    } else {
        // the combine's incoming state (lane-major)
        const float4 *Sin = reinterpret_cast<const float4 *>(p.wsS + ((size_t)(seg * p.P - 1) * p.BH + bh) * kD * kD) +
                            64 * cw + l;
#pragma unroll
        for (int k4 = 0; k4 < 16; ++k4) {
            const float4 x = Sin[256 * k4];
            f32x16_t &A = S[k4 >> 2];
            const int i = 4 * (k4 & 3);
            A[i + 0] = x.x; A[i + 1] = x.y; A[i + 2] = x.z; A[i + 3] = x.w;
        }
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
                bool fstale = false;
                if constexpr (LR) {
                    // The chunk's gate logits, recomputed on the matrix cores as the
                    // producers do (consumer wave cw: channels 32cw..32cw+31) into the
                    // K-bar^T (g) and V^T (tau) areas, which the fallback leaves unused.
                    const size_t zrow = (size_t)(bh / p.H) * p.T;
                    LrOps cops;
                    Zops<NT> cz;
                    lr_load_ops(cops, p.Ug, p.bg, p.Ut, p.bt, bh % p.H, cw, l);
                    load_zops<NT>(cz, rsrc_bytes(p.zg + zrow * kRank, Tb * (int)kZRow),
                                  rsrc_bytes(p.zt + zrow * kRank, Tb * (int)kZRow), t0, l);
                    lr_stage<NT, kTRow>(cz, cops, buf + kOffKbT, buf + kOffVT, cw, l);
                    fstale = consumer_barrier(sCBar, cbar_target, l);
                }
                // The inputs of each 4-token sub-block (element k of the lane: token
                // k >> 1, channel l + 64 (k & 1); v of its column n for the 4 tokens)
                // are loaded in one batch: one memory round trip per sub-block.
                struct FallRaw {
                    bf16_t g[8], th[8], k[8], q[8], v[4];
                };
                auto fall_load = [&](FallRaw &R, int sb) {
#pragma unroll
                    for (int k8 = 0; k8 < 8; ++k8) {
                        const int t = t0 + sb + (k8 >> 1);
                        if (t < t_end) {
                            const size_t x = (rowbase + t) * kD + l + 64 * (k8 & 1);
                            if constexpr (!LR) {
                                R.g[k8] = p.g[x];
                                R.th[k8] = p.th[x];
                            }
                            R.k[k8] = p.k[x];
                            R.q[k8] = p.q[x];
                        }
                    }
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
                        if (t0 + sb + tt < t_end) R.v[tt] = p.v[(rowbase + t0 + sb + tt) * kD + n];
                };
                auto fall_sub = [&](int sb) {
                    FallRaw R;
                    fall_load(R, sb);
#pragma unroll
                    for (int k8 = 0; k8 < 8; ++k8) {
                        const int tt = k8 >> 1, i = l + 64 * (k8 & 1), e = tt * 128 + i, t = t0 + sb + tt;
                        float a = 1.f, bk = 0.f, qq = 0.f;
                        if (t < t_end) {
                            float gv, tv, l2a, l2b;
                            if constexpr (LR) {
                                const int so = (i * kTRow + sb + tt) * 2;
                                gv = bf2f(*reinterpret_cast<const bf16_t *>(buf + kOffKbT + so));
                                tv = bf2f(*reinterpret_cast<const bf16_t *>(buf + kOffVT + so));
                            } else {
                                gv = bf2f(R.g[k8]);
                                tv = bf2f(R.th[k8]);
                            }
                            ddts_log2_gates(gv, tv, l2a, l2b);
                            a = exp2_fast(l2a);
                            bk = exp2_fast(l2b) * bf2f(R.k[k8]);
                            qq = bf2f(R.q[k8]);
                        }
                        fa[e] = a; fb[e] = bk; fq[e] = qq;
                    }
                    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                    __builtin_amdgcn_wave_barrier();
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) {
                        const int t = t0 + sb + tt;
                        if (t >= t_end) continue;
                        const float vn = bf2f(R.v[tt]);
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
                        if (h == 0) p.o[(rowbase + t) * kD + n] = fstale ? (bf16_t)0x7fc0 : f2bf(part);
                    }
                    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                };
                for (int sb = 0; sb < C; sb += 4) fall_sub(sb);
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
                // masked score tiles A^T[j][i] = Kh[j] . Qt[i] (j <= i) of each half
                // against its own reference: consumer wave cw builds the diagonal
                // tile of half cw and stores it as A[i][j] (j in permuted order)
                if (cw < NT) {
                    const int It = cw;
                    f32x16_t at = {};
#pragma unroll
                    for (int s = 0; s < 8; ++s) {
                        const bf16x8_t a = lds16(buf, kOffK + ((32 * It + l32) * kQRow + 16 * s + 8 * h) * 2);
                        const bf16x8_t b = lds16(buf, kOffQ + ((32 * It + l32) * kQRow + 16 * s + 8 * h) * 2);
                        at = mfma(a, b, at);
                    }
                    const int i = 32 * It + l32;
#pragma unroll
                    for (int a4 = 0; a4 < 4; ++a4) {
                        float x[4];
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4) {
                            const int j = 32 * It + 8 * a4 + 4 * h + r4;
                            x[r4] = (j <= i) ? at[4 * a4 + r4] : 0.f;
                        }
                        *reinterpret_cast<uint2 *>(sA + (i * kARow + perm16(32 * It + 8 * a4 + 4 * h)) * 2) =
                            make_uint2(pack2(x[0], x[1]), pack2(x[2], x[3]));
                    }
                }
                // the four consumer waves meet; a wait that gave up leaves score
                // tiles that may be stale: this chunk's outputs are then written as
                // NaN, never as silent garbage
                const bool stale = consumer_barrier(sCBar, cbar_target, l);
                const float *gam = reinterpret_cast<const float *>(buf + kOffGam);
                // Per half: o^T tiles (32 value channels, this wave's, x 32 tokens) =
                // S^T Qt^T + V^T A^T, the same fragments as o = Qt S + A V with the
                // operands swapped, so that a lane holds one token and 4
                // consecutive channels per register group; and the state through
                // the half, S <- diag(gamma) S + Kb^T V.  For two halves the first
                // half's state update is issued before its outputs (which use the
                // bf16 state taken before it), so that its latency is hidden.
                auto out = [&](int It) {
                    f32x16_t acc = {};
#pragma unroll
                    for (int s = 0; s < 8; ++s)
                        acc = mfma(Sb[s], lds16(buf, kOffQ + ((32 * It + l32) * kQRow + 16 * s + 8 * h) * 2), acc);
#pragma unroll
                    for (int s = 2 * It; s < 2 * It + 2; ++s)
                        acc = mfma(vB[s], lds16(sA, ((32 * It + l32) * kARow + 16 * s + 8 * h) * 2), acc);
                    const int t = t0 + 32 * It + l32;
                    if (t < t_end) {
                        bf16_t *op = p.o + (rowbase + t) * kD + 32 * cw + 4 * h;
                        // (the NaN is written as a bit pattern: this file is built
                        // without NaN semantics for arithmetic)
                        constexpr uint32_t kNaN2 = 0x7fc07fc0u;
#pragma unroll
                        for (int a4 = 0; a4 < 4; ++a4)
                            *reinterpret_cast<uint2 *>(op + 8 * a4) =
                                stale ? make_uint2(kNaN2, kNaN2)
                                      : make_uint2(pack2(acc[4 * a4 + 0], acc[4 * a4 + 1]),
                                                   pack2(acc[4 * a4 + 2], acc[4 * a4 + 3]));
                    }
                };
                auto adv = [&](int It) {
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                        for (int a4 = 0; a4 < 4; ++a4) {
                            const float4 gm = *reinterpret_cast<const float4 *>(gam + kD * It + 32 * mt + 8 * a4 + 4 * h);
                            S[mt][4 * a4 + 0] *= gm.x; S[mt][4 * a4 + 1] *= gm.y;
                            S[mt][4 * a4 + 2] *= gm.z; S[mt][4 * a4 + 3] *= gm.w;
                        }
#pragma unroll
                        for (int s = 2 * It; s < 2 * It + 2; ++s)
                            S[mt] = mfma(lds16(buf, kOffKbT + ((32 * mt + l32) * kTRow + 16 * s + 8 * h) * 2), vB[s], S[mt]);
                    }
                };
                if constexpr (NT == 2) {
                    adv(0);
                    out(0);
#pragma unroll
                    for (int s = 0; s < 8; ++s) Sb[s] = cvt8(S[s >> 1], 8 * (s & 1));
                    out(1);
                    adv(1);
                } else {
                    out(0);
                    adv(0);
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

// Phase 2 when the output pass does not fold: run the sub-segment states left
// to right, S <- diag(2^{A_j}) S + S_loc[j], storing S into the slot of the
// last sub-segment of every segment (the incoming state of the next segment).
// One thread per (b,h, float4 of the lane-major layout: 4 rows of one state
// column); all loads of a thread are independent and issued up front.
__global__ __launch_bounds__(256)
void scan_combine_kernel(const float *__restrict__ S0, float *wsS, const float *__restrict__ wsA,
                         int BH, int nsub, int P) {
    const size_t idx4 = (size_t)blockIdx.x * 256 + threadIdx.x;  // float4 index
    constexpr size_t per4 = (size_t)kD * kD / 4;                 // 4096 float4 per state
    if (idx4 >= (size_t)BH * per4) return;
    const size_t bh = idx4 / per4;
    const int rem = (int)(idx4 % per4), k4 = rem >> 8, lane = rem & 255;
    const int w = lane >> 6, l = lane & 63;
    const int row0 = 32 * (k4 >> 2) + 8 * (k4 & 3) + 4 * (l >> 5), col = 32 * w + (l & 31);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (S0) {
        const float *b = S0 + bh * kD * kD + (size_t)row0 * kD + col;
        s = make_float4(b[0], b[kD], b[2 * kD], b[3 * kD]);
    }
    constexpr int kBatch = 8;
    for (int j0 = 0; j0 < nsub; j0 += kBatch) {
        float4 x[kBatch], d[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = j0 + u;
            if (j < nsub) {
                x[u] = reinterpret_cast<const float4 *>(wsS)[(size_t)j * BH * per4 + idx4];
                d[u] = *reinterpret_cast<const float4 *>(wsA + ((size_t)j * BH + bh) * kD + row0);
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = j0 + u;
            if (j < nsub) {
                s.x = fmaf(d[u].x, s.x, x[u].x); s.y = fmaf(d[u].y, s.y, x[u].y);
                s.z = fmaf(d[u].z, s.z, x[u].z); s.w = fmaf(d[u].w, s.w, x[u].w);
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

uint64_t scan_mfma_launch_items(long long BH, int T, int chunk) {
    const long long nchunks = ((long long)T + chunk - 1) / chunk;
    if (BH <= 0 || nchunks <= 0) return 0;
    const Plan3 q = plan3(BH, nchunks);
    uint64_t m = (uint64_t)q.G * BH * 512;                                   // output pass
    if (q.G > 1) {
        m = std::max<uint64_t>(m, (uint64_t)(q.G - 1) * q.P * BH * 256);     // state pass
        m = std::max<uint64_t>(m, ((uint64_t)BH * kD * kD / 4 + 255) / 256 * 256);  // combine
    }
    return m;
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
    p.fold = nsub <= kFoldMax;
    p.sub_len = q.sub * a.chunk;
    p.cu = a.cu; p.H = a.H; p.total = a.total;
    p.order = a.cu ? a.order : nullptr;
    p.zg = (const bf16_t *)a.zg; p.zt = (const bf16_t *)a.zt;
    p.Ug = (const bf16_t *)a.Ug; p.Ut = (const bf16_t *)a.Ut; p.bg = a.bg; p.bt = a.bt;
    const bool vl = a.cu != nullptr, lr = a.zg != nullptr;
    if (q.G > 1) {
        launch_scan_state(p, vl, lr, (unsigned)(nsub * BH), st);
        if (!p.fold) {
            const size_t n4 = (size_t)BH * kD * kD / 4;
            hipLaunchKernelGGL(scan_combine_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st,
                               a.S0, p.wsS, p.wsA, BH, nsub, q.P);
        }
    }
    const dim3 grid(q.G * BH), blk(512);
    if (a.chunk == 64) {
        if (lr) hipLaunchKernelGGL((scan_full_kernel<64, false, true>), grid, blk, 0, st, p);
        else if (vl) hipLaunchKernelGGL((scan_full_kernel<64, true, false>), grid, blk, 0, st, p);
        else hipLaunchKernelGGL((scan_full_kernel<64, false, false>), grid, blk, 0, st, p);
    } else {
        if (lr) hipLaunchKernelGGL((scan_full_kernel<32, false, true>), grid, blk, 0, st, p);
        else if (vl) hipLaunchKernelGGL((scan_full_kernel<32, true, false>), grid, blk, 0, st, p);
        else hipLaunchKernelGGL((scan_full_kernel<32, false, false>), grid, blk, 0, st, p);
    }
}

}  // namespace rodimus
