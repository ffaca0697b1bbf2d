// scan_bwd_mfma.hip -- backward of the chunked DDTS-gated scan on gfx950
// matrix cores (bf16 inputs, dk = dv = 128; fp32 gradients, fp32 state
// arithmetic, bf16 matrix-core operands).
//
// The per-chunk gradient formulas are those of scan_bwd_body.h (CodeFuse
// article, Rodimus block paragraph: S_t = diag(a_t) S_{t-1} + (beta_t k_t)^T v_t,
// o_t = q_t S_t).  Here the intra-chunk pairwise weights are factored as
// 2^{Lam_i} * 2^{mu_j - Lam_j} (base-2 units, Lam = in-chunk inclusive
// cumulative log2 a, mu = log2 beta), so that every product is a matrix-core
// contraction.  With Qt = q 2^{Lam}, Kh = k 2^{mu - Lam}, Kb = Kh 2^{Gam}, S
// the state entering a 32-token chunk and G the gradient of the state leaving
// it:
//     dP  = tril(dO V^T)          A  = tril(Qt Kh^T)
//     dq  = 2^{Lam} (dP Kh + dO S^T)
//     dk  = 2^{mu-Lam} (dP^T Qt) + 2^{mu+Gam-Lam} (V G^T)
//     dv  = A^T dO + Kb G
//     dLam = q dq - k dk,  dmu = k dk,
//     dGam = sum_j Kb_j (V G^T)_j + 2^{Gam} rowsum(G * S),
//     dlam_t = sum_{t' >= t} dLam_t' + dGam,
// then the gate chain rule (natural-log gradients; 2^{x/ln 2} = e^x).  A chunk
// whose decay span exceeds kSpan2 would overflow Kh; such chunks are listed and
// handed to the exact pairwise routine of scan_bwd_body.h.
//
// Kernels:
//   bwd_state_kernel    the state (forward order) and its gradient (reverse
//                       order) per segment of 32-token chunks, on matrix cores;
//                       writes a bf16 checkpoint of each at every chunk: S
//                       entering the chunk and G leaving it, in fragment order
//                       (frag_index), so that the gradient kernel loads them as
//                       ready operands.  Segments start from zero (the first
//                       from S0, the last from dS_T); each writes its fp32 edge
//                       state and total decay.
//   bwd_combine_kernel  (several segments only) runs the segment edges across
//                       the sequence: the true state entering and gradient
//                       leaving each segment (fragment order, bf16), and dS0.
//                       A checkpoint c of segment s is completed on load as
//                       S_c = S_loc_c + diag(2^{D_c}) S_in(s).
//   bwd_grad_kernel     one workgroup per 32-token chunk: the two checkpoints
//                       (G's transposed operands through LDS: an identity
//                       product per 32x32 block turns its rows into columns),
//                       all products above on the matrix cores and the
//                       element-wise epilogue in the producer-lane layout.  Two
//                       workgroups per CU.
//   bwd_fallback_kernel the listed wide-span chunks, with the exact routine.
#include <algorithm>

#include "launch.h"
#include "mfma_common.h"
#include "scan_bwd_body.h"

namespace rodimus {

namespace {

constexpr int kCk = 32;              // tokens per checkpoint (one gradient workgroup)
constexpr int kSub = 32;             // tokens per gradient workgroup
constexpr int kFrag = 32 * 64 * 8;   // bf16 per 128x128 matrix in fragment order (32 KiB)
constexpr int kT32 = 32 + 8;         // bf16 per transposed LDS row of 32 tokens (+16 B)
constexpr int kQR = kD + 8;          // bf16 per token row [t][128] (+16 B)
constexpr int kSR = kD + 4;          // fp32 per staging row (+16 B)
constexpr int kSlowWG = 256;         // fallback workgroups (one fp32 S/G scratch pair each)
constexpr int kMaxT = 1 << 23;       // 32-bit buffer offsets (T * 256 bytes)
constexpr int kCUs = 256;

struct P {
    const bf16_t *q, *k, *v, *g, *th, *dO;
    const float *S0, *dST;
    float *dq, *dk, *dv, *dg, *dth, *dS0;
    bf16_t *ckS, *ckG;            // [BH][nck] checkpoints, fragment order
    float *sigS, *sigG;           // [BH][nck][128] 2^{log2 decay to / from the segment edge}
    float *segS, *segG;           // [BH][nseg][128][128] fp32 segment edge states (row-major)
    float *segDS, *segDG;         // [BH][nseg][128] total log2 decay of each segment
    bf16_t *fixS, *fixG;          // [BH][nseg] incoming state / outgoing gradient, fragment order
    int *bad;                     // [0] = count, then entries bh * nck + chunk
    float *slot;                  // [kSlowWG][2][128][128] fallback scratch
    int BH, T, nck, nseg, seg_ck;
    // packed variable-length batch (seq_rows): sequence s = bh / H in rows
    // cu[s] .. cu[s+1]-1 of head h = bh % H's [total] rows; T = longest length
    const int *cu;
    int H, total;
    const int *order;  // packed batch: longest-first order of the sequences, or null
};

// ------------------------------------------------------------ state passes
// Role 0: S (forward over the segment); role 1: G (reverse), in 32-token steps
// with a checkpoint at every step.  Wave w keeps the transposed 128 x 32 slice
// X^T[n][32w..32w+31] (rows n = value channel) in accumulators.
constexpr int kStS = 32;   // tokens per state step
__global__ __launch_bounds__(256, 2)
void bwd_state_kernel(P p) {
    __shared__ __attribute__((aligned(16))) char smem[2 * kD * kT32 * 2 + 2 * kD * 4];
    char *sX = smem, *sY = smem + kD * kT32 * 2;
    // log2 decay of the current step per channel, and its power of two
    float *sGam = reinterpret_cast<float *>(smem + 2 * kD * kT32 * 2), *sGamE = sGam + kD;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, l32 = l & 31;
    // the two roles of one (b,h, segment) are adjacent block ids, so that in a
    // packed batch both roles of the longest sequences are dispatched first
    const bool rev = blockIdx.x & 1;
    const int id = (int)(blockIdx.x >> 1);
    const int bh = seq_head(p.order, p.H, uni(id % p.BH)), seg = uni(id / p.BH);
    if (blockIdx.x == 0 && tid == 0) p.bad[0] = 0;
    size_t rowbase;
    int len;
    seq_rows(p.cu, p.H, p.total, p.T, bh, rowbase, len);
    // this segment's intervals that hold tokens of the sequence (none: the
    // segment passes the state and its gradient through unchanged)
    const int ncl = (len + kCk - 1) / kCk;
    const int c_hi = min(min(p.nck, (seg + 1) * p.seg_ck), ncl), c_lo = min(seg * p.seg_ck, c_hi);
    const int r = l & 15, cg = (w << 2) | (l >> 4);
    const int rr = 32 * w + l32;  // key channel of this lane's transposed columns (role 1: also n of G)

    Rsrc rs;  // X operand tensor (k or q) in .k, Y operand tensor (v or dO) in .v
    rs.k = rsrc((rev ? p.q : p.k) + rowbase * kD, len);
    rs.v = rsrc((rev ? p.dO : p.v) + rowbase * kD, len);
    rs.g = rsrc(p.g + rowbase * kD, len);
    rs.th = rsrc(p.th + rowbase * kD, len);
    rs.q = rs.k;

    f32x16_t A[4];
    const float *init = rev ? (seg == p.nseg - 1 && p.dST ? p.dST + (size_t)bh * kD * kD : nullptr)
                            : (seg == 0 && p.S0 ? p.S0 + (size_t)bh * kD * kD : nullptr);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (init) x = *reinterpret_cast<const float4 *>(init + rr * kD + 32 * q + 8 * a4 + 4 * h);
            A[q][4 * a4 + 0] = x.x; A[q][4 * a4 + 1] = x.y; A[q][4 * a4 + 2] = x.z; A[q][4 * a4 + 3] = x.w;
        }
    }
    float dacc = 0.f;  // log2 decay between the segment edge and the current step, channel rr

    Raw<kStS, false> R;
    const int nst = c_hi - c_lo;
    const int st_first = rev ? c_hi - 1 : c_lo;
    if (nst > 0) load_raw<kStS, false>(R, rs, st_first * kStS, r, cg);
    for (int it = 0; it < nst; ++it) {
        const int stp = rev ? st_first - it : st_first + it;
        const int t0 = stp * kStS;
        {
            // checkpoint: S entering chunk stp (role 0) / G leaving it (role 1)
            const size_t ck = (size_t)bh * p.nck + stp;
            bf16_t *dA = (rev ? p.ckG : p.ckS) + ck * kFrag;
#pragma unroll
            for (int s = 0; s < 8; ++s)
                st_stream(reinterpret_cast<bf16x8_t *>(dA + ((8 * w + s) * 64 + l) * 8), cvt8(A[s >> 1], 8 * (s & 1)));
            if (h == 0) (rev ? p.sigG : p.sigS)[ck * kD + rr] = exp2_fast(dacc);
        }

        // operands: X^T (Kb or Qt) and Y^T (V or dO), tokens in permuted order
        float l2a[2][8], l2b[2][8], lend[8];
        gates_scan_gt<kStS>(R.g, R.th, t0, len, r, l, l2a, l2b, lend);
        float xT[8][2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            float xf[8];
            unpack8(R.k[tt], xf);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                xT[e][tt] = xf[e] * exp2_fast(rev ? l2a[tt][e] : l2b[tt][e] + lend[e] - l2a[tt][e]);
        }
        store_vt<2, kT32>(sY, cg, r, R.v);
#pragma unroll
        for (int e = 0; e < 8; ++e) store_t_rows<2, kT32>(sX, 8 * cg + e, r, xT[e]);
        if (r == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sGam[8 * cg + e] = lend[e];
                sGamE[8 * cg + e] = exp2_fast(lend[e]);
            }
        }
        if (it + 1 < nst) load_raw<kStS, false>(R, rs, (rev ? stp - 1 : stp + 1) * kStS, r, cg);
        __syncthreads();

        // A (X^T layout): columns rr decay by 2^{Gam[rr]}; A += Y^T X
        const float gr = sGam[rr];
        dacc += gr;
        const float er = sGamE[rr];
        const bf16x8_t xB0 = lds16(sX, (rr * kT32 + 8 * h) * 2), xB1 = lds16(sX, (rr * kT32 + 16 + 8 * h) * 2);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            A[q] *= er;
            A[q] = mfma(lds16(sY, ((32 * q + l32) * kT32 + 8 * h) * 2), xB0, A[q]);
            A[q] = mfma(lds16(sY, ((32 * q + l32) * kT32 + 16 + 8 * h) * 2), xB1, A[q]);
        }
        __syncthreads();
    }

    // segment edge: local end state (role 0) / local entering gradient (role 1)
    float *edge;
    if (p.nseg == 1) {
        if (!rev || !p.dS0) return;
        edge = p.dS0 + (size_t)bh * kD * kD;  // one segment: the gradient entering it is dS0
    } else {
        const size_t sb = (size_t)bh * p.nseg + seg;
        edge = (rev ? p.segG : p.segS) + sb * kD * kD;
        if (h == 0) (rev ? p.segDG : p.segDS)[sb * kD + rr] = dacc;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
            *reinterpret_cast<float4 *>(edge + rr * kD + 32 * q + 8 * a4 + 4 * h) =
                make_float4(A[q][4 * a4 + 0], A[q][4 * a4 + 1], A[q][4 * a4 + 2], A[q][4 * a4 + 3]);
}

// ----------------------------------------------------------------- combine
// The state entering each segment (left to right) and the gradient leaving
// each segment (right to left), stored bf16 in fragment order for the gradient
// kernel; the gradient entering segment 0 is dS0.  One thread per (b,h,
// fragment slot): the 8 values one lane holds of one operand fragment, which
// frag_index places at row r, columns c0..c0+3 and c0+8..c0+11, so that each
// load is a 16-byte run of a row and each store one 16-byte slot.
__global__ __launch_bounds__(256)
void bwd_combine_kernel(P p) {
    constexpr int kSlots = kFrag / 8;  // 2048 per 128 x 128 matrix
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)p.BH * kSlots) return;
    const int bh = (int)(idx / kSlots), slot = (int)(idx % kSlots);
    const int f = slot >> 6, ln = slot & 63;
    const int r = 32 * (f >> 3) + (ln & 31), c0 = 16 * (f & 7) + 4 * (ln >> 5);
    auto row8 = [&](const float *m, float (&x)[8]) {
        const float4 a = *reinterpret_cast<const float4 *>(m + r * kD + c0);
        const float4 b = *reinterpret_cast<const float4 *>(m + r * kD + c0 + 8);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    };
    auto put = [&](bf16_t *m, const float (&x)[8]) {
        *reinterpret_cast<uint4 *>(m + (size_t)slot * 8) =
            make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
    };
    float S[8], G[8], x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) S[e] = G[e] = 0.f;
    for (int s = 0; s < p.nseg; ++s) {
        const size_t sb = (size_t)bh * p.nseg + s;
        if (s > 0) put(p.fixS + sb * kFrag, S);
        const float d = exp2_fast(p.segDS[sb * kD + r]);
        row8(p.segS + sb * kD * kD, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) S[e] = fmaf(d, S[e], x[e]);
    }
    for (int s = p.nseg - 1; s >= 0; --s) {
        const size_t sb = (size_t)bh * p.nseg + s;
        if (s < p.nseg - 1) put(p.fixG + sb * kFrag, G);
        const float d = exp2_fast(p.segDG[sb * kD + r]);
        row8(p.segG + sb * kD * kD, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) G[e] = fmaf(d, G[e], x[e]);
    }
    if (p.dS0) {
        float *o = p.dS0 + (size_t)bh * kD * kD + r * kD + c0;
        *reinterpret_cast<float4 *>(o) = make_float4(G[0], G[1], G[2], G[3]);
        *reinterpret_cast<float4 *>(o + 8) = make_float4(G[4], G[5], G[6], G[7]);
    }
}

// ---------------------------------------------------------- gradient kernel
// LDS (bytes).  Token rows [32][136] bf16 (channels permuted): Qt, Kh, Kb, dO,
// V; transposed rows [128][40] bf16 (tokens permuted): Qt^T, Kh^T, dO^T; the
// fp32 decay term.  G's columns pass through the Qt^T / Kh^T area before those
// are written; the fp32 staging of the epilogue aliases all operand rows.
constexpr int kRowB = kSub * kQR * 2;           // 8704
constexpr int kTB = kD * kT32 * 2;              // 10240
constexpr int kOffQr = 0, kOffKr = kRowB, kOffKbr = 2 * kRowB, kOffDOr = 3 * kRowB, kOffVr = 4 * kRowB;
constexpr int kOffQT = 5 * kRowB, kOffKT = kOffQT + kTB, kOffDOT = kOffKT + kTB;
constexpr int kOffDec = kOffDOT + kTB;
constexpr int kGradLDS = kOffDec + kD * 4;
static_assert(4 * kSub * kSR * 4 <= kOffDec, "staging fits in the dead operand rows");
static_assert(64 * kD * 2 <= 2 * kTB, "half of G's columns fit in the Qt^T / Kh^T area");
static_assert(kGradLDS <= 80 * 1024, "two workgroups per CU");

__device__ __forceinline__ bf16x8_t pack_frag(const float (&x)[8]) {
    return __builtin_bit_cast(bf16x8_t, make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]),
                                                   pack2(x[4], x[5]), pack2(x[6], x[7])));
}
__device__ __forceinline__ float bf_round(float x) { return lo_bf(pack2(x, 0.f)); }
__device__ __forceinline__ uint4 ld_raw(const bf16_t *base, int f, int l) {
    return *reinterpret_cast<const uint4 *>(base + ((size_t)f * 64 + l) * 8);
}
// x + sig * y for 8 packed bf16, rounded back to bf16
__device__ __forceinline__ uint4 fix_raw(const uint4 &x, const uint4 &y, float sig) {
    float a[8], b[8];
    unpack8(x, a);
    unpack8(y, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = fmaf(sig, b[e], a[e]);
    return __builtin_bit_cast(uint4, pack_frag(a));
}

// Identity operands: fragment j of lane (l32, h) holds 1 where the column of
// k-slot 8h + e of the j-th 16-column block equals l32.
__device__ __forceinline__ void make_ident(bf16x8_t (&Id)[2], int l32, int h) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (16 * j + perm16(8 * h + e) == l32) ? 1.f : 0.f;
        Id[j] = pack_frag(x);
    }
}
// byte offset of 16-byte chunk ch (0..15) of column n (0..63 within a pass) of
// G in the transposition area (XOR-swizzled by column: no bank conflicts, no
// padding)
__device__ __forceinline__ int gt_off(int n, int ch) { return kOffQT + n * (kD * 2) + ((ch ^ (n & 15)) << 4); }

// One 32-token chunk c of one (b,h).
__global__ __launch_bounds__(256, 2)
void bwd_grad_kernel(P p) {
    __shared__ __attribute__((aligned(16))) char smem[kGradLDS];
    float *sDec = reinterpret_cast<float *>(smem + kOffDec);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, l32 = l & 31;
    const int ckb = (int)blockIdx.x;
    const int bh = uni(ckb / p.nck), c = uni(ckb % p.nck);
    size_t rowbase;
    int len;
    seq_rows(p.cu, p.H, p.total, p.T, bh, rowbase, len);
    const int t0 = c * kCk;
    if (t0 >= len) return;
    const int seg = c / p.seg_ck;
    const bool fixS = seg > 0, fixG = seg < p.nseg - 1;
    const size_t ck = (size_t)bh * p.nck + c, sb = (size_t)bh * p.nseg + seg;
    const int r = l & 15, cg = (w << 2) | (l >> 4);
    const int rr = 32 * w + l32;

    const __amdgpu_buffer_rsrc_t rq = rsrc(p.q + rowbase * kD, len), rk = rsrc(p.k + rowbase * kD, len);
    const __amdgpu_buffer_rsrc_t rv = rsrc(p.v + rowbase * kD, len), rg = rsrc(p.g + rowbase * kD, len);
    const __amdgpu_buffer_rsrc_t rth = rsrc(p.th + rowbase * kD, len), rdo = rsrc(p.dO + rowbase * kD, len);

    // this chunk's inputs (tokens past the end read 0)
    uint4 Rq[2], Rk[2], Rv[2], Rg[2], Rth[2], Rdo[2];
    load_one<2>(Rg, rg, t0, r, cg);
    load_one<2>(Rth, rth, t0, r, cg);
    load_one<2>(Rq, rq, t0, r, cg);
    load_one<2>(Rk, rk, t0, r, cg);
    load_one<2>(Rv, rv, t0, r, cg);
    load_one<2>(Rdo, rdo, t0, r, cg);
    // the chunk's two checkpoints (S entering, G leaving), in flight while the
    // gate map and the operand rows are built
    uint4 rS[8], rG[8];
    {
        const bf16_t *cS = p.ckS + ck * kFrag, *cG = p.ckG + ck * kFrag;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            rS[s] = ld_raw(cS, 8 * w + s, l);
            rG[s] = ld_raw(cG, 8 * w + s, l);
        }
    }

    // this chunk's gates; span check (Kh = k 2^{mu - Lam} must stay finite)
    uint32_t qTp[8], kTp[8];  // Qt^T / Kh^T rows of this lane's 8 channels, 2 tokens packed
    {
        float l2a[2][8], l2b[2][8], lend[8];
        gates_scan_gt<kSub>(Rg, Rth, t0, len, r, l, l2a, l2b, lend);
        bool bad = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) bad |= lend[e] < -kSpan2;
        if (__syncthreads_or(bad)) {
            if (tid == 0) {
                const int i = atomicAdd(p.bad, 1);
                p.bad[1 + i] = (int)ck;
            }
            return;
        }
        // token-row operands and dO^T
        float qT[8][2], kT[8][2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            float qf[8], kf[8], qt[8], kh[8], kb[8];
            unpack8(Rq[tt], qf);
            unpack8(Rk[tt], kf);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qt[e] = qf[e] * exp2_fast(l2a[tt][e]);
                kh[e] = kf[e] * exp2_fast(l2b[tt][e] - l2a[tt][e]);
                kb[e] = kf[e] * exp2_fast(l2b[tt][e] + lend[e] - l2a[tt][e]);
                qT[e][tt] = qt[e];
                kT[e][tt] = kh[e];
            }
            const int t = 2 * r + tt;
            store_q_row<kQR>(smem + kOffQr, t, cg, qt);
            store_q_row<kQR>(smem + kOffKr, t, cg, kh);
            store_q_row<kQR>(smem + kOffKbr, t, cg, kb);
            store_raw_row<kQR>(smem + kOffDOr, t, cg, Rdo[tt]);
            store_raw_row<kQR>(smem + kOffVr, t, cg, Rv[tt]);
        }
        store_vt<2, kT32>(smem + kOffDOT, cg, r, Rdo);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            qTp[e] = pack2(qT[e][0], qT[e][1]);
            kTp[e] = pack2(kT[e][0], kT[e][1]);
        }
    }
    // S entering and G leaving this chunk, bf16 operands: the checkpoints of
    // later / earlier segments completed with the segment fix-up
    bf16x8_t Sf[8], Gf[8], GTf[8];
    {
        uint4 fS[8], fG[8];
        const float sigS = fixS ? p.sigS[ck * kD + rr] : 0.f;
        const float sigG = fixG ? p.sigG[ck * kD + rr] : 0.f;
        if (fixS) {
#pragma unroll
            for (int s = 0; s < 8; ++s) fS[s] = ld_raw(p.fixS + sb * kFrag, 8 * w + s, l);
        }
        if (fixG) {
#pragma unroll
            for (int s = 0; s < 8; ++s) fG[s] = ld_raw(p.fixG + sb * kFrag, 8 * w + s, l);
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            Sf[s] = __builtin_bit_cast(bf16x8_t, fixS ? fix_raw(rS[s], fS[s], sigS) : rS[s]);
            Gf[s] = __builtin_bit_cast(bf16x8_t, fixG ? fix_raw(rG[s], fG[s], sigG) : rG[s]);
        }
    }
    // G's columns (G^T operands) through LDS, in two passes of 64 columns over
    // the Qt^T / Kh^T area (written only after the first product): each wave
    // turns its 32 rows into columns by an identity product per 32x32 block,
    // leaving column 32t + l32 of its rows (fragments 2w, 2w+1 of that column's
    // operand) in lane l32 of block t.
    {
        bf16x8_t Id[2];
        make_ident(Id, l32, h);
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            __syncthreads();  // pass 0: operand rows written; pass 1: pass 0 read
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const int t = 2 * pass + tb;
                f32x16_t cc = {};
                cc = mfma(Gf[2 * t], Id[0], cc);
                cc = mfma(Gf[2 * t + 1], Id[1], cc);
                const int n = 32 * tb + l32;
                *reinterpret_cast<bf16x8_t *>(smem + gt_off(n, 2 * (2 * w) + h)) = cvt8(cc, 0);
                *reinterpret_cast<bf16x8_t *>(smem + gt_off(n, 2 * (2 * w + 1) + h)) = cvt8(cc, 8);
            }
            __syncthreads();
            if ((w >> 1) == pass) {
#pragma unroll
                for (int s = 0; s < 8; ++s) GTf[s] = lds16(smem, gt_off(rr - 64 * pass, 2 * s + h));
            }
        }
    }

    auto rowf = [&](int off, int row, int s) { return lds16(smem, off + (row * kQR + 16 * s + 8 * h) * 2); };
    auto trf = [&](int off, int row, int ks) { return lds16(smem, off + (row * kT32 + 16 * ks + 8 * h) * 2); };

    // ---- matrix-core products (wave w: output columns 32w..32w+31) ----
    // dv = A^T dO + Kb G (rows j, column rr), straight to memory
    {
        f32x16_t acc = {};
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = mfma(rowf(kOffQr, l32, s), rowf(kOffKr, l32, s), acc);   // A[i][j]
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (l32 > 8 * (i >> 2) + 4 * h + (i & 3)) acc[i] = 0.f;
        const bf16x8_t opA0 = cvt8(acc, 0), opA1 = cvt8(acc, 8);
        f32x16_t av = {};
#pragma unroll
        for (int s = 0; s < 8; ++s) av = mfma(rowf(kOffKbr, l32, s), GTf[s], av);
        av = mfma(opA0, trf(kOffDOT, rr, 0), av);
        av = mfma(opA1, trf(kOffDOT, rr, 1), av);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = 8 * (i >> 2) + 4 * h + (i & 3);
            if (t0 + j < len) st_stream(&p.dv[(rowbase + t0 + j) * kD + rr], av[i]);
        }
    }
    __syncthreads();  // G's columns are read: Qt^T, Kh^T take their place
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        *reinterpret_cast<uint32_t *>(smem + kOffQT + ((8 * cg + e) * kT32 + perm16(2 * r)) * 2) = qTp[e];
        *reinterpret_cast<uint32_t *>(smem + kOffKT + ((8 * cg + e) * kT32 + perm16(2 * r)) * 2) = kTp[e];
    }
    // V G^T, and the decay term rowsum(G * S) of key channel rr
    f32x16_t ax = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) ax = mfma(rowf(kOffVr, l32, s), Gf[s], ax);
    float dec = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        float a8[8], b8[8];
        unpack_frag(Sf[s], a8);
        unpack_frag(Gf[s], b8);
#pragma unroll
        for (int e = 0; e < 8; ++e) dec = fmaf(a8[e], b8[e], dec);
    }
    dec += __shfl_xor(dec, 32);
    // dO S^T
    f32x16_t a1 = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) a1 = mfma(rowf(kOffDOr, l32, s), Sf[s], a1);
    // dP (rows i, columns j) and dP^T, masked to j <= i
    bf16x8_t opP[2], opPT[2];
    {
        f32x16_t acc = {};
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = mfma(rowf(kOffDOr, l32, s), rowf(kOffVr, l32, s), acc);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (l32 > 8 * (i >> 2) + 4 * h + (i & 3)) acc[i] = 0.f;
        opP[0] = cvt8(acc, 0); opP[1] = cvt8(acc, 8);
        acc = f32x16_t{};
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = mfma(rowf(kOffVr, l32, s), rowf(kOffDOr, l32, s), acc);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (8 * (i >> 2) + 4 * h + (i & 3) > l32) acc[i] = 0.f;
        opPT[0] = cvt8(acc, 0); opPT[1] = cvt8(acc, 8);
    }
    __syncthreads();  // Qt^T, Kh^T written
    // in-chunk parts: dP Kh and dP^T Qt
    f32x16_t aI = {}, kI = {};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        aI = mfma(opPT[ks], trf(kOffKT, rr, ks), aI);
        kI = mfma(opP[ks], trf(kOffQT, rr, ks), kI);
    }
    __syncthreads();  // operand rows are dead: stage the accumulators
    float *sQI = reinterpret_cast<float *>(smem), *sQ1 = sQI + kSub * kSR, *sKI = sQ1 + kSub * kSR,
          *sX2 = sKI + kSub * kSR;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = 8 * (i >> 2) + 4 * h + (i & 3);
        sQI[t * kSR + rr] = aI[i];
        sQ1[t * kSR + rr] = a1[i];
        sKI[t * kSR + rr] = kI[i];
        sX2[t * kSR + rr] = ax[i];
    }
    if (h == 0) sDec[rr] = dec;
    // the epilogue's g and tau again (L2-resident), once the accumulators are
    // free; q and k stay in the registers of the first load (kept through the
    // products: 16 VGPRs more, no spills, where also keeping g and tau spills)
    uint4 Eq[2], Ek[2], Eg[2], Eth[2];
    load_one<2>(Eg, rg, t0, r, cg);
    load_one<2>(Eth, rth, t0, r, cg);
    __syncthreads();

    // ---- epilogue, producer layout: tokens 2r, 2r+1, channels 8cg..8cg+7 ----
    // The in-chunk parts of dLam use the same bf16-rounded Qt, Kh as the
    // products, so that their reverse cumulative sum telescopes exactly.
    float l2a[2][8], l2b[2][8], lend[8];
    gates_scan_gt<kSub>(Eg, Eth, t0, len, r, l, l2a, l2b, lend);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        Eq[i] = Rq[i];
        Ek[i] = Rk[i];
    }
    float dlam[2][8], dmu[2][8], ebs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ebs[e] = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int t = 2 * r + tt;
        float qi[8], q1[8], ki[8], xa[8], qf[8], kf[8], dqv[8], dkv[8];
        const float *rows[4] = {sQI + t * kSR + 8 * cg, sQ1 + t * kSR + 8 * cg, sKI + t * kSR + 8 * cg,
                                sX2 + t * kSR + 8 * cg};
        float *dst[4] = {qi, q1, ki, xa};
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            *reinterpret_cast<float4 *>(dst[a]) = *reinterpret_cast<const float4 *>(rows[a]);
            *reinterpret_cast<float4 *>(dst[a] + 4) = *reinterpret_cast<const float4 *>(rows[a] + 4);
        }
        unpack8(Eq[tt], qf);
        unpack8(Ek[tt], kf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float eq = exp2_fast(l2a[tt][e]), ekh = exp2_fast(l2b[tt][e] - l2a[tt][e]);
            const float ekb = exp2_fast(l2b[tt][e] + lend[e] - l2a[tt][e]);
            const float qt = bf_round(qf[e] * eq), kh = bf_round(kf[e] * ekh);
            const float kbx = kf[e] * ekb * xa[e];
            dqv[e] = eq * (qi[e] + q1[e]);
            dkv[e] = fmaf(ekh, ki[e], ekb * xa[e]);
            dlam[tt][e] = fmaf(qt, qi[e], -kh * ki[e]) + fmaf(qf[e] * eq, q1[e], -kbx);
            dmu[tt][e] = kf[e] * dkv[e];
            ebs[e] += kbx;
        }
        if (t0 + t < len) {
            float *oq = p.dq + (rowbase + t0 + t) * kD + 8 * cg, *ok = p.dk + (rowbase + t0 + t) * kD + 8 * cg;
            st_stream(reinterpret_cast<float4 *>(oq), make_float4(dqv[0], dqv[1], dqv[2], dqv[3]));
            st_stream(reinterpret_cast<float4 *>(oq + 4), make_float4(dqv[4], dqv[5], dqv[6], dqv[7]));
            st_stream(reinterpret_cast<float4 *>(ok), make_float4(dkv[0], dkv[1], dkv[2], dkv[3]));
            st_stream(reinterpret_cast<float4 *>(ok + 4), make_float4(dkv[4], dkv[5], dkv[6], dkv[7]));
        }
        __builtin_amdgcn_sched_barrier(0);  // one token at a time (register pressure)
    }
    float dl[2][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float x = ebs[e];  // sum over the 16 lanes of the row: all 32 tokens
        x += row_shr<1>(x);
        x += row_shr<2>(x);
        x += row_shr<4>(x);
        x += row_shr<8>(x);
        const float dG = bcast_lane(x, (l & 48) | 15) + exp2_fast(lend[e]) * sDec[8 * cg + e];
        // reverse inclusive cumulative sum of dLam over the 32 tokens
        const float s1 = dlam[1][e], s0 = dlam[0][e] + s1;
        float y = s0;
        y += row_shl<1>(y);
        y += row_shl<2>(y);
        y += row_shl<4>(y);
        y += row_shl<8>(y);
        const float later = row_shl<1>(y);  // tokens of the lanes after this one
        dl[1][e] = s1 + later + dG;
        dl[0][e] = s0 + later + dG;
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int t = 2 * r + tt;
        if (t0 + t >= len) continue;
        float gf[8], tf[8], dgv[8], dtv[8];
        unpack8(Eg[tt], gf);
        unpack8(Eth[tt], tf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // recompute the gate exponentials here rather than keep the
            // epilogue's first ones alive (register pressure)
            asm volatile("" : "+v"(gf[e]), "+v"(tf[e]));
            ddts_gate_grads(gf[e], tf[e], dl[tt][e], dmu[tt][e], dgv[e], dtv[e]);
        }
        float *og = p.dg + (rowbase + t0 + t) * kD + 8 * cg, *ot = p.dth + (rowbase + t0 + t) * kD + 8 * cg;
        st_stream(reinterpret_cast<float4 *>(og), make_float4(dgv[0], dgv[1], dgv[2], dgv[3]));
        st_stream(reinterpret_cast<float4 *>(og + 4), make_float4(dgv[4], dgv[5], dgv[6], dgv[7]));
        st_stream(reinterpret_cast<float4 *>(ot), make_float4(dtv[0], dtv[1], dtv[2], dtv[3]));
        st_stream(reinterpret_cast<float4 *>(ot + 4), make_float4(dtv[4], dtv[5], dtv[6], dtv[7]));
    }
}

// --------------------------------------------------------------- fallback
// Listed chunks, exactly: S entering and G leaving the chunk (its checkpoints
// with the segment fix-ups) in fp32 (row-major, this workgroup's scratch slot),
// then the pairwise routine.
__global__ __launch_bounds__(256)
void bwd_fallback_kernel(P p) {
    __shared__ float smem[kBodyFloats];
    const int n_bad = p.bad[0];
    const int tid = threadIdx.x;
    float *Ss = p.slot + (size_t)blockIdx.x * 2 * kD * kD, *Gs = Ss + kD * kD;
    for (int i = blockIdx.x; i < n_bad; i += gridDim.x) {
        const int ent = p.bad[1 + i];
        const int bh = ent / p.nck, c = ent % p.nck;
        const int seg = c / p.seg_ck;
        const size_t ck = (size_t)ent, sb = (size_t)bh * p.nseg + seg;
        size_t rowbase;
        int len;
        seq_rows(p.cu, p.H, p.total, p.T, bh, rowbase, len);
        const int n = tid & 127;
        for (int rr = tid >> 7; rr < kD; rr += 2) {
            const int fi = frag_index(rr, n);
            float s = bf2f(p.ckS[ck * kFrag + fi]);
            if (seg > 0) s = fmaf(p.sigS[ck * kD + rr], bf2f(p.fixS[sb * kFrag + fi]), s);
            float gg = bf2f(p.ckG[ck * kFrag + fi]);
            if (seg < p.nseg - 1) gg = fmaf(p.sigG[ck * kD + rr], bf2f(p.fixG[sb * kFrag + fi]), gg);
            Ss[rr * kD + n] = s;
            Gs[rr * kD + n] = gg;
        }
        __syncthreads();
        chunk_grads_body<bf16_t>(p.q, p.k, p.v, p.g, p.th, p.dO, Ss, Gs, p.dq, p.dk, p.dv, p.dg, p.dth, rowbase,
                                 len, kD, kD, c, smem);
        __syncthreads();
    }
}

// --------------------------------------------------------------- planning
struct Plan {
    int nck, nseg, seg_ck;
    size_t o_ckS, o_ckG, o_sigS, o_sigG, o_segS, o_segG, o_segDS, o_segDG, o_fixS, o_fixG, o_bad, o_slot, bytes;
};

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

Plan plan(long long BH, int T) {
    Plan q{};
    q.nck = (T + kCk - 1) / kCk;
    // state passes: two roles x BH x nseg workgroups, about two per CU
    long long nseg = (kCUs + BH - 1) / BH;
    if (nseg > q.nck) nseg = q.nck;
    if (nseg < 1) nseg = 1;
    q.seg_ck = (int)((q.nck + nseg - 1) / nseg);
    q.nseg = (q.nck + q.seg_ck - 1) / q.seg_ck;
    const size_t F = (size_t)kFrag * 2, nck = (size_t)BH * q.nck, nsg = (size_t)BH * q.nseg;
    size_t o = 0;
    q.o_ckS = o; o += up256(nck * F);
    q.o_ckG = o; o += up256(nck * F);
    q.o_sigS = o; o += up256(nck * kD * 4);
    q.o_sigG = o; o += up256(nck * kD * 4);
    q.o_segS = o; o += up256(nsg * kD * kD * 4);
    q.o_segG = o; o += up256(nsg * kD * kD * 4);
    q.o_segDS = o; o += up256(nsg * kD * 4);
    q.o_segDG = o; o += up256(nsg * kD * 4);
    q.o_fixS = o; o += up256(nsg * F);
    q.o_fixG = o; o += up256(nsg * F);
    q.o_bad = o; o += up256((1 + nck) * 4);
    q.o_slot = o; o += (size_t)kSlowWG * 2 * kD * kD * 4;
    q.bytes = o;
    return q;
}

}  // namespace

bool scan_bwd_mfma_supported(int T, int dk, int dv, int dtype) {
    return dtype == 1 && dk == kD && dv == kD && T < kMaxT;
}

size_t scan_bwd_mfma_workspace(int B, int H, int T) {
    if (B <= 0 || H <= 0 || T <= 0) return 0;
    return plan((long long)B * H, T).bytes;
}

uint64_t scan_bwd_mfma_launch_items(long long BH, int T) {
    if (BH <= 0 || T <= 0) return 0;
    const Plan q = plan(BH, T);
    uint64_t m = (uint64_t)2 * BH * q.nseg * 256;                               // state passes
    if (q.nseg > 1) m = std::max<uint64_t>(m, (uint64_t)BH * (kFrag / 8));      // combine
    m = std::max<uint64_t>(m, (uint64_t)BH * q.nck * 256);                      // gradients
    return std::max<uint64_t>(m, (uint64_t)kSlowWG * 256);                      // fallback
}

void launch_scan_bwd_mfma(const ScanBwdArgs &a, hipStream_t st) {
    const int BH = a.B * a.H;
    const Plan q = plan(BH, a.T);
    char *ws = reinterpret_cast<char *>(a.workspace);
    P p;
    p.q = (const bf16_t *)a.q; p.k = (const bf16_t *)a.k; p.v = (const bf16_t *)a.v;
    p.g = (const bf16_t *)a.g; p.th = (const bf16_t *)a.tau; p.dO = (const bf16_t *)a.dO;
    p.S0 = a.S0; p.dST = a.dS_T;
    p.dq = a.dq; p.dk = a.dk_; p.dv = a.dv_; p.dg = a.dg; p.dth = a.dtau; p.dS0 = a.dS0;
    p.ckS = (bf16_t *)(ws + q.o_ckS); p.ckG = (bf16_t *)(ws + q.o_ckG);
    p.sigS = (float *)(ws + q.o_sigS); p.sigG = (float *)(ws + q.o_sigG);
    p.segS = (float *)(ws + q.o_segS); p.segG = (float *)(ws + q.o_segG);
    p.segDS = (float *)(ws + q.o_segDS); p.segDG = (float *)(ws + q.o_segDG);
    p.fixS = (bf16_t *)(ws + q.o_fixS); p.fixG = (bf16_t *)(ws + q.o_fixG);
    p.bad = (int *)(ws + q.o_bad);
    p.slot = (float *)(ws + q.o_slot);
    p.BH = BH; p.T = a.T; p.nck = q.nck; p.nseg = q.nseg; p.seg_ck = q.seg_ck;
    p.cu = a.cu; p.H = a.H; p.total = a.total;
    p.order = a.cu ? a.order : nullptr;
    hipLaunchKernelGGL(bwd_state_kernel, dim3((unsigned)(2 * BH * q.nseg)), dim3(256), 0, st, p);
    if (q.nseg > 1) {
        const size_t n = (size_t)BH * (kFrag / 8);
        hipLaunchKernelGGL(bwd_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
    }
    hipLaunchKernelGGL(bwd_grad_kernel, dim3((unsigned)((size_t)BH * q.nck)), dim3(256), 0, st, p);
    hipLaunchKernelGGL(bwd_fallback_kernel, dim3(kSlowWG), dim3(256), 0, st, p);
}

}  // namespace rodimus
