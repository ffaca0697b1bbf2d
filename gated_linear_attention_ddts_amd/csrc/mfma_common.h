// mfma_common.h -- building blocks shared by the gfx950 matrix-core scan
// kernels (forward prefill and backward): bf16 packing, DPP row scans, the
// v_mfma_f32_32x32x16_bf16 wrapper, buffer loads with scalar descriptors, the
// producer-lane input layout and the in-chunk gate scan, and the LDS stores
// that lay operands out for 16-byte fragment reads.
//
// MFMA v_mfma_f32_32x32x16_bf16: operand A[m][k] sits in lane m + 32*(k/8),
// element k%8; B[k][n] in lane n + 32*(k/8), element k%8; the accumulator
// C[m][n] in lane n + 32*((m/4)%2), register 4*(m/8) + m%4.  Eight
// accumulator registers [8j, 8j+8) of a lane therefore hold, for lane half h,
// the rows {16j+4h..16j+4h+3, 16j+8+4h..16j+8+4h+3}; used as an operand they
// contract k in that order.  LDS rows that feed the other operand store their
// k index in the matching order (blocks of 4 placed 0,2,1,3 inside each 16,
// perm16 below), so that every fragment read is one 16-byte ds_read.
#pragma once
#include "device_common.h"

namespace rodimus {

constexpr int kD = 128;            // dk = dv on the matrix-core paths
constexpr float kSpan2 = 112.f;    // 2^112 ~ 5e33: k * 2^{-Lam} stays finite in fp32/bf16

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    f32x2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ float lo_bf(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ void unpack8(const uint4 &x, float *f) {
    f[0] = lo_bf(x.x); f[1] = hi_bf(x.x); f[2] = lo_bf(x.y); f[3] = hi_bf(x.y);
    f[4] = lo_bf(x.z); f[5] = hi_bf(x.z); f[6] = lo_bf(x.w); f[7] = hi_bf(x.w);
}

template <int K>
__device__ __forceinline__ float row_shr(float x) {  // lane i <- lane i-K inside 16-lane rows, else 0
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x110 + K, 0xf, 0xf, false));
}
template <int K>
__device__ __forceinline__ float row_shl(float x) {  // lane i <- lane i+K inside 16-lane rows, else 0
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x100 + K, 0xf, 0xf, false));
}
__device__ __forceinline__ float bcast_lane(float x, int src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}
__device__ __forceinline__ f32x16_t mfma(const bf16x8_t &a, const bf16x8_t &b, const f32x16_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8_t lds16(const char *base, int byte_off) {
    return *reinterpret_cast<const bf16x8_t *>(base + byte_off);
}
// 8 accumulator registers [base, base+8) as a bf16 operand
__device__ __forceinline__ bf16x8_t cvt8(const f32x16_t &s, int base) {
    uint4 u = make_uint4(pack2(s[base + 0], s[base + 1]), pack2(s[base + 2], s[base + 3]),
                         pack2(s[base + 4], s[base + 5]), pack2(s[base + 6], s[base + 7]));
    return __builtin_bit_cast(bf16x8_t, u);
}
// 8 bf16 of a fragment as floats
__device__ __forceinline__ void unpack_frag(const bf16x8_t &x, float *f) {
    unpack8(__builtin_bit_cast(uint4, x), f);
}
// Position of index x in the permuted order (blocks of 4 placed 0,2,1,3 in each 16).
__device__ __forceinline__ int perm16(int x) {
    const int blk = (x >> 2) & 3;
    return (x & ~15) | (((blk & 1) << 1 | (blk >> 1)) << 2) | (x & 3);
}

// Workgroup-uniform values computed with integer division end up in vector
// registers; readfirstlane moves them to scalar registers so that buffer
// descriptors are scalar (no per-lane waterfall loops).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ const bf16_t *uni_ptr(const bf16_t *p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return reinterpret_cast<const bf16_t *>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const bf16_t *base, int T) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)uni_ptr(base), (short)0, uni(T * kD * 2), 0x00020000);
}
// Byte offsets are unsigned 32-bit: rows up to T + 63 (a ragged last chunk)
// times 256 bytes stay below 2^32 for T < kMaxT, and rows at or past T read
// zeros (buffer bounds).
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// ------------------------------------------------------------------ producer
// Producer lane (256 of them): channel group cg (channels 8cg..8cg+7) and
// token group r (tokens TPR*r .. TPR*r+TPR-1).  In the 16-row layout the 16
// lanes of a DPP row share cg and together cover the C tokens of the chunk;
// in the by-halves layout (chunk_scan_half) lanes 8 apart take consecutive
// token groups of one half and the 8 lanes of a block one 128-byte piece of a
// row.  The loaders below take any (r, cg).
// LR: the gate inputs come separately (Zops); g and th are then unused.
template <int C, bool WITH_Q, bool LR = false>
struct Raw {
    static constexpr int TPR = C / 16, NG = LR ? 1 : TPR;
    uint4 q[WITH_Q ? TPR : 1], k[TPR], g[NG], th[NG], v[TPR];
};

struct Rsrc {
    __amdgpu_buffer_rsrc_t q, k, v, g, th;
};

// Rank of the low-rank gate factors, and the bytes of one factor row.
constexpr int kRank = 16;
constexpr uint32_t kZRow = kRank * 2;

// Descriptor over `bytes` bytes (reads past the end return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_bytes(const bf16_t *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)uni_ptr(base), (short)0, uni(bytes), 0x00020000);
}

// Loads past T read zeros (buffer bounds).
template <int C, bool WITH_Q, bool LR>
__device__ __forceinline__ void load_raw(Raw<C, WITH_Q, LR> &R, const Rsrc &rs, int t0, int r, int cg) {
    constexpr int TPR = C / 16;
#pragma unroll
    for (int tt = 0; tt < TPR; ++tt) {
        const uint32_t off = (uint32_t)(t0 + TPR * r + tt) * (kD * 2u) + 16u * cg;
        if (WITH_Q) R.q[tt] = bload(rs.q, off);
        R.k[tt] = bload(rs.k, off);
        if (!LR) {
            R.g[tt] = bload(rs.g, off);
            R.th[tt] = bload(rs.th, off);
        }
        R.v[tt] = bload(rs.v, off);
    }
}

// Next chunk's gate-logit rows.
template <int C, bool WITH_Q, bool LR>
__device__ __forceinline__ void load_gates(Raw<C, WITH_Q, LR> &R, const Rsrc &rs, int t0, int r, int cg) {
    constexpr int TPR = C / 16;
#pragma unroll
    for (int tt = 0; tt < TPR; ++tt) {
        const uint32_t off = (uint32_t)(t0 + TPR * r + tt) * (kD * 2u) + 16u * cg;
        R.g[tt] = bload(rs.g, off);
        R.th[tt] = bload(rs.th, off);
    }
}

// One tensor's TPR vectors of chunk t0 (for prefetching each tensor right
// after the last use of its registers).
template <int TPR>
__device__ __forceinline__ void load_one(uint4 (&x)[TPR], __amdgpu_buffer_rsrc_t rs, int t0, int r, int cg) {
#pragma unroll
    for (int tt = 0; tt < TPR; ++tt) x[tt] = bload(rs, (uint32_t)(t0 + TPR * r + tt) * (kD * 2u) + 16u * cg);
}

// ------------------------------------------------- low-rank gate factors
// The gate logits of a chunk from rank-16 factor rows on the matrix cores.
// Producer wave w owns key channels 32w..32w+31; per 32-token tile and gate,
//     G[t][c] = silu(Z_g[t][:]) . U_g[c][:] + b_g[c]       (tau: no silu)
// is one v_mfma_f32_32x32x16_bf16 with A = the tile's factor rows (lane
// m + 32*(k/8): token m, ranks 8(k/8)..+7, one 16-byte load), B = U^T (lane
// n + 32*(k/8): channel 32w+n, same ranks, held for the whole kernel) and the
// accumulator initialised with the bias (one value per lane: channel n).  The
// wave writes the bf16 logits into its own 32 channel rows of an LDS area
// laid out [channel][token] (rows of ROW bf16), then each lane reads back its
// channels and tokens in the producer layout.
struct LrOps {
    bf16x8_t ug, ut;    // B operands
    float bg, bt;       // biases of channel 32w + (lane & 31)
};

__device__ __forceinline__ void lr_load_ops(LrOps &o, const bf16_t *Ug, const float *bg, const bf16_t *Ut,
                                            const float *bt, int h, int w, int l) {
    const size_t c = (size_t)h * kD + 32 * w + (l & 31);
    o.ug = *reinterpret_cast<const bf16x8_t *>(Ug + c * kRank + 8 * (l >> 5));
    o.ut = *reinterpret_cast<const bf16x8_t *>(Ut + c * kRank + 8 * (l >> 5));
    o.bg = bg[c];
    o.bt = bt[c];
}

// A-operand factor rows of NTL 32-token tiles starting at token t0 (rows past
// the descriptor's end read zeros).
template <int NTL>
struct Zops {
    uint4 g[NTL], t[NTL];
};

template <int NTL>
__device__ __forceinline__ void load_zops(Zops<NTL> &z, __amdgpu_buffer_rsrc_t rg, __amdgpu_buffer_rsrc_t rt, int t0,
                                          int l) {
#pragma unroll
    for (int tl = 0; tl < NTL; ++tl) {
        const uint32_t off = (uint32_t)(t0 + 32 * tl + (l & 31)) * kZRow + 16u * (l >> 5);
        z.g[tl] = bload(rg, off);
        z.t[tl] = bload(rt, off);
    }
}

__device__ __forceinline__ float silu(float x) {
    return x * __builtin_amdgcn_rcpf(1.f + exp2_fast(-x * kLog2e));
}

// silu of 8 bf16 values, rounded back to bf16 (the operand precision).
__device__ __forceinline__ bf16x8_t silu8(const uint4 &x) {
    float f[8];
    unpack8(x, f);
    const uint4 u = make_uint4(pack2(silu(f[0]), silu(f[1])), pack2(silu(f[2]), silu(f[3])),
                               pack2(silu(f[4]), silu(f[5])), pack2(silu(f[6]), silu(f[7])));
    return __builtin_bit_cast(bf16x8_t, u);
}

// Logits of the NTL tiles into the wave's rows 32w..32w+31 of sg (g) and st
// (tau), token columns 0..32*NTL-1.
template <int NTL, int ROW>
__device__ __forceinline__ void lr_stage(const Zops<NTL> &z, const LrOps &o, char *sg, char *st, int w, int l) {
    const int n = l & 31, hh = l >> 5;
#pragma unroll
    for (int tl = 0; tl < NTL; ++tl) {
#pragma unroll
        for (int gate = 0; gate < 2; ++gate) {
            const float b = gate ? o.bt : o.bg;
            f32x16_t acc;
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = b;
            const bf16x8_t a = gate ? __builtin_bit_cast(bf16x8_t, z.t[tl]) : silu8(z.g[tl]);
            acc = mfma(a, gate ? o.ut : o.ug, acc);
            char *row = (gate ? st : sg) + ((32 * w + n) * ROW + 32 * tl + 4 * hh) * 2;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<uint2 *>(row + 16 * j) =
                    make_uint2(pack2(acc[4 * j], acc[4 * j + 1]), pack2(acc[4 * j + 2], acc[4 * j + 3]));
        }
    }
}

// Producer lane (r, cg): the staged logits of its channels 8cg..8cg+7 and
// tokens TPR*r.., as TPR/2 words (two tokens each) per channel.
template <int TPR, int ROW>
__device__ __forceinline__ void lr_read(const char *sg, const char *st, int r, int cg,
                                        uint32_t (&gw)[8][TPR / 2], uint32_t (&tw)[8][TPR / 2]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int off = ((8 * cg + e) * ROW + TPR * r) * 2;
        if constexpr (TPR == 4) {
            const uint2 a = *reinterpret_cast<const uint2 *>(sg + off), b = *reinterpret_cast<const uint2 *>(st + off);
            gw[e][0] = a.x; gw[e][1] = a.y; tw[e][0] = b.x; tw[e][1] = b.y;
        } else {
            gw[e][0] = *reinterpret_cast<const uint32_t *>(sg + off);
            tw[e][0] = *reinterpret_cast<const uint32_t *>(st + off);
        }
    }
}

// In-chunk inclusive scan of log2 a (l2a on entry): on return l2a holds Lam
// (inclusive cumulative log2 a), lend the chunk total Lam[C-1] of each of the
// lane's 8 channels.  Tokens at or beyond tend get a = 1, beta = 0.
template <int C>
__device__ __forceinline__ void chunk_scan(int t0, int tend, int r, int l, float (&l2a)[C / 16][8],
                                           float (&l2b)[C / 16][8], float (&lend)[8]) {
    constexpr int TPR = C / 16;
    if (t0 + C > tend) {  // ragged last chunk
#pragma unroll
        for (int tt = 0; tt < TPR; ++tt)
            if (t0 + TPR * r + tt >= tend) {
#pragma unroll
                for (int e = 0; e < 8; ++e) { l2a[tt][e] = 0.f; l2b[tt][e] = -INFINITY; }
            }
    }
#pragma unroll
    for (int tt = 1; tt < TPR; ++tt)
#pragma unroll
        for (int e = 0; e < 8; ++e) l2a[tt][e] += l2a[tt - 1][e];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float x = l2a[TPR - 1][e];
        x += row_shr<1>(x);
        x += row_shr<2>(x);
        x += row_shr<4>(x);
        x += row_shr<8>(x);
        const float excl = row_shr<1>(x);
        lend[e] = bcast_lane(x, (l & 48) | 15);
#pragma unroll
        for (int tt = 0; tt < TPR; ++tt) l2a[tt][e] += excl;
    }
}

// gfx950's row swaps with one value in both operands.  v_permlane16_swap
// exchanges the odd 16-lane rows of one operand with the even rows of the
// other, v_permlane32_swap the upper 32 lanes of one with the lower 32 of the
// other: every lane receives x at its own position in rows (row & 2) and
// (row & 2) + 1, or in lanes l mod 32 and 32 + l mod 32.

__device__ __forceinline__ void row_pair16(float x, float &even, float &odd) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    even = __uint_as_float(p[0]);
    odd = __uint_as_float(p[1]);
}
__device__ __forceinline__ void row_pair32(float x, float &lo, float &hi) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    lo = __uint_as_float(p[0]);
    hi = __uint_as_float(p[1]);
}

// In-chunk scan for the producer layout by halves of a 64-token chunk: wave
// pair w >> 1 holds one 32-token half, lane block i = l >> 3 its tokens
// 4i .. 4i+3 of the half (lanes 8 apart), lane l & 7 a channel group, so that
// each load instruction reads 128 contiguous bytes of 8 token rows.  Each
// half is scanned from its own first token (the exponent reference of its
// products): on return l2a holds Lam from the half's first token (inclusive),
// l2b log2 beta, htot the half's total, per channel.  Blocks 2k, 2k+1 share a
// 16-lane row: their prefix comes from a row shift by 8, the rows' totals from
// the two row swaps.  Tokens at or beyond tend get a = 1, beta = 0.
template <int C>
__device__ __forceinline__ void chunk_scan_half(int t0, int tend, int r, int l, float (&l2a)[C / 16][8],
                                                float (&l2b)[C / 16][8], float (&htot)[8]) {
    static_assert(C == 64, "halves of 64-token chunks");
    constexpr int TPR = C / 16;
    if (t0 + C > tend) {  // ragged last chunk
#pragma unroll
        for (int tt = 0; tt < TPR; ++tt)
            if (t0 + TPR * r + tt >= tend) {
#pragma unroll
                for (int e = 0; e < 8; ++e) { l2a[tt][e] = 0.f; l2b[tt][e] = -INFINITY; }
            }
    }
#pragma unroll
    for (int tt = 1; tt < TPR; ++tt)
#pragma unroll
        for (int e = 0; e < 8; ++e) l2a[tt][e] += l2a[tt - 1][e];
    const int row = l >> 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        // Every cross-lane read here feeds arithmetic that all lanes run: a
        // read whose only use is one arm of a lane-dependent select can be
        // moved under a branch, where the lanes it reads from are switched
        // off and yield 0.  The two shifts fill 0 across the row's edge, so
        // both blocks of a row get the same sum, added in the same order.
        const float x = l2a[TPR - 1][e];  // this block's total
        const float t = row_shr<8>(x);    // the even block's, in the odd block; 0 in the even one
        const float u = row_shl<8>(x);    // the odd block's, in the even block; 0 in the odd one
        const float rt = (x + t) + u;     // the row's two blocks
        float re, ro, plo, phi;
        row_pair16(rt, re, ro);
        row_pair32(re + ro, plo, phi);
        const float excl = ((row & 1) ? re : 0.f) + ((row & 2) ? plo : 0.f) + t;
        htot[e] = plo + phi;
#pragma unroll
        for (int tt = 0; tt < TPR; ++tt) l2a[tt][e] += excl;
    }
}

template <int C>
__device__ __forceinline__ void gates_scan_half(const uint4 (&G)[C / 16], const uint4 (&TH)[C / 16], int t0,
                                                int tend, int r, int l, float (&l2a)[C / 16][8],
                                                float (&l2b)[C / 16][8], float (&htot)[8]) {
    constexpr int TPR = C / 16;
#pragma unroll
    for (int tt = 0; tt < TPR; ++tt) {
        float gf[8], tf[8];
        unpack8(G[tt], gf);
        unpack8(TH[tt], tf);
#pragma unroll
        for (int e = 0; e < 8; ++e) ddts_log2_gates_fast(gf[e], tf[e], l2a[tt][e], l2b[tt][e]);
    }
    chunk_scan_half<C>(t0, tend, r, l, l2a, l2b, htot);
}

// Gates and in-chunk inclusive scan: on return l2a holds Lam (inclusive
// cumulative log2 a), l2b log2 beta, lend the chunk total Lam[C-1] of each of
// the lane's 8 channels.  Tokens at or beyond tend get a = 1, beta = 0.
template <int C>
__device__ __forceinline__ void gates_scan_gt(const uint4 (&G)[C / 16], const uint4 (&TH)[C / 16], int t0,
                                              int tend, int r, int l, float (&l2a)[C / 16][8],
                                              float (&l2b)[C / 16][8], float (&lend)[8]) {
    constexpr int TPR = C / 16;
#pragma unroll
    for (int tt = 0; tt < TPR; ++tt) {
        float gf[8], tf[8];
        unpack8(G[tt], gf);
        unpack8(TH[tt], tf);
#pragma unroll
        for (int e = 0; e < 8; ++e) ddts_log2_gates_fast(gf[e], tf[e], l2a[tt][e], l2b[tt][e]);
    }
    chunk_scan<C>(t0, tend, r, l, l2a, l2b, lend);
}

// The same from logits staged per channel (lr_read's words).
template <int C>
__device__ __forceinline__ void gates_scan_cols(const uint32_t (&gw)[8][C / 32], const uint32_t (&tw)[8][C / 32],
                                                int t0, int tend, int r, int l, float (&l2a)[C / 16][8],
                                                float (&l2b)[C / 16][8], float (&lend)[8]) {
    constexpr int TPR = C / 16;
#pragma unroll
    for (int tt = 0; tt < TPR; ++tt)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t gu = gw[e][tt >> 1], tu = tw[e][tt >> 1];
            const float gv = (tt & 1) ? hi_bf(gu) : lo_bf(gu), tv = (tt & 1) ? hi_bf(tu) : lo_bf(tu);
            ddts_log2_gates_fast(gv, tv, l2a[tt][e], l2b[tt][e]);
        }
    chunk_scan<C>(t0, tend, r, l, l2a, l2b, lend);
}

// Row c of Kb^T / V^T: tokens TPR*r .. TPR*r+TPR-1 at their permuted position.
template <int TPR, int ROW>
__device__ __forceinline__ void store_t_rows(char *base, int c, int r, const float *x) {
    char *p = base + (c * ROW + perm16(TPR * r)) * 2;
    if (TPR == 4) *reinterpret_cast<uint2 *>(p) = make_uint2(pack2(x[0], x[1 % TPR]), pack2(x[2 % TPR], x[3 % TPR]));
    else *reinterpret_cast<uint32_t *>(p) = pack2(x[0], x[1 % TPR]);
}
// V^T rows 8cg..8cg+7 straight from the raw bf16 registers (no conversion).
template <int TPR, int ROW>
__device__ __forceinline__ void store_vt(char *base, int cg, int r, const uint4 (&v)[TPR]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t w[TPR];
#pragma unroll
        for (int tt = 0; tt < TPR; ++tt) {
            const uint32_t word = (e < 2) ? v[tt].x : (e < 4) ? v[tt].y : (e < 6) ? v[tt].z : v[tt].w;
            w[tt] = (e & 1) ? (word >> 16) : (word & 0xffffu);
        }
        char *p = base + ((8 * cg + e) * ROW + perm16(TPR * r)) * 2;
        if (TPR == 4) *reinterpret_cast<uint2 *>(p) = make_uint2(w[0] | (w[1 % TPR] << 16), w[2 % TPR] | (w[3 % TPR] << 16));
        else *reinterpret_cast<uint32_t *>(p) = w[0] | (w[1 % TPR] << 16);
    }
}

// Channels 8cg..8cg+7 of token row t of Qt / Kh at their permuted positions.
template <int ROW>
__device__ __forceinline__ void store_q_row(char *base, int t, int cg, const float *x) {
    char *p = base + (t * ROW) * 2;
    *reinterpret_cast<uint2 *>(p + perm16(8 * cg) * 2) = make_uint2(pack2(x[0], x[1]), pack2(x[2], x[3]));
    *reinterpret_cast<uint2 *>(p + perm16(8 * cg + 4) * 2) = make_uint2(pack2(x[4], x[5]), pack2(x[6], x[7]));
}

// Channels 8cg..8cg+7 of token row t, raw bf16 (no conversion), at their
// permuted positions.
template <int ROW>
__device__ __forceinline__ void store_raw_row(char *base, int t, int cg, const uint4 &x) {
    char *p = base + (t * ROW) * 2;
    *reinterpret_cast<uint2 *>(p + perm16(8 * cg) * 2) = make_uint2(x.x, x.y);
    *reinterpret_cast<uint2 *>(p + perm16(8 * cg + 4) * 2) = make_uint2(x.z, x.w);
}

// Fragment order of a 128x128 matrix X: fragment f = 8*(row/32) + col/16 holds,
// in lane (row%32) + 32*kb, the 8 elements X[row][col] whose col%16 sits at
// permuted positions 8kb..8kb+7.  Fragment 8w+s is then exactly the B operand
// (k = col) that wave w needs for output columns row in 32w..32w+31 and
// k-step s, and also what eight accumulator registers of a transposed 32-row
// tile hold.  Element index of X[row][col]:
__device__ __forceinline__ int frag_index(int row, int col) {
    const int pc = perm16(col & 15);
    const int f = 8 * (row >> 5) + (col >> 4);
    return (f * 64 + (row & 31) + 32 * (pc >> 3)) * 8 + (pc & 7);
}

}  // namespace rodimus
