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
// token group r (tokens TPR*r .. TPR*r+TPR-1); the 16 lanes of a DPP row
// share cg and together cover the C tokens of the chunk.
template <int C, bool WITH_Q>
struct Raw {
    static constexpr int TPR = C / 16;
    uint4 q[WITH_Q ? TPR : 1], k[TPR], g[TPR], th[TPR], v[TPR];
};

struct Rsrc {
    __amdgpu_buffer_rsrc_t q, k, v, g, th;
};

// Loads past T read zeros (buffer bounds).
template <int C, bool WITH_Q>
__device__ __forceinline__ void load_raw(Raw<C, WITH_Q> &R, const Rsrc &rs, int t0, int r, int cg) {
    constexpr int TPR = C / 16;
#pragma unroll
    for (int tt = 0; tt < TPR; ++tt) {
        const uint32_t off = (uint32_t)(t0 + TPR * r + tt) * (kD * 2u) + 16u * cg;
        if (WITH_Q) R.q[tt] = bload(rs.q, off);
        R.k[tt] = bload(rs.k, off);
        R.g[tt] = bload(rs.g, off);
        R.th[tt] = bload(rs.th, off);
        R.v[tt] = bload(rs.v, off);
    }
}

// One tensor's TPR vectors of chunk t0 (for prefetching each tensor right
// after the last use of its registers).
template <int TPR>
__device__ __forceinline__ void load_one(uint4 (&x)[TPR], __amdgpu_buffer_rsrc_t rs, int t0, int r, int cg) {
#pragma unroll
    for (int tt = 0; tt < TPR; ++tt) x[tt] = bload(rs, (uint32_t)(t0 + TPR * r + tt) * (kD * 2u) + 16u * cg);
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

template <int C, bool WITH_Q>
__device__ __forceinline__ void gates_scan(const Raw<C, WITH_Q> &R, int t0, int tend, int r, int l,
                                           float (&l2a)[C / 16][8], float (&l2b)[C / 16][8],
                                           float (&lend)[8]) {
    gates_scan_gt<C>(R.g, R.th, t0, tend, r, l, l2a, l2b, lend);
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
