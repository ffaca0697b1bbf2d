// swska.hip -- sliding-window shared-key attention (SW-SKA) on gfx950.
//
//   o[b,h,t] = sum_{s = max(0, t-w+1)}^{t} softmax_s(scale * q[b,h,t] . k[b,s]) v[b,h,s]
//
// One key matrix is shared by all heads while every head keeps its own values
// (SKA, "ICLR 2025 | Rodimus*: ..." (CodeFuse), SKA / Rodimus+ paragraphs and
// Fig. 4), inside sliding-window attention where each query sees the previous
// w keys including itself (MiniCPM-SALA blog, sections 1.1 and 2.1).
//
// Kernel: one workgroup = 32 NW consecutive queries of one (b, h); NW waves,
// 32 queries each (NW = 8 at d = 128, one workgroup per CU; NW = 4 at d = 64,
// two per CU).  Keys/values stream through LDS in tiles of 64, three buffers
// deep: while tile j is consumed, tile j+1's scores are computed and tile j+2
// is written from registers (tile j+3 in flight), so each staged tile serves
// 32 NW queries.  Per tile and wave, on v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T       keys on the M dimension, queries on lanes, so each lane
//                     owns one query's scores and the softmax reductions stay
//                     inside the lane (plus one exchange with lane^32);
//   online softmax    fp32, base 2, scale folded into one FMA; the output is
//                     rescaled only when a lane's running max grows by more than
//                     2^8 (exact: the final division uses the same reference);
//   O^T += V^T P^T    P^T taken straight from the S^T accumulators (bf16) with a
//                     permuted k order; V^T is stored in LDS in that key order,
//                     so each operand is one 16-byte read.
// The next tile's S^T products are issued inside the same straight-line code
// as this tile's max and exponentials, so that matrix and vector instructions
// of one wave overlap.
// Tiles entirely outside a wave's window are skipped; tiles on the window's two
// edges are masked element by element.  Workgroups are mapped so that each XCD
// works on a fixed pair of heads in increasing query order, which keeps the
// shared K and the per-head V of overlapping windows in that XCD's L2.
#include "device_common.h"
#include "launch.h"

namespace rodimus {

namespace {

constexpr int kBK = 64;
constexpr float kRescale = 8.f;  // log2 of the largest p before the output is rescaled

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    f32x2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ f32x16_t mfma(const bf16x8_t &a, const bf16x8_t &b, const f32x16_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Position of key index x inside V^T rows: blocks of 4 keys placed 0,2,1,3 in
// each 16, the k order in which the S^T accumulators hold the keys.
__device__ __forceinline__ int perm16(int x) {
    const int blk = (x >> 2) & 3;
    return (x & ~15) | (((blk & 1) << 1 | (blk >> 1)) << 2) | (x & 3);
}

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ const bf16_t *uni_ptr(const bf16_t *p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return reinterpret_cast<const bf16_t *>(((uint64_t)hi << 32) | lo);
}
// Buffer descriptor over rows [0, T) of a [T][D] bf16 matrix; reads past the
// end return zeros.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const bf16_t *base, int T) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)uni_ptr(base), (short)0, uni(T * D * 2), 0x00020000);
}
// Byte offsets are unsigned 32-bit: key rows up to T + 63 times D * 2 bytes stay
// below 2^32 whenever T * D * 2 < 2^31 (the supported range).
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

template <int D, int NT = 256>
struct Tile {
    static constexpr int KROW = D + 8;        // bf16 per K row in LDS
    static constexpr int VROW = kBK + 8;      // bf16 per V^T row in LDS
    static constexpr int KBYTES = kBK * KROW * 2;
    static constexpr int VBYTES = D * VROW * 2;
    static constexpr int BYTES = KBYTES + VBYTES;
    static constexpr int KVEC = kBK * D / 8 / NT;   // 16-byte K vectors per thread
    static constexpr int KPT = 8 * D / NT;          // keys per thread in the V transpose
};

template <int D, int NT>
__device__ __forceinline__ void fetch_tile(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int k0,
                                           uint4 (&rk)[Tile<D, NT>::KVEC], uint4 (&rv)[Tile<D, NT>::KPT]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < Tile<D, NT>::KVEC; ++i) {
        const int vi = tid + NT * i, row = vi / (D / 8), col = vi % (D / 8);
        rk[i] = bload(kr, (uint32_t)(k0 + row) * (D * 2u) + 16u * col);
    }
    constexpr int KPT = Tile<D, NT>::KPT;
    const int kg = tid % (kBK / KPT), dg = tid / (kBK / KPT);
#pragma unroll
    for (int i = 0; i < KPT; ++i) rv[i] = bload(vr, (uint32_t)(k0 + KPT * kg + i) * (D * 2u) + 16u * dg);
}

template <int D, int NT>
__device__ __forceinline__ void store_tile(char *buf, const uint4 (&rk)[Tile<D, NT>::KVEC],
                                           const uint4 (&rv)[Tile<D, NT>::KPT]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < Tile<D, NT>::KVEC; ++i) {
        const int vi = tid + NT * i, row = vi / (D / 8), col = vi % (D / 8);
        *reinterpret_cast<uint4 *>(buf + (row * Tile<D, NT>::KROW + 8 * col) * 2) = rk[i];
    }
    // V^T: row = value channel, KPT consecutive keys per write
    constexpr int KPT = Tile<D, NT>::KPT;
    const int kg = tid % (kBK / KPT), dg = tid / (kBK / KPT);
    char *vt = buf + Tile<D, NT>::KBYTES;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        // element e of keys 2i and 2i+1 -> one word (v_perm: the low or the high
        // halves of the two source words)
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[KPT / 2];
#pragma unroll
        for (int i = 0; i < KPT / 2; ++i) {
            const uint4 &a = rv[2 * i], &c = rv[2 * i + 1];
            const uint32_t wa = (e < 2) ? a.x : (e < 4) ? a.y : (e < 6) ? a.z : a.w;
            const uint32_t wc = (e < 2) ? c.x : (e < 4) ? c.y : (e < 6) ? c.z : c.w;
            w[i] = __builtin_amdgcn_perm(wc, wa, sel);
        }
        const int off = ((8 * dg + e) * Tile<D, NT>::VROW + perm16(KPT * kg)) * 2;
        if (KPT == 4) *reinterpret_cast<uint2 *>(vt + off) = make_uint2(w[0], w[1 % (KPT / 2)]);
        else *reinterpret_cast<uint32_t *>(vt + off) = w[0];
    }
}

// S^T tile (64 keys x this wave's 32 queries) of the K tile staged at buf
template <int D, int NT>
__device__ __forceinline__ void qk_tile(const char *buf, const bf16x8_t (&qB)[D / 16], f32x16_t (&S)[2], int l32,
                                        int h) {
    using TL = Tile<D, NT>;
    S[0] = f32x16_t{};
    S[1] = f32x16_t{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(buf + ((32 * mt + l32) * TL::KROW + 16 * s + 8 * h) * 2);
            S[mt] = mfma(a, qB[s], S[mt]);
        }
}

// Online softmax of one S^T tile and O^T += V^T P^T with the V^T tile at buf.
// With NEXT, the scores of the following tile (K tile at nbuf, into Sn) are
// issued on the matrix cores inside the same straight-line blocks as the max
// and the exponentials, so the two kinds of work overlap within the wave.
template <int D, int NT, bool NEXT>
__device__ __forceinline__ void softmax_pv(const char *buf, f32x16_t (&S)[2], f32x16_t (&O)[D / 32], float &m,
                                           float &lsum, bool edge, int k0, int qi, int window, int T,
                                           float scale_log2e, int l32, int h, const char *nbuf,
                                           const bf16x8_t (&qB)[D / 16], f32x16_t (&Sn)[2]) {
    using TL = Tile<D, NT>;
    auto qk_part = [&](int s0, int s1) {
#pragma unroll
        for (int s = s0; s < s1; ++s)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const bf16x8_t a =
                    *reinterpret_cast<const bf16x8_t *>(nbuf + ((32 * mt + l32) * TL::KROW + 16 * s + 8 * h) * 2);
                Sn[mt] = mfma(a, qB[s], Sn[mt]);
            }
    };
    if constexpr (NEXT) {
        Sn[0] = f32x16_t{};
        Sn[1] = f32x16_t{};
    }
    if (edge) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = k0 + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
                const bool ok = key <= qi && key > qi - window && key < T;
                S[mt][i] = ok ? S[mt][i] : -INFINITY;
            }
    }
    if constexpr (NEXT) qk_part(0, D / 32);
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[mt][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = mx * scale_log2e;   // scale > 0 keeps the order
    const bool grow = mnew > m + kRescale;
    if (__any(grow)) {
        const float corr = grow ? exp2_fast(m - mnew) : 1.f;  // m = -inf -> 0
        if (grow) m = mnew;
        lsum *= corr;
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) O[mt][i] *= corr;
    }
    const float mref = (m == -INFINITY) ? 0.f : m;
    if constexpr (NEXT) qk_part(D / 32, D / 16);
    // P in bf16 (the MFMA operand); the row sum adds those same rounded values
    // (v_dot2 against ones, two chains), so the normalised weights sum to one
    // exactly as used
    bf16x8_t P[4];
    const bf16x2_t one2 = {(__bf16)1.f, (__bf16)1.f};
    float ls1 = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = exp2_fast(fmaf(S[s >> 1][8 * (s & 1) + e], scale_log2e, -mref));
        uint4 u = make_uint4(pack2(p[0], p[1]), pack2(p[2], p[3]), pack2(p[4], p[5]), pack2(p[6], p[7]));
        P[s] = __builtin_bit_cast(bf16x8_t, u);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u.x), one2, lsum, false);
        ls1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u.y), one2, ls1, false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u.z), one2, lsum, false);
        ls1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u.w), one2, ls1, false);
    }
    lsum += ls1;
    // O^T += V^T P^T: k = key in the permuted order of the S^T accumulators
    const char *vt = buf + TL::KBYTES;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(vt + ((32 * mt + l32) * TL::VROW + 16 * s + 8 * h) * 2);
            O[mt] = mfma(a, P[s], O[mt]);
        }
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW)
void swska_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k,
                  const bf16_t *__restrict__ v, bf16_t *__restrict__ o,
                  int BH, int H, int T, int window, float scale_log2e, int nqb) {
    constexpr int NT = 64 * NW, kBQ = 32 * NW;
    using TL = Tile<D, NT>;
    // three tile buffers: tile j is consumed (softmax, P V) while tile j+1's
    // scores are computed from the next buffer and tile j+2 is written to the third
    __shared__ __attribute__((aligned(16))) char smem[3 * TL::BYTES];

    // XCD-aware block -> (b*H + h, query block): XCD x = id % 8 walks the heads
    // x, x + 8, ... in increasing query-block order.
    const int id = blockIdx.x;
    int bh, qb;
    if (BH % 8 == 0) {
        const int xcd = id % 8, slot = id / 8, per = BH / 8;
        bh = xcd + 8 * (slot % per);
        qb = slot / per;
    } else {
        bh = id % BH;
        qb = id / BH;
    }
    bh = uni(bh);
    qb = uni(qb);
    if (qb >= nqb) return;
    const int b = bh / H;

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5, l32 = l & 31;
    const int q0 = qb * kBQ;
    const int qw0 = q0 + 32 * w;            // this wave's first query
    const int qi = qw0 + l32;               // this lane's query
    const __amdgpu_buffer_rsrc_t kr = rsrc<D>(k + (size_t)b * T * D, T);
    const __amdgpu_buffer_rsrc_t vr = rsrc<D>(v + (size_t)bh * T * D, T);

    // Q^T operand fragments (B operand: n = query, k = channel)
    bf16x8_t qB[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        uint4 x = qi < T ? *reinterpret_cast<const uint4 *>(q + ((size_t)bh * T + qi) * D + 16 * s + 8 * h)
                         : make_uint4(0, 0, 0, 0);
        qB[s] = __builtin_bit_cast(bf16x8_t, x);
    }

    f32x16_t O[D / 32];
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) O[mt] = f32x16_t{};
    float m = -INFINITY, lsum = 0.f;

    const int lo = max(0, q0 - window + 1);
    const int hi = min(T, q0 + kBQ);        // exclusive (> lo: q0 < T)
    const int kt0 = (lo / kBK) * kBK;
    const int ntile = (hi - kt0 + kBK - 1) / kBK;
    // this wave's key range [wlo, whi]
    const int wlo = qw0 - window + 1, whi = qw0 + 31;
    auto skip = [&](int k0) { return (k0 + kBK - 1 < wlo) || (k0 > whi); };
    auto edge = [&](int k0) { return (k0 <= whi - window) || (k0 + kBK - 1 > qw0) || (k0 + kBK > T); };

    uint4 rk[TL::KVEC], rv[TL::KPT];
    fetch_tile<D, NT>(kr, vr, kt0, rk, rv);
    store_tile<D, NT>(smem, rk, rv);
    if (ntile > 1) {
        fetch_tile<D, NT>(kr, vr, kt0 + kBK, rk, rv);
        store_tile<D, NT>(smem + TL::BYTES, rk, rv);
    }
    __syncthreads();
    if (ntile > 2) fetch_tile<D, NT>(kr, vr, kt0 + 2 * kBK, rk, rv);

    // One step: scores of tile j+1 (into Sn) beside the softmax and P V of
    // tile j (from Sc), then tile j+2 to its buffer and tile j+3's loads issued.
    auto step = [&](int j, int bj, f32x16_t (&Sc)[2], f32x16_t (&Sn)[2]) {
        const int k0 = kt0 + j * kBK;
        const int b1 = bj == 2 ? 0 : bj + 1, b2 = b1 == 2 ? 0 : b1 + 1;
        const bool next = j + 1 < ntile && !skip(k0 + kBK);
        const char *cur = smem + bj * TL::BYTES, *nb = smem + b1 * TL::BYTES;
        if (!skip(k0)) {
            if (next)
                softmax_pv<D, NT, true>(cur, Sc, O, m, lsum, edge(k0), k0, qi, window, T, scale_log2e, l32, h, nb,
                                        qB, Sn);
            else
                softmax_pv<D, NT, false>(cur, Sc, O, m, lsum, edge(k0), k0, qi, window, T, scale_log2e, l32, h, nb,
                                         qB, Sn);
        } else if (next) {
            qk_tile<D, NT>(nb, qB, Sn, l32, h);
        }
        if (j + 2 < ntile) store_tile<D, NT>(smem + b2 * TL::BYTES, rk, rv);
        // the staging registers are free again: tile j+3's loads go out before
        // the barrier, so that the wait there overlaps their latency
        if (j + 3 < ntile) fetch_tile<D, NT>(kr, vr, k0 + 3 * kBK, rk, rv);
        __syncthreads();
        return b1;
    };
    f32x16_t Sa[2], Sb[2];
    if (!skip(kt0)) qk_tile<D, NT>(smem, qB, Sa, l32, h);
    int bj = 0;
    for (int j = 0; j < ntile; j += 2) {
        bj = step(j, bj, Sa, Sb);
        if (j + 1 < ntile) bj = step(j + 1, bj, Sb, Sa);
    }

    const float ltot = lsum + __shfl_xor(lsum, 32);
    const float inv = 1.f / ltot;
    if (qi < T) {
        bf16_t *op = o + ((size_t)bh * T + qi) * D;
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d0 = 32 * mt + 8 * a4 + 4 * h;
                *reinterpret_cast<uint2 *>(op + d0) =
                    make_uint2(pack2(O[mt][4 * a4 + 0] * inv, O[mt][4 * a4 + 1] * inv),
                               pack2(O[mt][4 * a4 + 2] * inv, O[mt][4 * a4 + 3] * inv));
            }
    }
}
}  // namespace

// The key and value descriptors address T rows of dk bf16 with 32-bit byte
// offsets: T * dk * 2 must stay below 2^31.
bool swska_supported(int T, int dk, int dv, int dtype) {
    return dtype == 1 && dk == dv && (dk == 128 || dk == 64) && (long long)T * dk * 2 < (1LL << 31);
}

uint64_t swska_launch_items(long long BH, int T, int dk) {
    if (dk == 128) return (uint64_t)BH * (((uint64_t)T + 255) / 256) * 512;
    return (uint64_t)BH * (((uint64_t)T + 127) / 128) * 256;
}

void launch_swska(const SkaArgs &a, hipStream_t st) {
    const int BH = a.B * a.H;
    const float sl2e = a.scale * kLog2e;
    const int window = a.window < a.T ? a.window : a.T;  // w >= T: every earlier key
    if (a.dk == 128) {
        const int nqb = (a.T + 255) / 256;
        hipLaunchKernelGGL((swska_kernel<128, 8>), dim3((unsigned)(BH * nqb)), dim3(512), 0, st, (const bf16_t *)a.q,
                           (const bf16_t *)a.k, (const bf16_t *)a.v, (bf16_t *)a.o, BH, a.H, a.T,
                           window, sl2e, nqb);
    } else {
        const int nqb = (a.T + 127) / 128;
        hipLaunchKernelGGL((swska_kernel<64, 4>), dim3((unsigned)(BH * nqb)), dim3(256), 0, st, (const bf16_t *)a.q,
                           (const bf16_t *)a.k, (const bf16_t *)a.v, (bf16_t *)a.o, BH, a.H, a.T,
                           window, sl2e, nqb);
    }
}

}  // namespace rodimus
