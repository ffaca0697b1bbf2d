// swska_decode.hip -- one decode step of sliding-window shared-key attention
// (SW-SKA) over ring-buffer window caches, on gfx950.
//
// The key is shared by all heads and every head keeps its own values (SKA,
// "ICLR 2025 | Rodimus*: ..." (CodeFuse), SKA / Rodimus+ paragraphs and Fig. 4,
// which state that sharing the key shrinks the window's KV cache); each query
// sees the previous `window` keys including its own (MiniCPM-SALA blog,
// sections 1.1 and 2.1; window 4096 with shared keys in section 3 of the
// Rodimus* deployment blog).  So the cache of one sequence is
//
//     k_cache [window][dk]      one key per slot, shared by the heads
//     v_cache [H][window][dv]   per head
//
// and position p lives in slot p mod window.  A step for a sequence that has
// seen t tokens writes the new token into slot t mod window and returns, per
// head, the attention of q over positions max(0, t-window+1) .. t, i.e. row t
// of the prefill SW-SKA over the whole sequence.
//
// The step is bound by HBM bytes: every head reads its whole value window
// (window x dv bf16) and the key window once per sequence, for about two flops
// per byte.  Both contractions run on the VALU in fp32.  Two kernels:
//
//   swska_decode_split: workgroup (n, HP heads, split of SPL slots), HP = 2
//       when H is even (else 1), so that each key slice loaded serves HP
//       heads; SPL = 1024 when that still gives 8 workgroups per CU, else 256.
//       Each thread takes every 16th row of the split (D = 128) and one
//       16-byte column slice of it; per group of rows it loads the key slice
//       and the HP value slices together, sums each head's dot product over
//       the lanes that hold the row, and folds the rows into a running
//       maximum, sum and output per head in base 2 (an online softmax per
//       thread).  The row threads are merged through LDS into each head's
//       record for the split: its maximum m, sum l and unnormalised fp32
//       output.  The H / HP workgroups of one (n, split) are consecutive on
//       one XCD, so the split's keys come from HBM once and from that XCD's
//       L2 for the other heads.  The workgroups of the split that holds the
//       new token's slot append v_new (and, for head 0, k_new) to the caches
//       and read that row from k_new / v_new, so no workgroup reads a cache
//       row that this step writes.
//   swska_decode_combine: per (n, h, channel), merges the splits with the
//       rescaling by 2^(m_s - max m) and normalises; one thread per sequence
//       then advances pos[n].
#include "device_common.h"
#include "launch.h"

namespace rodimus {

namespace {

constexpr int kSplit = 256;      // slots per split workgroup (the workspace is sized for it)
constexpr int kSplitLong = 1024; // slots per split workgroup when that still fills the GPU

template <int D>
struct Dec {
    static constexpr int VEC = D / 8;          // 16-byte vectors per row
    static constexpr int RP = 256 / VEC;       // row threads of the split workgroup
    static constexpr int PSTRIDE = D + 4;      // floats per partial record: o[D], m, l, pad
};

__device__ __forceinline__ void unpack8(const uint4 &x, float *f) {
    f[0] = __uint_as_float(x.x << 16); f[1] = __uint_as_float(x.x & 0xffff0000u);
    f[2] = __uint_as_float(x.y << 16); f[3] = __uint_as_float(x.y & 0xffff0000u);
    f[4] = __uint_as_float(x.z << 16); f[5] = __uint_as_float(x.z & 0xffff0000u);
    f[6] = __uint_as_float(x.w << 16); f[7] = __uint_as_float(x.w & 0xffff0000u);
}

// Window geometry of sequence n: the new slot and the number of slots [0, nvalid)
// that hold positions inside the window.
struct Geo {
    int jnew, nvalid;
};
__device__ __forceinline__ Geo geometry(const int *pos, int n, int W) {
    const int t = max(pos[n], 0);
    return Geo{t % W, (t + 1 >= W) ? W : t + 1};
}

// Workgroups b: XCD x = b mod 8 takes the pairs (n, split) x, x + 8, ..., the
// H / HP head groups of a pair in consecutive workgroups of that XCD.  Thread
// (r, c) takes the split's rows r, r + RP, ... and their 16-byte column slice
// c: per group of G rows it loads the key slice and the HP heads' value slices
// together, sums the key slice's dot product with each head's q over the VEC
// lanes of the row, and folds the rows into a running maximum, sum and output
// per head (base 2).  The RP row threads are merged through LDS at the end.
template <int D, int HP, int SPL, bool NTV>
__global__ __launch_bounds__(256)
void swska_decode_split(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_new,
                        const bf16_t *__restrict__ v_new, bf16_t *__restrict__ k_cache,
                        bf16_t *__restrict__ v_cache, const int *__restrict__ pos,
                        float *__restrict__ part, int N, int H, int W, int S, float scale_log2e) {
    using C = Dec<D>;
    __shared__ float sM[HP][C::RP], sL[HP][C::RP];
    __shared__ __attribute__((aligned(16))) float sO[HP][C::RP * D];

    const int HG = H / HP;   // head groups (H is a multiple of HP)
    const int i = (int)(blockIdx.x >> 3), pair = (i / HG) * 8 + (int)(blockIdx.x & 7), h0 = (i % HG) * HP;
    if (pair >= N * S) return;
    const int n = pair / S, s = pair % S, tid = threadIdx.x;
    const Geo g = geometry(pos, n, W);
    const int j0 = s * SPL;
    const int jend = max(0, min(min(SPL, W - j0), g.nvalid - j0));
    const int jn = g.jnew - j0;   // the new token's row, if this split holds it (then jn < jend)
    const int r = tid / C::VEC, c = tid % C::VEC;   // rows r, r + RP, ...; 16-byte column c

    // append the new token (one workgroup per cache row); this step reads
    // that row from k_new / v_new instead
    if (jn >= 0 && jn < SPL && tid < C::VEC) {
#pragma unroll
        for (int hh = 0; hh < HP; ++hh) {
            const size_t nh = (size_t)n * H + h0 + hh;
            reinterpret_cast<uint4 *>(v_cache + (nh * W + g.jnew) * D)[tid] =
                reinterpret_cast<const uint4 *>(v_new + nh * D)[tid];
        }
        if (h0 == 0)
            reinterpret_cast<uint4 *>(k_cache + ((size_t)n * W + g.jnew) * D)[tid] =
                reinterpret_cast<const uint4 *>(k_new + (size_t)n * D)[tid];
    }

    float qf[HP][8];
    const bf16_t *vrow[HP], *vn[HP];
#pragma unroll
    for (int hh = 0; hh < HP; ++hh) {
        const size_t nh = (size_t)n * H + h0 + hh;
        unpack8(*reinterpret_cast<const uint4 *>(q + nh * D + 8 * c), qf[hh]);
        vrow[hh] = v_cache + (nh * W + j0) * D + 8 * c;
        vn[hh] = v_new + nh * D + 8 * c;
    }
    const bf16_t *krow = k_cache + ((size_t)n * W + j0) * D + 8 * c, *kn = k_new + (size_t)n * D + 8 * c;
    constexpr int NP = SPL / C::RP;   // rows per thread
    constexpr int G = 4;                 // rows in flight per thread
    float m[HP], lsum[HP], o[HP][8];
#pragma unroll
    for (int hh = 0; hh < HP; ++hh) {
        m[hh] = -INFINITY;
        lsum[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
    }
#pragma unroll
    for (int p0 = 0; p0 < NP; p0 += G) {
        uint4 kv[G], vv[HP][G];
#pragma unroll
        for (int pp = 0; pp < G; ++pp) {
            const int jj = r + C::RP * (p0 + pp);
            kv[pp] = make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int hh = 0; hh < HP; ++hh) vv[hh][pp] = make_uint4(0, 0, 0, 0);
            if (jj < jend) {
                kv[pp] = *reinterpret_cast<const uint4 *>(jj == jn ? kn : krow + (size_t)jj * D);
#pragma unroll
                for (int hh = 0; hh < HP; ++hh) {
                    const uint4 *src = reinterpret_cast<const uint4 *>(jj == jn ? vn[hh] : vrow[hh] + (size_t)jj * D);
                    if constexpr (NTV)
                        vv[hh][pp] = __builtin_bit_cast(
                            uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(src)));
                    else
                        vv[hh][pp] = *src;
                }
            }
        }
        float sj[HP][G], mn[HP];
#pragma unroll
        for (int hh = 0; hh < HP; ++hh) mn[hh] = m[hh];
#pragma unroll
        for (int pp = 0; pp < G; ++pp) {
            float kf[8];
            unpack8(kv[pp], kf);
            const bool ok = r + C::RP * (p0 + pp) < jend;
#pragma unroll
            for (int hh = 0; hh < HP; ++hh) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d = fmaf(qf[hh][e], kf[e], d);
#pragma unroll
                for (int x = C::VEC / 2; x >= 1; x >>= 1) d += __shfl_xor(d, x);
                sj[hh][pp] = ok ? d * scale_log2e : -INFINITY;
                mn[hh] = fmaxf(mn[hh], sj[hh][pp]);
            }
        }
#pragma unroll
        for (int hh = 0; hh < HP; ++hh) {
            if (mn[hh] > -INFINITY) {   // else no valid row yet: nothing to fold
                const float f = exp2_fast(m[hh] - mn[hh]);   // exp2(-inf) = 0
                lsum[hh] *= f;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[hh][e] *= f;
#pragma unroll
                for (int pp = 0; pp < G; ++pp) {
                    const float pj = exp2_fast(sj[hh][pp] - mn[hh]);
                    float vf[8];
                    unpack8(vv[hh][pp], vf);
                    lsum[hh] += pj;
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(pj, vf[e], o[hh][e]);
                }
                m[hh] = mn[hh];
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // G rows in flight, no more
    }

    // merge the RP row threads of each head: the split's maximum, sum and output
#pragma unroll
    for (int hh = 0; hh < HP; ++hh) {
        *reinterpret_cast<float4 *>(&sO[hh][r * D + 8 * c]) = make_float4(o[hh][0], o[hh][1], o[hh][2], o[hh][3]);
        *reinterpret_cast<float4 *>(&sO[hh][r * D + 8 * c + 4]) = make_float4(o[hh][4], o[hh][5], o[hh][6], o[hh][7]);
        if (c == 0) {
            sM[hh][r] = m[hh];
            sL[hh][r] = lsum[hh];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < HP * D; idx += 256) {
        const int hh = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll 8
        for (int rr = 0; rr < C::RP; ++rr) M = fmaxf(M, sM[hh][rr]);
        float acc = 0.f, L = 0.f;
        if (M > -INFINITY) {
#pragma unroll 8
            for (int rr = 0; rr < C::RP; ++rr) {
                const float f = exp2_fast(sM[hh][rr] - M);
                acc = fmaf(f, sO[hh][rr * D + d], acc);
                L = fmaf(f, sL[hh][rr], L);
            }
        }
        float *rec = part + (((size_t)n * H + h0 + hh) * S + s) * C::PSTRIDE;
        rec[d] = acc;
        if (d == 0) {
            rec[D] = M;
            rec[D + 1] = L;
        }
    }
}

// One workgroup per (n, h), one thread per value channel; the (n, h) records of
// all splits are contiguous.  Each thread folds the splits in batches of 16
// (every load of a batch issued at once) into a running maximum, denominator
// and output, rescaling by 2^(m_s - max m); a split with no slot in the window
// has m = -inf and weight 0.
template <int D>
__global__ __launch_bounds__(D)
void swska_decode_combine(const float *__restrict__ part, bf16_t *__restrict__ o, int *__restrict__ pos,
                          int H, int S) {
    using C = Dec<D>;
    constexpr int B = 16;
    const int nh = blockIdx.x, d = threadIdx.x;
    const float *rec = part + (size_t)nh * S * C::PSTRIDE;
    float M = -INFINITY, L = 0.f, acc = 0.f;
    for (int s0 = 0; s0 < S; s0 += B) {
        float ms[B], ls[B], os[B];
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const float *r = rec + (size_t)(s0 + u) * C::PSTRIDE;
            const bool in = s0 + u < S;
            ms[u] = in ? r[D] : -INFINITY;
            ls[u] = in ? r[D + 1] : 0.f;
            os[u] = in ? r[d] : 0.f;
        }
        float mn = M;
#pragma unroll
        for (int u = 0; u < B; ++u) mn = fmaxf(mn, ms[u]);
        if (mn > -INFINITY) {
            const float f = exp2_fast(M - mn);   // exp2(-inf) = 0
            acc *= f;
            L *= f;
#pragma unroll
            for (int u = 0; u < B; ++u) {
                const float w = exp2_fast(ms[u] - mn);
                acc = fmaf(w, os[u], acc);
                L = fmaf(w, ls[u], L);
            }
            M = mn;
        }
    }
    o[(size_t)nh * D + d] = f2bf(acc / L);   // L > 0: the new token's own slot is in the window
    if (nh % H == 0 && d == 0) pos[nh / H] += 1;
}

}  // namespace

bool swska_decode_supported(int dk, int dv, int dtype) {
    return dtype == 1 && dk == dv && (dk == 128 || dk == 64);
}

// Workspace: the partial records [N][H][S][dv + 4] fp32.
static int value_splits(int window) { return (window + kSplit - 1) / kSplit; }

size_t swska_decode_workspace(int N, int H, int dv, int window) {
    return (size_t)N * H * value_splits(window) * (dv + 4) * sizeof(float);
}

size_t swska_decode_blocks(int N, int H, int window) {
    return ((size_t)N * value_splits(window) + 7) / 8 * 8 * H;
}

// Value windows larger than this are read with streaming (non-temporal)
// loads: they cannot stay in the 256 MB Infinity Cache from one step to the
// next, and the hint keeps them from displacing the keys, which the other
// heads' workgroups read again from L2.  Measured, 16 heads x 4096 slots x
// 128: 64 sequences (1.07 GB of values) 198-202 -> 175-176 us per step; 32
// sequences 107-109 -> 95 us; 16 sequences (268 MB) 47-50 against 50-51 us
// with the hint, so smaller windows keep ordinary loads.
constexpr size_t kValueStreamBytes = (size_t)384 << 20;

template <int D, int HP, int SPL>
static void launch_split(const SkaDecArgs &a, int S, float *part, hipStream_t st) {
    const size_t blocks = ((size_t)a.N * S + 7) / 8 * 8 * (a.H / HP);
    const bool ntv = (size_t)a.N * a.H * a.window * D * 2 > kValueStreamBytes;
    if (ntv)
        hipLaunchKernelGGL((swska_decode_split<D, HP, SPL, true>), dim3((unsigned)blocks), dim3(256), 0, st,
                           (const bf16_t *)a.q, (const bf16_t *)a.k_new, (const bf16_t *)a.v_new,
                           (bf16_t *)a.k_cache, (bf16_t *)a.v_cache, a.pos, part, a.N, a.H, a.window, S,
                           a.scale * kLog2e);
    else
        hipLaunchKernelGGL((swska_decode_split<D, HP, SPL, false>), dim3((unsigned)blocks), dim3(256), 0, st,
                           (const bf16_t *)a.q, (const bf16_t *)a.k_new, (const bf16_t *)a.v_new,
                           (bf16_t *)a.k_cache, (bf16_t *)a.v_cache, a.pos, part, a.N, a.H, a.window, S,
                           a.scale * kLog2e);
}

// Splits of kSplitLong slots when that leaves at least 8 split workgroups per
// CU (fewer records to combine, and each key and value stream runs longer),
// else of kSplit slots; two heads per workgroup when H is even.
template <int D>
static void launch_d(const SkaDecArgs &a, hipStream_t st) {
    float *part = reinterpret_cast<float *>(a.workspace);
    const int HP = a.H % 2 == 0 ? 2 : 1;
    const int SL = (a.window + kSplitLong - 1) / kSplitLong;
    const bool lng = (size_t)a.N * SL * (a.H / HP) >= 8 * 256;
    const int S = lng ? SL : value_splits(a.window);
    if (HP == 2) {
        if (lng) launch_split<D, 2, kSplitLong>(a, S, part, st);
        else launch_split<D, 2, kSplit>(a, S, part, st);
    } else {
        if (lng) launch_split<D, 1, kSplitLong>(a, S, part, st);
        else launch_split<D, 1, kSplit>(a, S, part, st);
    }
    hipLaunchKernelGGL(swska_decode_combine<D>, dim3((unsigned)((size_t)a.N * a.H)), dim3(D), 0, st, part,
                       (bf16_t *)a.o, a.pos, a.H, S);
}

void launch_swska_decode(const SkaDecArgs &a, hipStream_t st) {
    if (a.dk == 128)
        launch_d<128>(a, st);
    else
        launch_d<64>(a, st);
}

}  // namespace rodimus
