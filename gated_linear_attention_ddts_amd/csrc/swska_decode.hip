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
// per byte.  The value contraction runs on the VALU in fp32; the scores, a
// small (key block x heads) product per sequence, on the matrix cores with
// fp32 accumulation.  Three kernels:
//
//   swska_decode_scores: workgroup (n, 128-slot block).  The owner of the new
//       token's slot appends k_new / v_new to the caches.  The block's keys
//       are loaded once into MFMA operand registers (k_new for the new slot,
//       which no other workgroup reads) and scored against every head's query
//       on the matrix cores (keys x heads, 32 heads per tile); scores (scaled
//       to base 2) go to the workspace, -inf for slots outside the window.
//       The key window is read once for all heads.
//   swska_decode_values: workgroup (n, h, 256-slot split), few registers so
//       that many are resident: the split's base-2 softmax weights relative
//       to its own maximum, then the head's value rows streamed with 16-byte
//       loads (16 lanes per row, several rows in flight per thread), reduced
//       through LDS.  It writes per (n, h, split) the maximum m, the sum l and
//       the unnormalised fp32 output.
//   swska_decode_combine: per (n, h, channel), merges the splits with the
//       rescaling by 2^(m_s - max m) and normalises; one thread per sequence
//       then advances pos[n].
#include "device_common.h"
#include "launch.h"

namespace rodimus {

namespace {

constexpr int kSlots = 128;     // slots per scoring workgroup
constexpr int kSplit = 256;     // slots per value workgroup
constexpr int kMaxSplits = 1 << 11;  // window <= kSplit * kMaxSplits = 524288

template <int D>
struct Dec {
    static constexpr int VEC = D / 8;          // 16-byte vectors per row
    static constexpr int RP = 256 / VEC;       // rows per pass of the value workgroup
    static constexpr int PSTRIDE = D + 4;      // floats per partial record: o[D], m, l, pad
};

__device__ __forceinline__ void unpack8(const uint4 &x, float *f) {
    f[0] = __uint_as_float(x.x << 16); f[1] = __uint_as_float(x.x & 0xffff0000u);
    f[2] = __uint_as_float(x.y << 16); f[3] = __uint_as_float(x.y & 0xffff0000u);
    f[4] = __uint_as_float(x.z << 16); f[5] = __uint_as_float(x.z & 0xffff0000u);
    f[6] = __uint_as_float(x.w << 16); f[7] = __uint_as_float(x.w & 0xffff0000u);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
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

// S = Q K^T on v_mfma_f32_32x32x16_bf16: A[m][k] sits in lane m + 32*(k/8),
// element k%8; B[k][n] in lane n + 32*(k/8), element k%8; C[m][n] in lane
// n + 32*((m/4)%2), register 4*(m/8) + m%4.  Heads on M, keys (slots) on N, so
// that a score row is stored by consecutive lanes: each lane loads its slot's
// key fragments straight into registers (no LDS, no barrier), and the wave
// reuses them for every group of 32 heads.
template <int D>
__global__ __launch_bounds__(256)
void swska_decode_scores(const bf16_t *__restrict__ q, const bf16_t *__restrict__ k_new,
                         const bf16_t *__restrict__ v_new, bf16_t *__restrict__ k_cache,
                         bf16_t *__restrict__ v_cache, const int *__restrict__ pos,
                         float *__restrict__ scores, int H, int W, int Wp, int S, float scale_log2e) {
    using C = Dec<D>;
    const int n = blockIdx.x / S, s = blockIdx.x % S, tid = threadIdx.x;
    const Geo g = geometry(pos, n, W);
    const int j0 = s * kSlots;
    const int nsl = min(kSlots, W - j0);          // slots of this block
    const size_t kc = (size_t)n * W * D;          // this sequence's key window
    const bf16_t *kn = k_new + (size_t)n * D;

    // this lane's slot (A row) and key fragments; the new slot reads k_new,
    // slots outside the window are zero (and masked below)
    const int w = tid >> 6, l = tid & 63, hl = l >> 5, l32 = l & 31;
    const int j = 32 * w + l32, slot = j0 + j;
    const bool inwin = j < nsl && slot < g.nvalid;
    const bf16_t *krow = (slot == g.jnew) ? kn : k_cache + kc + (size_t)slot * D;
    bf16x8_t a[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
        const uint4 x = inwin ? *reinterpret_cast<const uint4 *>(krow + 16 * st + 8 * hl) : make_uint4(0, 0, 0, 0);
        a[st] = __builtin_bit_cast(bf16x8_t, x);
    }

    // the owner of the new slot appends k_new / v_new to the caches (no lane
    // reads that cache row: the slot's fragments come from k_new)
    if (g.jnew >= j0 && g.jnew < j0 + nsl) {
        for (int e = tid; e < C::VEC; e += 256)
            reinterpret_cast<uint4 *>(k_cache + kc + (size_t)g.jnew * D)[e] = reinterpret_cast<const uint4 *>(kn)[e];
        for (int e = tid; e < H * C::VEC; e += 256) {
            const int h = e / C::VEC, c = e % C::VEC;
            reinterpret_cast<uint4 *>(v_cache + (((size_t)n * H + h) * W + g.jnew) * D)[c] =
                reinterpret_cast<const uint4 *>(v_new + ((size_t)n * H + h) * D)[c];
        }
    }

    for (int hg = 0; hg < H; hg += 32) {
        const int head = hg + l32;
        bf16x8_t qB[D / 16];
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const uint4 x = head < H ? *reinterpret_cast<const uint4 *>(q + ((size_t)n * H + head) * D + 16 * st + 8 * hl)
                                     : make_uint4(0, 0, 0, 0);
            qB[st] = __builtin_bit_cast(bf16x8_t, x);
        }
        f32x16_t acc = {};
#pragma unroll
        for (int st = 0; st < D / 16; ++st) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qB[st], a[st], acc, 0, 0, 0);
        // register i: head hg + 8(i/4) + 4hl + i%4, slot j (this lane's)
        if (j < nsl) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int hh = hg + 8 * (i >> 2) + 4 * hl + (i & 3);
                if (hh < H) scores[((size_t)n * H + hh) * Wp + slot] = inwin ? acc[i] * scale_log2e : -INFINITY;
            }
        }
    }
}

template <int D>
__global__ __launch_bounds__(256)
void swska_decode_values(const bf16_t *__restrict__ v_cache, const int *__restrict__ pos,
                         const float *__restrict__ scores, float *__restrict__ part,
                         int H, int W, int Wp, int S) {
    using C = Dec<D>;
    __shared__ float sP[kSplit];
    __shared__ float sRed[4];
    __shared__ __attribute__((aligned(16))) float sO[C::RP * D];

    const int nh = blockIdx.x / S, s = blockIdx.x % S, n = nh / H, tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63;
    const Geo g = geometry(pos, n, W);
    const int j0 = s * kSplit;
    const int jend = max(0, min(min(kSplit, W - j0), g.nvalid - j0));   // valid slots [0, jend)

    // the split's weights relative to its own maximum
    const float sc = tid < jend ? scores[(size_t)nh * Wp + j0 + tid] : -INFINITY;
    const float wm = wave_max(sc);
    if (l == 0) sRed[w] = wm;
    __syncthreads();
    const float m = fmaxf(fmaxf(sRed[0], sRed[1]), fmaxf(sRed[2], sRed[3]));
    const float p = exp2_fast(sc - ((m == -INFINITY) ? 0.f : m));          // exp2(-inf) = 0
    sP[tid] = p;
    const float ws = wave_sum(p);
    __syncthreads();                                                      // sRed (max) read by all
    if (l == 0) sRed[w] = ws;
    __syncthreads();
    const float lsum = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);

    // value rows: thread -> row r (+ RP per pass), 16-byte column c
    const int r = tid / C::VEC, c = tid % C::VEC;
    const bf16_t *vrow = v_cache + ((size_t)nh * W + j0) * D + 8 * c;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int jj = r; jj < jend; jj += C::RP) {
        float vf[8];
        unpack8(*reinterpret_cast<const uint4 *>(vrow + (size_t)jj * D), vf);
        const float pj = sP[jj];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(pj, vf[e], o[e]);
    }
    *reinterpret_cast<float4 *>(sO + r * D + 8 * c) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4 *>(sO + r * D + 8 * c + 4) = make_float4(o[4], o[5], o[6], o[7]);
    __syncthreads();
    float *rec = part + ((size_t)nh * S + s) * C::PSTRIDE;
    if (tid < D) {
        float acc = 0.f;
#pragma unroll 8
        for (int rr = 0; rr < C::RP; ++rr) acc += sO[rr * D + tid];
        rec[tid] = acc;
    }
    if (tid == 0) {
        rec[D] = m;
        rec[D + 1] = lsum;
    }
}

// One workgroup per (n, h), one thread per value channel; the (n, h) records of
// all splits are contiguous.  The split weights 2^(m_s - max m) are formed
// once in LDS, then every channel sums its S partial outputs independently.
template <int D>
__global__ __launch_bounds__(D)
void swska_decode_combine(const float *__restrict__ part, bf16_t *__restrict__ o, int *__restrict__ pos,
                          int H, int S) {
    using C = Dec<D>;
    __shared__ float sF[kMaxSplits];
    __shared__ float sL;
    const int nh = blockIdx.x, d = threadIdx.x;
    const float *rec = part + (size_t)nh * S * C::PSTRIDE;
    if (d < 64) {  // wave 0: global maximum, weights, denominator
        float M = -INFINITY;
        for (int s = d; s < S; s += 64) M = fmaxf(M, rec[(size_t)s * C::PSTRIDE + D]);
        M = wave_max(M);
        float L = 0.f;
        for (int s = d; s < S; s += 64) {
            const float ms = rec[(size_t)s * C::PSTRIDE + D];
            const float f = (ms == -INFINITY) ? 0.f : exp2_fast(ms - M);  // a split with no slot in the window
            sF[s] = f;
            L = fmaf(f, rec[(size_t)s * C::PSTRIDE + D + 1], L);
        }
        L = wave_sum(L);
        if (d == 0) sL = L;
    }
    __syncthreads();
    float acc = 0.f;
#pragma unroll 8
    for (int s = 0; s < S; ++s) acc = fmaf(sF[s], rec[(size_t)s * C::PSTRIDE + d], acc);
    o[(size_t)nh * D + d] = f2bf(acc / sL);
    if (nh % H == 0 && d == 0) pos[nh / H] += 1;
}

}  // namespace

bool swska_decode_supported(int dk, int dv, int dtype) {
    return dtype == 1 && dk == dv && (dk == 128 || dk == 64);
}

// Workspace: scores [N][H][Wp] fp32 (Wp = window rounded up to kSplit), then
// the partial records [N][H][S][dv + 4] fp32.
static int value_splits(int window) { return (window + kSplit - 1) / kSplit; }

size_t swska_decode_workspace(int N, int H, int dv, int window) {
    const size_t S = value_splits(window), Wp = S * kSplit;
    return (size_t)N * H * (Wp + S * (dv + 4)) * sizeof(float);
}

void launch_swska_decode(const SkaDecArgs &a, hipStream_t st) {
    const int SA = (a.window + kSlots - 1) / kSlots, S = value_splits(a.window), Wp = S * kSplit;
    const float sl2e = a.scale * kLog2e;
    float *scores = reinterpret_cast<float *>(a.workspace);
    float *part = scores + (size_t)a.N * a.H * Wp;
    const dim3 g1((unsigned)((size_t)a.N * SA)), g2((unsigned)((size_t)a.N * a.H * S)),
        g3((unsigned)((size_t)a.N * a.H));
    if (a.dk == 128) {
        hipLaunchKernelGGL(swska_decode_scores<128>, g1, dim3(256), 0, st, (const bf16_t *)a.q,
                           (const bf16_t *)a.k_new, (const bf16_t *)a.v_new, (bf16_t *)a.k_cache,
                           (bf16_t *)a.v_cache, a.pos, scores, a.H, a.window, Wp, SA, sl2e);
        hipLaunchKernelGGL(swska_decode_values<128>, g2, dim3(256), 0, st, (const bf16_t *)a.v_cache, a.pos,
                           scores, part, a.H, a.window, Wp, S);
        hipLaunchKernelGGL(swska_decode_combine<128>, g3, dim3(128), 0, st, part, (bf16_t *)a.o, a.pos, a.H, S);
    } else {
        hipLaunchKernelGGL(swska_decode_scores<64>, g1, dim3(256), 0, st, (const bf16_t *)a.q,
                           (const bf16_t *)a.k_new, (const bf16_t *)a.v_new, (bf16_t *)a.k_cache,
                           (bf16_t *)a.v_cache, a.pos, scores, a.H, a.window, Wp, SA, sl2e);
        hipLaunchKernelGGL(swska_decode_values<64>, g2, dim3(256), 0, st, (const bf16_t *)a.v_cache, a.pos,
                           scores, part, a.H, a.window, Wp, S);
        hipLaunchKernelGGL(swska_decode_combine<64>, g3, dim3(64), 0, st, part, (bf16_t *)a.o, a.pos, a.H, S);
    }
}

}  // namespace rodimus
