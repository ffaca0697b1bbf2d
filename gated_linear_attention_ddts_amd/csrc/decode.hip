// decode.hip -- fused recurrent step  S' = diag(a) S + (beta*k)^T v,  o = q S'
//
// The O(1)-state inference form of the Rodimus block (CodeFuse article,
// Rodimus block paragraph), with the state resident in HBM and updated in
// place (MiniCPM-SALA blog, section 3.3).  The step is bound by HBM: the fp32
// state is read once and written once (2 * dk * dv * 4 bytes per head-step);
// q, k, v, g, tau and o add 5*dk + 2*dv elements.
//
// Fast kernel (dk, dv powers of two): one workgroup per (sequence, head).
// Thread (cg, rg) owns the float4 column group cg (columns 4cg..4cg+3) and the
// rows rg, rg + RG, rg + 2RG, ...; consecutive lanes own consecutive column
// groups, so every state load/store instruction touches whole 512-byte rows.
// All state loads are issued before the gate math so that they are in flight
// while the gates are evaluated.  The partial dot products q . S'[:, j] of the
// RG row groups are reduced through LDS.
//
// State loads (measured, 128x128 heads): a state updated in place and small
// enough to stay largely in the 256 MB Infinity Cache between steps is read
// with ordinary loads (N = 256: 80.7 us per step against 90.4 with streaming
// loads); a state written elsewhere (S_out != S_in) or updated in place but
// larger than 640 MiB is read with non-temporal loads (ping-pong N = 256: 91.6
// against 102.9 us; in place N = 1024: 390 against 441 us).
#include "device_common.h"
#include "launch.h"

namespace rodimus {

template <typename Tin, int DK, int DV, bool NTLOAD>
__global__ __launch_bounds__((DK * DV / 4 < 256 ? DK * DV / 4 : 256))
void decode_step_kernel(const Tin *__restrict__ q, const Tin *__restrict__ k,
                        const Tin *__restrict__ v, const Tin *__restrict__ g,
                        const Tin *__restrict__ th, const float *S_in, float *S_out,
                        Tin *__restrict__ o) {
    constexpr int CG = DV / 4;                              // float4 column groups
    constexpr int NT = (DK * CG < 256) ? DK * CG : 256;    // threads
    constexpr int RG = NT / CG;                             // row groups
    constexpr int RPT = DK / RG;                            // rows per thread
    static_assert(NT % 64 == 0 || NT < 64, "thread count");

    const int nh = blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;

    const float4 *Si = reinterpret_cast<const float4 *>(S_in + (size_t)nh * DK * DV);
    float4 *So = reinterpret_cast<float4 *>(S_out + (size_t)nh * DK * DV);

    float4 s[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        if constexpr (NTLOAD) {
            const f32x4_nt t =
                __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt *>(Si + (rg + r * RG) * CG + cg));
            s[r] = make_float4(t[0], t[1], t[2], t[3]);
        } else {
            s[r] = Si[(rg + r * RG) * CG + cg];
        }
    }

    __shared__ float a_s[DK], bk_s[DK], q_s[DK];
    __shared__ float v_s[DV];
    __shared__ float4 red[RG][CG];

    for (int i = tid; i < DK; i += NT) {
        size_t e = (size_t)nh * DK + i;
        float la, lb;
        ddts_log_gates(Elem<Tin>::ld(g, e), Elem<Tin>::ld(th, e), la, lb);
        a_s[i] = exp2_fast(la * kLog2e);
        bk_s[i] = exp2_fast(lb * kLog2e) * Elem<Tin>::ld(k, e);
        q_s[i] = Elem<Tin>::ld(q, e);
    }
    for (int j = tid; j < DV; j += NT) v_s[j] = Elem<Tin>::ld(v, (size_t)nh * DV + j);
    __syncthreads();

    const float4 vv = make_float4(v_s[4 * cg], v_s[4 * cg + 1], v_s[4 * cg + 2], v_s[4 * cg + 3]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int i = rg + r * RG;
        const float a = a_s[i], b = bk_s[i], qi = q_s[i];
        float4 x = s[r];
        x.x = fmaf(a, x.x, b * vv.x);
        x.y = fmaf(a, x.y, b * vv.y);
        x.z = fmaf(a, x.z, b * vv.z);
        x.w = fmaf(a, x.w, b * vv.w);
        acc.x = fmaf(qi, x.x, acc.x);
        acc.y = fmaf(qi, x.y, acc.y);
        acc.z = fmaf(qi, x.z, acc.z);
        acc.w = fmaf(qi, x.w, acc.w);
        st_stream(&So[i * CG + cg], x);
    }
    red[rg][cg] = acc;
    __syncthreads();
    if (rg == 0) {
        float4 t = red[0][cg];
#pragma unroll
        for (int r = 1; r < RG; ++r) {
            float4 u = red[r][cg];
            t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
        }
        const size_t ob = (size_t)nh * DV + 4 * cg;
        Elem<Tin>::st(o, ob + 0, t.x);
        Elem<Tin>::st(o, ob + 1, t.y);
        Elem<Tin>::st(o, ob + 2, t.z);
        Elem<Tin>::st(o, ob + 3, t.w);
    }
}

// Any dk, dv (multiples of 16 up to 128): one thread per state column, loop
// over rows.  Loads are still coalesced across the column index.
template <typename Tin>
__global__ __launch_bounds__(128)
void decode_step_generic_kernel(const Tin *__restrict__ q, const Tin *__restrict__ k,
                                const Tin *__restrict__ v, const Tin *__restrict__ g,
                                const Tin *__restrict__ th, const float *S_in, float *S_out,
                                Tin *__restrict__ o, int dk, int dv) {
    const int nh = blockIdx.x;
    const int j = threadIdx.x;
    __shared__ float a_s[128], bk_s[128], q_s[128];
    for (int i = j; i < dk; i += blockDim.x) {
        size_t e = (size_t)nh * dk + i;
        float la, lb;
        ddts_log_gates(Elem<Tin>::ld(g, e), Elem<Tin>::ld(th, e), la, lb);
        a_s[i] = exp2_fast(la * kLog2e);
        bk_s[i] = exp2_fast(lb * kLog2e) * Elem<Tin>::ld(k, e);
        q_s[i] = Elem<Tin>::ld(q, e);
    }
    __syncthreads();
    if (j >= dv) return;
    const float vj = Elem<Tin>::ld(v, (size_t)nh * dv + j);
    const float *Si = S_in + (size_t)nh * dk * dv;
    float *So = S_out + (size_t)nh * dk * dv;
    float acc = 0.f;
    for (int i = 0; i < dk; ++i) {
        float x = fmaf(a_s[i], Si[(size_t)i * dv + j], bk_s[i] * vj);
        acc = fmaf(q_s[i], x, acc);
        So[(size_t)i * dv + j] = x;
    }
    Elem<Tin>::st(o, (size_t)nh * dv + j, acc);
}

// In-place states up to this size are read with ordinary loads (see above).
constexpr size_t kInPlaceCachedBytes = (size_t)640 << 20;

template <typename Tin, int DK, int DV>
static void launch_fast(const DecodeArgs &a, hipStream_t st) {
    constexpr int CG = DV / 4;
    constexpr int NT = (DK * CG < 256) ? DK * CG : 256;
    const size_t state_bytes = (size_t)a.N * a.H * DK * DV * sizeof(float);
    const bool nt = a.S_out != a.S_in || state_bytes > kInPlaceCachedBytes;
    if (nt)
        hipLaunchKernelGGL((decode_step_kernel<Tin, DK, DV, true>), dim3(a.N * a.H), dim3(NT), 0, st,
                           (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v, (const Tin *)a.g,
                           (const Tin *)a.tau, a.S_in, a.S_out, (Tin *)a.o);
    else
        hipLaunchKernelGGL((decode_step_kernel<Tin, DK, DV, false>), dim3(a.N * a.H), dim3(NT), 0, st,
                           (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v, (const Tin *)a.g,
                           (const Tin *)a.tau, a.S_in, a.S_out, (Tin *)a.o);
}

template <typename Tin>
static void launch_typed(const DecodeArgs &a, hipStream_t st) {
#define RODIMUS_DEC_CASE(DK_, DV_) \
    if (a.dk == DK_ && a.dv == DV_) return launch_fast<Tin, DK_, DV_>(a, st);
    RODIMUS_DEC_CASE(128, 128)
    RODIMUS_DEC_CASE(64, 64)
    RODIMUS_DEC_CASE(128, 64)
    RODIMUS_DEC_CASE(64, 128)
    RODIMUS_DEC_CASE(32, 32)
    RODIMUS_DEC_CASE(16, 32)
    RODIMUS_DEC_CASE(32, 64)
    RODIMUS_DEC_CASE(16, 16)
#undef RODIMUS_DEC_CASE
    hipLaunchKernelGGL((decode_step_generic_kernel<Tin>), dim3(a.N * a.H), dim3(128), 0, st,
                       (const Tin *)a.q, (const Tin *)a.k, (const Tin *)a.v, (const Tin *)a.g,
                       (const Tin *)a.tau, a.S_in, a.S_out, (Tin *)a.o, a.dk, a.dv);
}

// One workgroup per (sequence, head) of at most 256 threads.
uint64_t decode_launch_items(long long NH) { return (uint64_t)NH * 256; }

void launch_decode_step(const DecodeArgs &a, hipStream_t st) {
    if (a.dtype == 0) launch_typed<float>(a, st);
    else launch_typed<bf16_t>(a, st);
}

}  // namespace rodimus
