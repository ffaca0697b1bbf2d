// scan_state.hip -- phase 1 of the segment-parallel matrix-core prefill: the
// local end state (from zero) and the total log2 decay of every sub-segment,
// for the output pass (scan_mfma.hip) to fold into each segment's incoming
// state.  Method and layouts: scan_mfma.hip's header (CodeFuse article,
// "ICLR 2025 | Rodimus*: ...", Rodimus block paragraph: the recurrence
// S_t = diag(a_t) S_{t-1} + (beta_t k_t)^T v_t run chunkwise).
//
// Kept in a translation unit of its own so that it is compiled with the
// instruction-level-parallelism scheduler (-amdgpu-sched-strategy=max-ilp),
// which shortens this pass by about 3% and lengthens the output pass by 6%.
#include "scan_mfma.h"

namespace rodimus {
namespace prefill {

namespace {

// One sub-segment's local end state.  Processed in chunks of 32 tokens whatever
// the caller's C (the result does not depend on the chunking), which leaves
// room in the registers for two chunks of raw inputs in flight.
template <int TPR, bool LR>
__device__ __forceinline__ void state_chunk(Raw<16 * TPR, false, LR> &R, Zops<1> &Z, const LrOps &ops,
                                            __amdgpu_buffer_rsrc_t rzg, __amdgpu_buffer_rsrc_t rzt, const Rsrc &rs,
                                            int t0, int tnext, char *sKbT, char *sVT, f32x16_t (&S)[4],
                                            float (&rho)[8], int r, int cg, int l, int w, int h, int l32, int T) {
    float l2a[TPR][8], l2b[TPR][8], lend[8];
    // The prefetches are always issued, from past the rows' end when there is
    // no next chunk, in the order of the first loads (v, then the gate inputs,
    // then k), so that each wait of the in-order load counter is exact.
    const int tn = tnext >= 0 ? tnext : kNoRow;
    if constexpr (LR) {
        // logits of the 32-token chunk on the matrix cores, staged in this
        // wave's rows of the K-bar^T (g) and V^T (tau) areas
        lr_stage<1, kTRow>(Z, ops, sKbT, sVT, w, l);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        uint32_t gw[8][TPR / 2], tw[8][TPR / 2];
        lr_read<TPR, kTRow>(sKbT, sVT, r, cg, gw, tw);
        store_vt<TPR, kTRow>(sVT, cg, r, R.v);   // after the reads, in LDS order
        load_one<TPR>(R.v, rs.v, tn, r, cg);
        load_zops<1>(Z, rzg, rzt, tn, l);
        gates_scan_cols<16 * TPR>(gw, tw, t0, T, r, l, l2a, l2b, lend);
    } else {
        store_vt<TPR, kTRow>(sVT, cg, r, R.v);
        load_one<TPR>(R.v, rs.v, tn, r, cg);
        gates_scan_gt<16 * TPR>(R.g, R.th, t0, T, r, l, l2a, l2b, lend);
        load_gates<16 * TPR, false>(R, rs, tn, r, cg);
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
    load_one<TPR>(R.k, rs.k, tn, r, cg);
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

template <bool VL, bool LR>
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
    __amdgpu_buffer_rsrc_t rzg, rzt;
    LrOps ops;
    if constexpr (LR) {
        const size_t zrow = (size_t)(bh / p.H) * p.T;
        rzg = rsrc_bytes(p.zg + zrow * kRank, Tb * (int)kZRow);
        rzt = rsrc_bytes(p.zt + zrow * kRank, Tb * (int)kZRow);
        lr_load_ops(ops, p.Ug, p.bg, p.Ut, p.bt, bh % p.H, w, l);
    } else {
        rs.g = rsrc(p.g + rowbase * kD, Tb);
        rs.th = rsrc(p.th + rowbase * kD, Tb);
    }
    rs.q = rs.k;

    f32x16_t S[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) S[mt] = f32x16_t{};
    float rho[8];  // log2 decay of the chunks after the current one, per channel
#pragma unroll
    for (int e = 0; e < 8; ++e) rho[e] = 0.f;

    // chunks are visited last to first; two chunks of raw inputs are in flight
    Raw<CS, false, LR> Ra, Rb;
    Zops<1> Za, Zb;
    const int c0 = nch - 1;
    {
        // the first two chunks in the order of the loop's prefetches (v, then
        // the gate inputs, then k), always issued
        const int ta = c0 >= 0 ? t_begin + c0 * CS : kNoRow, tb = c0 >= 1 ? t_begin + (c0 - 1) * CS : kNoRow;
        load_one<TPR>(Ra.v, rs.v, ta, r, cg);
        if constexpr (LR) load_zops<1>(Za, rzg, rzt, ta, l);
        else load_gates<CS, false>(Ra, rs, ta, r, cg);
        load_one<TPR>(Ra.k, rs.k, ta, r, cg);
        load_one<TPR>(Rb.v, rs.v, tb, r, cg);
        if constexpr (LR) load_zops<1>(Zb, rzg, rzt, tb, l);
        else load_gates<CS, false>(Rb, rs, tb, r, cg);
        load_one<TPR>(Rb.k, rs.k, tb, r, cg);
    }
    for (int c = c0; c >= 0; c -= 2) {
        state_chunk<TPR, LR>(Ra, Za, ops, rzg, rzt, rs, t_begin + c * CS, c >= 2 ? t_begin + (c - 2) * CS : -1,
                             sKbT, sVT, S, rho, r, cg, l, w, h, l32, Tb);
        if (c >= 1)
            state_chunk<TPR, LR>(Rb, Zb, ops, rzg, rzt, rs, t_begin + (c - 1) * CS,
                                 c >= 3 ? t_begin + (c - 3) * CS : -1, sKbT, sVT, S, rho, r, cg, l, w, h, l32, Tb);
    }
    float4 *So = reinterpret_cast<float4 *>(p.wsS + ((size_t)sub * p.BH + bh) * kD * kD) + 64 * w + l;
#pragma unroll
    for (int k4 = 0; k4 < 16; ++k4) {
        const f32x16_t &A = S[k4 >> 2];
        const int i = 4 * (k4 & 3);
        So[256 * k4] = make_float4(A[i + 0], A[i + 1], A[i + 2], A[i + 3]);
    }
    if (r == 0) {
        float *A = p.wsA + ((size_t)sub * p.BH + bh) * kD + 8 * cg;
#pragma unroll
        for (int e = 0; e < 8; ++e) A[e] = exp2_fast(rho[e]);
    }
}

}  // namespace

void launch_scan_state(const Params &p, bool vl, bool lr, unsigned nblocks, hipStream_t st) {
    const dim3 g1(nblocks), b1(256);
    if (lr) hipLaunchKernelGGL((scan_state_kernel<false, true>), g1, b1, 0, st, p);
    else if (vl) hipLaunchKernelGGL((scan_state_kernel<true, false>), g1, b1, 0, st, p);
    else hipLaunchKernelGGL((scan_state_kernel<false, false>), g1, b1, 0, st, p);
}

}  // namespace prefill
}  // namespace rodimus
