// scan_mfma.h -- what the two translation units of the bf16 matrix-core
// prefill share: the launch parameters, the row span of a (b,h) and the LDS
// row pitch of the transposed operand tiles.  The output pass and the launcher
// are in scan_mfma.hip; the state pass (phase 1 of the segment-parallel form)
// is in scan_state.hip, a unit of its own so that it is scheduled with its own
// compiler options.
#pragma once

#include "mfma_common.h"

namespace rodimus {
namespace prefill {

constexpr int kMaxT = 1 << 23;     // 32-bit buffer offsets (T * 256 bytes)
// A chunk start whose rows lie past the end of every descriptor (T < kMaxT):
// loads from it return zeros and fetch nothing, and its byte offsets, up to
// (kMaxT + 63) * 256 + 240, still fit 32 bits.
constexpr int kNoRow = kMaxT;
constexpr int kTRow = 64 + 8;      // bf16 per row of sKbT / sVT    [128][C]

struct Params {
    const bf16_t *q, *k, *v, *g, *th;
    const float *S0;  // [BH][128][128] or null (zeros)
    bf16_t *o;
    float *S_T;       // [BH][128][128] or null
    float *wsS;       // [(G-1)*P][BH][16][256] float4: sub-segment states (lane-major) / incoming states
    float *wsA;       // [(G-1)*P][BH][128] total decay of each sub-segment (a power of two)
    int BH, T, G, seg_len, P, sub_len;
    int fold;         // the output pass folds the sub-segment states itself (no combine)
    // packed variable-length batch: sequence s = bh / H occupies rows
    // cu[s] .. cu[s+1]-1 of head h = bh % H's [total][128] rows; T is then the
    // longest length (the segment plan)
    const int *cu;
    int H, total;
    const int *order;  // packed batch: longest-first order of the sequences, or null
    // low-rank gates (LR kernels): factor rows zg, zt [B][T][16] bf16 shared by
    // the heads; per-head factors Ug, Ut [H][128][16] bf16 and biases bg, bt
    // [H][128] fp32
    const bf16_t *zg, *zt, *Ug, *Ut;
    const float *bg, *bt;
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

// Phase 1 of the segment-parallel prefill: the local end state and total
// decay of each of the (G-1)*P sub-segments of every (b,h), into p.wsS and
// p.wsA (one 256-thread workgroup per sub-segment and (b,h): grid nsub * BH).
// vl: packed ragged batch; lr: gate logits from low-rank factors.
void launch_scan_state(const Params &p, bool vl, bool lr, unsigned nblocks, hipStream_t st);

}  // namespace prefill
}  // namespace rodimus
