// launch.h -- host-side launchers behind the C ABI (validated arguments only).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rodimus {

struct ScanArgs {
    const void *q, *k, *v, *g, *tau;
    const float *S0;  // nullable
    void *o;
    float *S_T;       // nullable
    int B, H, T, dk, dv, chunk, dtype;
    void *workspace;
    size_t workspace_bytes;
    // packed variable-length batch (nullable): B sequences, sequence s in rows
    // cu[s] .. cu[s+1]-1 of each head's [total][d] rows, T = longest length;
    // order (nullable): longest-first order of the sequences
    const int *cu = nullptr;
    int total = 0;
    int *order = nullptr;
    // low-rank gates (nullable; batched layout, bf16, dk = dv = 128 only): the
    // rank-16 factor rows zg, zt [B][T][16] replace g and tau; Ug, Ut
    // [H][128][16] bf16 and bg, bt [H][128] fp32 are the per-head factors
    const void *zg = nullptr, *zt = nullptr, *Ug = nullptr, *Ut = nullptr;
    const float *bg = nullptr, *bt = nullptr;
};

struct ScanBwdArgs {
    const void *q, *k, *v, *g, *tau;
    const float *S0;   // nullable
    const void *dO;
    const float *dS_T; // nullable
    float *dq, *dk_, *dv_, *dg, *dtau;
    float *dS0;        // nullable
    int B, H, T, dk, dv, dtype;
    void *workspace;
    // packed variable-length batch (nullable), as in ScanArgs
    const int *cu = nullptr;
    int total = 0;
    int *order = nullptr;
};

struct DecodeArgs {
    const void *q, *k, *v, *g, *tau;
    const float *S_in;
    float *S_out;
    void *o;
    int N, H, dk, dv, dtype;
};

struct SkaArgs {
    const void *q, *k, *v;
    void *o;
    int B, H, T, dk, dv, window;
    float scale;
    int dtype;
};

struct SkaDecArgs {
    const void *q, *k_new, *v_new;
    void *k_cache, *v_cache;
    int *pos;
    void *o;
    int N, H, dk, dv, window;
    float scale;
    int dtype;
    void *workspace;
};

// Longest-first order of the sequences of a packed batch (seq_order.hip):
// order[rank] = sequence, ranked by length for N <= kOrderMax and counted by
// 64-token chunk count above that.  It sits in the workspace after the plan's
// own bytes (seq_order_bytes(N) of them).
constexpr int kOrderMax = 4096;
size_t seq_order_bytes(int N);
void launch_seq_order(const int *cu, int N, int total, int T, int *order, hipStream_t st);

// Segment plan of the prefill: number of T-segments per (b,h) and workspace.
struct ScanPlan {
    bool mfma;     // bf16, dk = dv = 128 MFMA kernel
    int segments;  // >= 1
    size_t workspace_bytes;
};
ScanPlan plan_scan(int B, int H, int T, int dk, int dv, int chunk, int dtype);

// Work-items (workgroups x threads, in x) of the largest launch a call makes.
// HIP rejects a launch of 2^32 work-items or more, so the C ABI refuses such
// sizes with RODIMUS_ERR_INVALID_ARG before launching anything.
constexpr uint64_t kMaxLaunchItems = 1ull << 32;
uint64_t scan_mfma_launch_items(long long BH, int T, int chunk);
uint64_t scan_generic_launch_items(long long BH);
uint64_t scan_bwd_mfma_launch_items(long long BH, int T);
uint64_t scan_bwd_launch_items(long long BH, int T);
uint64_t decode_launch_items(long long NH);
uint64_t swska_launch_items(long long BH, int T, int dk);

void launch_decode_step(const DecodeArgs &a, hipStream_t st);
void launch_scan_generic(const ScanArgs &a, hipStream_t st);
void launch_scan_mfma(const ScanArgs &a, const ScanPlan &p, hipStream_t st);
void launch_state_copy(const float *S0, float *S_T, size_t n, hipStream_t st);
size_t scan_bwd_workspace(int B, int H, int T, int dk, int dv);
void launch_scan_bwd(const ScanBwdArgs &a, hipStream_t st);
bool scan_bwd_mfma_supported(int T, int dk, int dv, int dtype);
size_t scan_bwd_mfma_workspace(int B, int H, int T);
void launch_scan_bwd_mfma(const ScanBwdArgs &a, hipStream_t st);
bool swska_supported(int T, int dk, int dv, int dtype);
void launch_swska(const SkaArgs &a, hipStream_t st);
bool swska_decode_supported(int dk, int dv, int dtype);
size_t swska_decode_workspace(int N, int H, int dv, int window);
size_t swska_decode_blocks(int N, int H, int window);   // workgroups of the split kernel
void launch_swska_decode(const SkaDecArgs &a, hipStream_t st);

}  // namespace rodimus
