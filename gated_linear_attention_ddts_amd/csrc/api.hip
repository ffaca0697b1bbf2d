// api.hip -- the C ABI of librodimus: argument validation and dispatch.
// Every check runs before any HIP call; see include/rodimus.h for the
// contract of each entry point.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/rodimus.h"
#include "launch.h"

namespace rodimus {

static bool ok_ptr(const void *p) { return p != nullptr && ((uintptr_t)p & 15) == 0; }
static bool ok_opt_ptr(const void *p) { return p == nullptr || ((uintptr_t)p & 15) == 0; }
static bool ok_head_dim(int d) { return d >= 16 && d <= 128 && d % 16 == 0; }
static bool ok_dtype(int dt) { return dt == RODIMUS_F32 || dt == RODIMUS_BF16; }

static int hip_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? RODIMUS_OK : RODIMUS_ERR_HIP;
}

__global__ void state_copy_kernel(const float *__restrict__ src, float *__restrict__ dst, size_t n) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) dst[i] = src ? src[i] : 0.f;
}

void launch_state_copy(const float *S0, float *S_T, size_t n, hipStream_t st) {
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) return;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, S0, S_T, n);
}

}  // namespace rodimus

using namespace rodimus;

extern "C" {

const char *rodimus_status_string(int status) {
    switch (status) {
        case RODIMUS_OK: return "RODIMUS_OK";
        case RODIMUS_ERR_INVALID_ARG: return "RODIMUS_ERR_INVALID_ARG: invalid argument";
        case RODIMUS_ERR_UNSUPPORTED: return "RODIMUS_ERR_UNSUPPORTED: shape/dtype not compiled";
        case RODIMUS_ERR_HIP: return "RODIMUS_ERR_HIP: HIP runtime error";
        case RODIMUS_ERR_TOO_LARGE:
            return "RODIMUS_ERR_TOO_LARGE: needs more scratch than the fixed no-allocation buffer holds";
        default: return "RODIMUS_UNKNOWN_STATUS";
    }
}

// Every launch of a prefill stays below HIP's 2^32 work-items.
static bool scan_launch_fits(const ScanPlan &plan, int B, int H, int T, int chunk) {
    const long long BH = (long long)B * H;
    const uint64_t items = plan.mfma ? scan_mfma_launch_items(BH, T, chunk) : scan_generic_launch_items(BH);
    return items < kMaxLaunchItems;
}

static bool scan_bwd_launch_fits(bool mfma, int B, int H, int T) {
    const long long BH = (long long)B * H;
    return (mfma ? scan_bwd_mfma_launch_items(BH, T) : scan_bwd_launch_items(BH, T)) < kMaxLaunchItems;
}

static bool scan_sizes_ok(int B, int H, int T, int dk, int dv, int chunk, int dtype) {
    if (B < 0 || H < 0 || T < 0) return false;
    if (!ok_head_dim(dk) || !ok_head_dim(dv) || !ok_dtype(dtype)) return false;
    if (!(chunk == 0 || chunk == 16 || chunk == 32 || chunk == 64)) return false;
    // element counts must fit the kernels' index arithmetic
    if ((long long)B * H > (1LL << 30)) return false;
    if ((long long)B * H * T * (dk > dv ? dk : dv) > (1LL << 46)) return false;
    return true;
}

size_t rodimus_scan_prefill_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk,
                                            int dtype) {
    if (!scan_sizes_ok(B, H, T, dk, dv, chunk, dtype)) return 0;
    return plan_scan(B, H, T, dk, dv, chunk == 0 ? 64 : chunk, dtype).workspace_bytes;
}

// ------------------------------------------------------------ fixed scratch
// rodimus_scan_prefill_noalloc keeps the segment-parallel states in this
// array instead of a caller workspace.  34 MiB holds the largest segment plan
// of any prefill (33,684,480 bytes: B*H = 1, 256 segments of 2 sub-segments).
// Each device holds its own copy, from the first call on it until the process
// ends.  In host code the array's name is only a host-side stand-in: the
// kernels get its device address from scratch_on_current_device().
constexpr size_t kScratchBytes = (size_t)34 << 20;
static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// Device address of `scratch` on the current device, looked up once per
// device with that device current, then kept.
static int scratch_on_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return RODIMUS_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return RODIMUS_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return RODIMUS_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return RODIMUS_OK;
}

// The prefill behind both entry points.  With use_scratch, the segment states
// go to this device's fixed scratch array (looked up only once validation has
// passed and only if the plan needs it) instead of the caller's workspace.
static int scan_prefill_impl(const void *q, const void *k, const void *v, const void *g,
                             const void *tau, const float *S0, void *o, float *S_T,
                             int B, int H, int T, int dk, int dv, int chunk, int dtype,
                             void *workspace, size_t workspace_bytes, bool use_scratch, void *stream) {
    if (!scan_sizes_ok(B, H, T, dk, dv, chunk, dtype)) return RODIMUS_ERR_INVALID_ARG;
    if (!ok_opt_ptr(S0) || !ok_opt_ptr(S_T) || !ok_opt_ptr(workspace))
        return RODIMUS_ERR_INVALID_ARG;
    if (S0 && S_T && S0 == S_T) return RODIMUS_ERR_INVALID_ARG;
    if (chunk == 0) chunk = 64;
    hipStream_t st = (hipStream_t)stream;
    if (B == 0 || H == 0) return RODIMUS_OK;
    const size_t nstate = (size_t)B * H * dk * dv;
    if (T == 0) {
        if (S_T) {
            launch_state_copy(S0, S_T, nstate, st);
            return hip_status();
        }
        return RODIMUS_OK;
    }
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(g) || !ok_ptr(tau) || !ok_ptr(o))
        return RODIMUS_ERR_INVALID_ARG;
    ScanPlan plan = plan_scan(B, H, T, dk, dv, chunk, dtype);
    if (!scan_launch_fits(plan, B, H, T, chunk)) return RODIMUS_ERR_INVALID_ARG;
    if (use_scratch && plan.workspace_bytes > 0) {
        if (plan.workspace_bytes > kScratchBytes) return RODIMUS_ERR_TOO_LARGE;
        const int rc = scratch_on_current_device(&workspace);
        if (rc != RODIMUS_OK) return rc;
        workspace_bytes = kScratchBytes;
    }
    if (plan.workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.workspace_bytes))
        return RODIMUS_ERR_INVALID_ARG;
    ScanArgs a{q, k, v, g, tau, S0, o, S_T, B, H, T, dk, dv, chunk, dtype, workspace,
               workspace_bytes};
    if (plan.mfma) launch_scan_mfma(a, plan, st);
    else launch_scan_generic(a, st);
    return hip_status();
}

int rodimus_scan_prefill(const void *q, const void *k, const void *v, const void *g,
                         const void *tau, const float *S0, void *o, float *S_T,
                         int B, int H, int T, int dk, int dv, int chunk, int dtype,
                         void *workspace, size_t workspace_bytes, void *stream) {
    return scan_prefill_impl(q, k, v, g, tau, S0, o, S_T, B, H, T, dk, dv, chunk, dtype, workspace,
                             workspace_bytes, false, stream);
}

int rodimus_scan_prefill_noalloc(const void *q, const void *k, const void *v, const void *g,
                                 const void *tau, const float *S0, void *o, float *S_T,
                                 int B, int H, int T, int dk, int dv, int chunk, int dtype,
                                 void *stream) {
    return scan_prefill_impl(q, k, v, g, tau, S0, o, S_T, B, H, T, dk, dv, chunk, dtype, nullptr, 0,
                             true, stream);
}

int rodimus_scan_prefill_lowrank(const void *q, const void *k, const void *v, const void *zg,
                                 const void *zt, const void *Ug, const float *bg, const void *Ut,
                                 const float *bt, const float *S0, void *o, float *S_T, int B, int H,
                                 int T, int dk, int dv, int rank, int chunk, int dtype, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    if (!scan_sizes_ok(B, H, T, dk, dv, chunk, dtype) || rank <= 0) return RODIMUS_ERR_INVALID_ARG;
    if (!ok_opt_ptr(S0) || !ok_opt_ptr(S_T) || !ok_opt_ptr(workspace)) return RODIMUS_ERR_INVALID_ARG;
    if (S0 && S_T && S0 == S_T) return RODIMUS_ERR_INVALID_ARG;
    if (chunk == 0) chunk = 64;
    if (dtype != RODIMUS_BF16 || dk != 128 || dv != 128 || rank != 16 || (chunk != 32 && chunk != 64))
        return RODIMUS_ERR_UNSUPPORTED;
    if ((long long)T * 32 >= (1LL << 31)) return RODIMUS_ERR_UNSUPPORTED;
    hipStream_t st = (hipStream_t)stream;
    if (B == 0 || H == 0) return RODIMUS_OK;
    if (T == 0) {
        if (S_T) {
            launch_state_copy(S0, S_T, (size_t)B * H * dk * dv, st);
            return hip_status();
        }
        return RODIMUS_OK;
    }
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(zg) || !ok_ptr(zt) || !ok_ptr(Ug) || !ok_ptr(Ut) ||
        !ok_ptr(bg) || !ok_ptr(bt) || !ok_ptr(o))
        return RODIMUS_ERR_INVALID_ARG;
    ScanPlan plan = plan_scan(B, H, T, dk, dv, chunk, dtype);
    if (!plan.mfma) return RODIMUS_ERR_UNSUPPORTED;
    if (!scan_launch_fits(plan, B, H, T, chunk)) return RODIMUS_ERR_INVALID_ARG;
    if (plan.workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.workspace_bytes))
        return RODIMUS_ERR_INVALID_ARG;
    ScanArgs a{q, k, v, nullptr, nullptr, S0, o, S_T, B, H, T, dk, dv, chunk, dtype, workspace,
               workspace_bytes};
    a.zg = zg; a.zt = zt; a.Ug = Ug; a.Ut = Ut; a.bg = bg; a.bt = bt;
    launch_scan_mfma(a, plan, st);
    return hip_status();
}

size_t rodimus_scan_prefill_varlen_workspace_bytes(int N, int H, int max_seqlen, int dk, int dv,
                                                   int chunk, int dtype) {
    if (!scan_sizes_ok(N, H, max_seqlen, dk, dv, chunk, dtype)) return 0;
    return rodimus_scan_prefill_workspace_bytes(N, H, max_seqlen, dk, dv, chunk, dtype) + seq_order_bytes(N);
}

int rodimus_scan_prefill_varlen(const void *q, const void *k, const void *v, const void *g,
                                const void *tau, const float *S0, void *o, float *S_T,
                                const int *cu_seqlens, int N, int H, int total_T, int max_seqlen,
                                int dk, int dv, int chunk, int dtype, void *workspace,
                                size_t workspace_bytes, void *stream) {
    if (!scan_sizes_ok(N, H, max_seqlen, dk, dv, chunk, dtype) || total_T < 0)
        return RODIMUS_ERR_INVALID_ARG;
    if ((long long)H * total_T * (dk > dv ? dk : dv) > (1LL << 46)) return RODIMUS_ERR_INVALID_ARG;
    if (!ok_opt_ptr(S0) || !ok_opt_ptr(S_T) || !ok_opt_ptr(workspace)) return RODIMUS_ERR_INVALID_ARG;
    if (S0 && S_T && S0 == S_T) return RODIMUS_ERR_INVALID_ARG;
    if (chunk == 0) chunk = 64;
    hipStream_t st = (hipStream_t)stream;
    if (N == 0 || H == 0) return RODIMUS_OK;
    if (cu_seqlens == nullptr || ((uintptr_t)cu_seqlens & 3) != 0) return RODIMUS_ERR_INVALID_ARG;
    if (max_seqlen == 0 || total_T == 0) {  // every sequence is empty
        if (S_T) {
            launch_state_copy(S0, S_T, (size_t)N * H * dk * dv, st);
            return hip_status();
        }
        return RODIMUS_OK;
    }
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(g) || !ok_ptr(tau) || !ok_ptr(o))
        return RODIMUS_ERR_INVALID_ARG;
    ScanPlan plan = plan_scan(N, H, max_seqlen, dk, dv, chunk, dtype);
    if (!scan_launch_fits(plan, N, H, max_seqlen, chunk)) return RODIMUS_ERR_INVALID_ARG;
    const size_t need = plan.workspace_bytes + seq_order_bytes(N);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return RODIMUS_ERR_INVALID_ARG;
    ScanArgs a{q, k, v, g, tau, S0, o, S_T, N, H, max_seqlen, dk, dv, chunk, dtype, workspace,
               workspace_bytes};
    a.cu = cu_seqlens;
    a.total = total_T;
    if (plan.mfma && seq_order_bytes(N) > 0) {  // longest sequences first
        a.order = reinterpret_cast<int *>(static_cast<char *>(workspace) + plan.workspace_bytes);
        launch_seq_order(cu_seqlens, N, total_T, max_seqlen, a.order, st);
    }
    if (plan.mfma) launch_scan_mfma(a, plan, st);
    else launch_scan_generic(a, st);
    return hip_status();
}

size_t rodimus_scan_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int dtype) {
    if (!scan_sizes_ok(B, H, T, dk, dv, 0, dtype)) return 0;
    if (scan_bwd_mfma_supported(T, dk, dv, dtype)) return scan_bwd_mfma_workspace(B, H, T);
    return scan_bwd_workspace(B, H, T, dk, dv);
}

int rodimus_scan_backward(const void *q, const void *k, const void *v, const void *g,
                          const void *tau, const float *S0, const void *dO, const float *dS_T,
                          float *dq, float *dk_, float *dv_, float *dg, float *dtau, float *dS0,
                          int B, int H, int T, int dk, int dv, int dtype,
                          void *workspace, size_t workspace_bytes, void *stream) {
    if (!scan_sizes_ok(B, H, T, dk, dv, 0, dtype)) return RODIMUS_ERR_INVALID_ARG;
    if (!ok_opt_ptr(S0) || !ok_opt_ptr(dS_T) || !ok_opt_ptr(dS0) || !ok_opt_ptr(workspace))
        return RODIMUS_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    if (B == 0 || H == 0) return RODIMUS_OK;
    const size_t nstate = (size_t)B * H * dk * dv;
    if (T == 0) {  // nothing but the final-state gradient flows back to S0
        if (dS0) {
            launch_state_copy(dS_T, dS0, nstate, st);
            return hip_status();
        }
        return RODIMUS_OK;
    }
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(g) || !ok_ptr(tau) || !ok_ptr(dO) ||
        !ok_ptr(dq) || !ok_ptr(dk_) || !ok_ptr(dv_) || !ok_ptr(dg) || !ok_ptr(dtau))
        return RODIMUS_ERR_INVALID_ARG;
    const bool mfma = scan_bwd_mfma_supported(T, dk, dv, dtype);
    if (!scan_bwd_launch_fits(mfma, B, H, T)) return RODIMUS_ERR_INVALID_ARG;
    const size_t need = mfma ? scan_bwd_mfma_workspace(B, H, T) : scan_bwd_workspace(B, H, T, dk, dv);
    if (workspace == nullptr || workspace_bytes < need) return RODIMUS_ERR_INVALID_ARG;
    ScanBwdArgs a{q, k, v, g, tau, S0, dO, dS_T, dq, dk_, dv_, dg, dtau, dS0, B, H, T, dk, dv, dtype,
                  workspace};
    if (mfma) launch_scan_bwd_mfma(a, st);
    else launch_scan_bwd(a, st);
    return hip_status();
}

size_t rodimus_scan_backward_varlen_workspace_bytes(int N, int H, int max_seqlen, int dk, int dv, int dtype) {
    if (!scan_sizes_ok(N, H, max_seqlen, dk, dv, 0, dtype)) return 0;
    return rodimus_scan_backward_workspace_bytes(N, H, max_seqlen, dk, dv, dtype) + seq_order_bytes(N);
}

int rodimus_scan_backward_varlen(const void *q, const void *k, const void *v, const void *g,
                                 const void *tau, const float *S0, const void *dO, const float *dS_T,
                                 float *dq, float *dk_, float *dv_, float *dg, float *dtau, float *dS0,
                                 const int *cu_seqlens, int N, int H, int total_T, int max_seqlen,
                                 int dk, int dv, int dtype, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    if (!scan_sizes_ok(N, H, max_seqlen, dk, dv, 0, dtype) || total_T < 0) return RODIMUS_ERR_INVALID_ARG;
    if ((long long)H * total_T * (dk > dv ? dk : dv) > (1LL << 46)) return RODIMUS_ERR_INVALID_ARG;
    if (!ok_opt_ptr(S0) || !ok_opt_ptr(dS_T) || !ok_opt_ptr(dS0) || !ok_opt_ptr(workspace))
        return RODIMUS_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    if (N == 0 || H == 0) return RODIMUS_OK;
    if (cu_seqlens == nullptr || ((uintptr_t)cu_seqlens & 3) != 0) return RODIMUS_ERR_INVALID_ARG;
    if (max_seqlen == 0 || total_T == 0) {  // every sequence is empty
        if (dS0) {
            launch_state_copy(dS_T, dS0, (size_t)N * H * dk * dv, st);
            return hip_status();
        }
        return RODIMUS_OK;
    }
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(g) || !ok_ptr(tau) || !ok_ptr(dO) ||
        !ok_ptr(dq) || !ok_ptr(dk_) || !ok_ptr(dv_) || !ok_ptr(dg) || !ok_ptr(dtau))
        return RODIMUS_ERR_INVALID_ARG;
    const bool mfma = scan_bwd_mfma_supported(max_seqlen, dk, dv, dtype);
    if (!scan_bwd_launch_fits(mfma, N, H, max_seqlen)) return RODIMUS_ERR_INVALID_ARG;
    const size_t base = mfma ? scan_bwd_mfma_workspace(N, H, max_seqlen) : scan_bwd_workspace(N, H, max_seqlen, dk, dv);
    if (workspace == nullptr || workspace_bytes < base + seq_order_bytes(N)) return RODIMUS_ERR_INVALID_ARG;
    ScanBwdArgs a{q, k, v, g, tau, S0, dO, dS_T, dq, dk_, dv_, dg, dtau, dS0, N, H, max_seqlen, dk, dv, dtype,
                  workspace};
    a.cu = cu_seqlens;
    a.total = total_T;
    if (mfma && seq_order_bytes(N) > 0) {  // longest sequences first
        a.order = reinterpret_cast<int *>(static_cast<char *>(workspace) + base);
        launch_seq_order(cu_seqlens, N, total_T, max_seqlen, a.order, st);
    }
    if (mfma) launch_scan_bwd_mfma(a, st);
    else launch_scan_bwd(a, st);
    return hip_status();
}

int rodimus_decode_step(const void *q, const void *k, const void *v, const void *g,
                        const void *tau, const float *S_in, float *S_out, void *o,
                        int N, int H, int dk, int dv, int dtype, void *stream) {
    if (N < 0 || H < 0 || !ok_head_dim(dk) || !ok_head_dim(dv) || !ok_dtype(dtype))
        return RODIMUS_ERR_INVALID_ARG;
    // one workgroup of up to 256 threads per (sequence, head): N*H < 2^24
    if (decode_launch_items((long long)N * H) >= kMaxLaunchItems) return RODIMUS_ERR_INVALID_ARG;
    if (N == 0 || H == 0) return RODIMUS_OK;
    if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v) || !ok_ptr(g) || !ok_ptr(tau) || !ok_ptr(S_in) ||
        !ok_ptr(S_out) || !ok_ptr(o))
        return RODIMUS_ERR_INVALID_ARG;
    // S_out must equal S_in or not overlap it at all.
    const size_t sbytes = (size_t)N * H * dk * dv * sizeof(float);
    const char *a0 = (const char *)S_in, *b0 = (const char *)S_out;
    if (a0 != b0 && a0 < b0 + sbytes && b0 < a0 + sbytes) return RODIMUS_ERR_INVALID_ARG;
    DecodeArgs a{q, k, v, g, tau, S_in, S_out, o, N, H, dk, dv, dtype};
    launch_decode_step(a, (hipStream_t)stream);
    return hip_status();
}

int sw_ska_attn(const void *q, const void *k_shared, const void *v, void *o,
                int B, int H, int T, int dk, int dv, int window, float scale, int dtype,
                void *stream) {
    if (B < 0 || H < 0 || T < 0 || window < 1 || !ok_head_dim(dk) || !ok_head_dim(dv) ||
        !ok_dtype(dtype))
        return RODIMUS_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !(scale < 3.0e38f)) return RODIMUS_ERR_INVALID_ARG;
    if ((long long)B * H * T * (dk > dv ? dk : dv) > (1LL << 46)) return RODIMUS_ERR_INVALID_ARG;
    if (!swska_supported(T, dk, dv, dtype)) return RODIMUS_ERR_UNSUPPORTED;
    if (swska_launch_items((long long)B * H, T, dk) >= kMaxLaunchItems) return RODIMUS_ERR_INVALID_ARG;
    if (B == 0 || H == 0 || T == 0) return RODIMUS_OK;
    if (!ok_ptr(q) || !ok_ptr(k_shared) || !ok_ptr(v) || !ok_ptr(o)) return RODIMUS_ERR_INVALID_ARG;
    SkaArgs a{q, k_shared, v, o, B, H, T, dk, dv, window, scale, dtype};
    launch_swska(a, (hipStream_t)stream);
    return hip_status();
}

static bool ska_decode_sizes_ok(int N, int H, int dk, int dv, int window, int dtype) {
    if (N < 0 || H < 0 || window < 1 || window > (1 << 19)) return false;
    if (!ok_head_dim(dk) || !ok_head_dim(dv) || !ok_dtype(dtype)) return false;
    // grids (below 2^32 work-items per launch) and element counts must fit the
    // kernels' index arithmetic
    if ((long long)N * H >= (1LL << 24) || swska_decode_blocks(N, H, window) >= (1u << 24)) return false;
    if ((long long)N * H * window * (dk > dv ? dk : dv) > (1LL << 46)) return false;
    return true;
}

size_t sw_ska_decode_workspace_bytes(int N, int H, int dk, int dv, int window, int dtype) {
    if (!ska_decode_sizes_ok(N, H, dk, dv, window, dtype) || !swska_decode_supported(dk, dv, dtype))
        return 0;
    return swska_decode_workspace(N, H, dv, window);
}

int sw_ska_decode_step(const void *q, const void *k_new, const void *v_new, void *k_cache,
                       void *v_cache, int *pos, void *o, int N, int H, int dk, int dv, int window,
                       float scale, int dtype, void *workspace, size_t workspace_bytes, void *stream) {
    if (!ska_decode_sizes_ok(N, H, dk, dv, window, dtype)) return RODIMUS_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !(scale < 3.0e38f)) return RODIMUS_ERR_INVALID_ARG;
    if (!swska_decode_supported(dk, dv, dtype)) return RODIMUS_ERR_UNSUPPORTED;
    if (N == 0 || H == 0) return RODIMUS_OK;
    if (!ok_ptr(q) || !ok_ptr(k_new) || !ok_ptr(v_new) || !ok_ptr(k_cache) || !ok_ptr(v_cache) ||
        !ok_ptr(o) || pos == nullptr || ((uintptr_t)pos & 3) != 0)
        return RODIMUS_ERR_INVALID_ARG;
    const size_t need = swska_decode_workspace(N, H, dv, window);
    if (!ok_ptr(workspace) || workspace_bytes < need) return RODIMUS_ERR_INVALID_ARG;
    SkaDecArgs a{q, k_new, v_new, k_cache, v_cache, pos, o, N, H, dk, dv, window, scale, dtype, workspace};
    launch_swska_decode(a, (hipStream_t)stream);
    return hip_status();
}

}  // extern "C"
