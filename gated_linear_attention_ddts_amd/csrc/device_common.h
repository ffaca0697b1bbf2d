// device_common.h -- device helpers shared by the gfx950 kernels of librodimus.
//
// Element types: fp32 inputs are `float`; bf16 inputs are raw 16-bit patterns
// held as `unsigned short` (conversion to float is exact; conversion from
// float rounds to nearest even through the hardware v_cvt_pk_bf16_f32).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rodimus {

typedef unsigned short bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf2f(bf16_t u) { return __uint_as_float((uint32_t)u << 16); }

__device__ __forceinline__ bf16_t f2bf(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(bf16_t, b);
}

// Generic element load/store for the two input types.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float ld(const float *p, size_t i) { return p[i]; }
    static __device__ __forceinline__ void st(float *p, size_t i, float x) { p[i] = x; }
};
template <> struct Elem<bf16_t> {
    static __device__ __forceinline__ float ld(const bf16_t *p, size_t i) { return bf2f(p[i]); }
    static __device__ __forceinline__ void st(bf16_t *p, size_t i, float x) { p[i] = f2bf(x); }
};

// Fast base-2 exponent / logarithm (single v_exp_f32 / v_log_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// DDTS gate map in natural-log units:
//   tau = sigmoid(theta),  L = log1p(exp(-|g|)),
//   log a    = -tau * (max(-g, 0) + L)    = -tau * softplus(-g)
//   log beta = -tau * (max( g, 0) + L)    = -tau * softplus( g)
// theta = -inf gives tau = 0 exactly (a = beta = 1).  log1p is evaluated as
// log(u) * x / (u - 1) with u = 1 + x (exact when u == 1), which keeps the
// relative error of L near one ulp for small x.
__device__ __forceinline__ void ddts_log_gates(float g, float theta, float &la, float &lb) {
    float et = exp2_fast(-fabsf(theta) * kLog2e);         // e^{-|theta|} in (0, 1]
    float tau = (theta >= 0.f ? 1.f : et) * __builtin_amdgcn_rcpf(1.f + et);
    float x = exp2_fast(-fabsf(g) * kLog2e);              // e^{-|g|} in (0, 1]
    float u = 1.f + x;
    float L = (u == 1.f) ? x : log2_fast(u) * kLn2 * (x / (u - 1.f));
    la = -tau * (fmaxf(-g, 0.f) + L);
    lb = -tau * (fmaxf(g, 0.f) + L);
}

// Same gate map in base-2 units (log2 a, log2 beta), for kernels that feed
// v_exp_f32 directly.
__device__ __forceinline__ void ddts_log2_gates(float g, float theta, float &l2a, float &l2b) {
    float et = exp2_fast(-fabsf(theta) * kLog2e);
    float tau = (theta >= 0.f ? 1.f : et) * __builtin_amdgcn_rcpf(1.f + et);
    float x = exp2_fast(-fabsf(g) * kLog2e);
    float u = 1.f + x;
    float L2 = (u == 1.f) ? x * kLog2e : log2_fast(u) * (x / (u - 1.f));
    l2a = -tau * (fmaxf(-g, 0.f) * kLog2e + L2);
    l2b = -tau * (fmaxf(g, 0.f) * kLog2e + L2);
}

// Cheaper base-2 gate map for the bf16 MFMA path (no division, no select):
//   tau = 1 / (1 + 2^{-theta log2 e})   (theta = -inf -> 1/inf = 0, +inf -> 1)
//   L2  = log2(1 + 2^{-|g| log2 e})     (absolute error ~2^-24; relative error of
//                                         small L2 grows as |g| grows, which stays
//                                         far below the bf16 operand rounding)
//   log2 a = -tau (max(-g,0) log2 e + L2),   log2 beta = -tau (max(g,0) log2 e + L2)
__device__ __forceinline__ void ddts_log2_gates_fast(float g, float theta, float &l2a, float &l2b) {
    const float tau = __builtin_amdgcn_rcpf(1.f + exp2_fast(-theta * kLog2e));
    const float L2 = log2_fast(1.f + exp2_fast(-fabsf(g) * kLog2e));
    l2a = -tau * fmaf(fmaxf(-g, 0.f), kLog2e, L2);
    l2b = -tau * fmaf(fmaxf(g, 0.f), kLog2e, L2);
}

__device__ __forceinline__ bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// Streaming stores for results written in whole cache lines that this call
// never reads back (the decode state written for the next step, the fp32
// gradients, the backward's checkpoints, read back by the next kernel from
// HBM anyway).  The non-temporal hint raises the decode step's sustained HBM
// rate from 6.1 to 6.7 TB/s.  It is not used for stores that leave a line
// partly written per instruction (the bf16 outputs written 8 bytes per lane):
// there it made the prefill 65% slower.
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_stream(float *p, float x) { __builtin_nontemporal_store(x, p); }
__device__ __forceinline__ void st_stream(float4 *p, const float4 &x) {
    __builtin_nontemporal_store(f32x4_nt{x.x, x.y, x.z, x.w}, reinterpret_cast<f32x4_nt *>(p));
}
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_stream(bf16x8_t *p, const bf16x8_t &x) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_nt, x), reinterpret_cast<u32x4_nt *>(p));
}

// Sequence-head handled by the workgroup in dispatch slot bh = pos * H + h of
// a packed batch: the sequence at position pos of the longest-first order
// (order null: table order).  bh must be wave-uniform; so is the result.
__device__ __forceinline__ int seq_head(const int *order, int H, int bh) {
    if (order == nullptr) return bh;
    const int pos = bh / H;
    return __builtin_amdgcn_readfirstlane(order[pos]) * H + (bh - pos * H);
}

}  // namespace rodimus
