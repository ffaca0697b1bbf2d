/*
 * rodimus.h -- C ABI of the MI355X (gfx950) Rodimus* token-mixer library
 *              (librodimus.so).
 *
 * The library computes the operations of the Rodimus* token mixer, each in
 * hand-written HIP kernels launched asynchronously on the caller's stream:
 *
 *  rodimus_scan_prefill  the DDTS-gated linear-attention recurrence over a
 *                        whole prompt, in chunkwise-parallel form (also over
 *                        a packed batch of ragged sequences, _varlen, and with
 *                        the gate logits expanded in-kernel from low-rank
 *                        factors, _lowrank);
 *  rodimus_scan_backward its gradients with respect to every input (also
 *                        over the packed batch, _varlen);
 *  rodimus_decode_step   one recurrent step on a resident fixed-size state;
 *  sw_ska_attn           sliding-window attention with one key matrix shared
 *                        by all heads (SW-SKA), over a whole sequence;
 *  sw_ska_decode_step    one SW-SKA token per sequence over ring-buffer
 *                        window caches.
 *
 * Sources.  The Rodimus block paragraph of "ICLR 2025 | Rodimus*: ..."
 * (CodeFuse article) describes the recurrent state with a selection gate, a
 * temperature gate and an input gate, trained chunkwise in parallel with
 * sub-quadratic cost and run at inference with an O(1)-size state; the page
 * does not print the formula.  This library computes, per (batch b, head h),
 * with S in R^{dk x dv} (rows = key channels):
 *
 *     log a_t    = -sigmoid(tau_t) * softplus(-g_t)          (per key channel)
 *     log beta_t = -sigmoid(tau_t) * softplus( g_t)
 *     S_t = diag(a_t) S_{t-1} + (beta_t * k_t)^T v_t,        o_t = q_t S_t
 *
 * i.e. a = s^T, beta = (1 - s)^T with selection s = sigmoid(g) and temperature
 * T = sigmoid(tau); tau = 0 gives the tempered_gate_init of 0.5 listed in the
 * module configuration (section 3 of the Rodimus* deployment blog,
 * m.nxbn.cn/news/205411).  SW-SKA follows the SKA / Rodimus+ paragraphs and
 * Fig. 4 of the CodeFuse article (keys shared across heads, values per head),
 * with softmax(q k^T * scale) v (MiniCPM-SALA blog, wzjinhao.cn/news/68323,
 * section 1.1) restricted to the previous `window` keys including the query's
 * own position (same blog, section 2.1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All pointers are DEVICE pointers (hipMalloc'd or equivalent) owned by the
 *    caller; the library keeps no pointer after the call returns and
 *    allocates nothing.  Its only global state is the fixed scratch array of
 *    rodimus_scan_prefill_noalloc and that array's address per device; every
 *    other entry point is thread-safe.
 *  - Tensors are contiguous, row-major, 16-byte aligned.
 *  - dtype selects the element type of q, k, v, g, tau and o:
 *    RODIMUS_F32 (float) or RODIMUS_BF16 (bfloat16 bit patterns).  Recurrent
 *    states are always float.  Internal arithmetic is fp32 (MFMA operands
 *    bf16 with fp32 accumulation on the bf16 path); o is rounded to nearest
 *    even.
 *  - stream is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work; nothing is synchronised inside the library.
 *  - ABI types: `int dtype` carries a rodimus_dtype value and `void *stream` a
 *    hipStream_t.  Both are passed as plain C types so that this header needs
 *    no HIP header and binds from any FFI; they are the same width and
 *    calling convention as the enum and the pointer typedef they stand for.
 *  - Arguments are validated before any HIP call.  On a non-OK return nothing
 *    has been launched, except RODIMUS_ERR_HIP (a launch error reported by the
 *    runtime).  No exception crosses the ABI.
 *  - Launch size: HIP refuses a launch of 2^32 work-items or more.  Every
 *    entry point computes the largest launch its arguments need and returns
 *    RODIMUS_ERR_INVALID_ARG (nothing launched) if it would reach that limit;
 *    the limits are stated per entry point below.
 *  - Inputs must be finite, except tau = -inf, which is defined (a = beta = 1).
 */
#ifndef RODIMUS_H
#define RODIMUS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RODIMUS_OK = 0,
    RODIMUS_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size, small workspace */
    RODIMUS_ERR_UNSUPPORTED = -2, /* valid but outside the compiled kernel set */
    RODIMUS_ERR_HIP = -3,         /* the HIP runtime reported an error */
    RODIMUS_ERR_TOO_LARGE = -4    /* needs more scratch than rodimus_scan_prefill_noalloc's fixed buffer */
} rodimus_status;

typedef enum { RODIMUS_F32 = 0, RODIMUS_BF16 = 1 } rodimus_dtype;

/*
 * Bytes of device workspace rodimus_scan_prefill needs for these arguments
 * (0 when it needs none).  The segment-parallel path used when B*H is too
 * small to fill the GPU keeps, per segment boundary and (b,h), a float state
 * [dk x dv] and a float log-decay vector [dk].  Returns 0 for arguments that
 * rodimus_scan_prefill would reject.
 */
size_t rodimus_scan_prefill_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk,
                                            int dtype);

/*
 * Chunkwise-parallel prefill of the recurrence above (CodeFuse article,
 * Rodimus block paragraph: chunkwise-parallel training/prefill form).
 *
 *   q, k, g, tau : [B, H, T, dk]      v, o : [B, H, T, dv]     (dtype)
 *   S0           : [B, H, dk, dv] float, the state before token 0;
 *                  NULL means zeros.
 *   S_T          : [B, H, dk, dv] float, receives the state after token T-1;
 *                  NULL skips it.  May not alias S0.
 *   chunk        : C in {16, 32, 64}, or 0 for 64.  The result does not depend
 *                  on C beyond rounding.  Paths: bf16 with dk = dv = 128 and
 *                  C in {32, 64} runs on the matrix cores; every other
 *                  combination (fp32, other head sizes, and C = 16 at any
 *                  dtype) runs the fp32 vector-unit chunked kernel, one
 *                  64-lane wave per (b,h) and 64 value columns, which at the
 *                  1.6B shape is an order of magnitude slower.  C = 16 exists
 *                  for small head sizes and parity checks, not for speed.
 *   workspace    : device scratch of at least
 *                  rodimus_scan_prefill_workspace_bytes(...) bytes (may be
 *                  NULL when that is 0).  Its contents are overwritten.
 *
 * Sizes: B, H, T >= 0 (T = 0 copies S0, or zeros, to S_T); dk, dv multiples
 * of 16 in [16, 128]; B*H <= 2^30 and B*H*T*max(dk,dv) <= 2^46.  Launch size:
 * the matrix-core path launches one 512-thread workgroup per (b,h) and
 * segment (B*H < 2^23 once B*H >= 256), the vector path one 64-thread wave per
 * (b,h) (B*H < 2^26).  A too-small workspace or a size beyond these gives
 * RODIMUS_ERR_INVALID_ARG.
 */
int rodimus_scan_prefill(const void *q, const void *k, const void *v, const void *g,
                         const void *tau, const float *S0, void *o, float *S_T,
                         int B, int H, int T, int dk, int dv, int chunk, int dtype,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * rodimus_scan_prefill with the gate logits produced inside the kernels from
 * low-rank factors, so that g and tau ([B,H,T,dk] each, a third of the
 * prefill's input bytes) never pass through device memory.  The CodeFuse
 * article's Rodimus block paragraph computes the selection and temperature
 * gates from the token through learnable weights, and the module
 * configuration in section 3 of the Rodimus* deployment blog names SiLU as
 * the selection gate's activation; neither page prints the projection.  The
 * reading computed here: each token's hidden state is projected (outside this
 * library, e.g. as extra output columns of the q/k/v projection) to two
 * rank-R factor rows z_g, z_tau shared by all heads, and per head h and key
 * channel c
 *
 *     g[b,h,t,c]   = sum_r silu(z_g[b,t,r]) * U_g[h,c,r]   + b_g[h,c]
 *     tau[b,h,t,c] = sum_r      z_tau[b,t,r] * U_tau[h,c,r] + b_tau[h,c]
 *
 * then exactly the recurrence of rodimus_scan_prefill.
 *
 *   q, k : [B, H, T, dk]    v, o : [B, H, T, dv]         (bf16)
 *   zg, zt : [B, T, rank]   the factor rows z_g, z_tau   (bf16)
 *   Ug, Ut : [H, dk, rank]  per-head up-projections      (bf16)
 *   bg, bt : [H, dk]        per-head biases              (float)
 *   S0, S_T, chunk, workspace: as for rodimus_scan_prefill, with the same
 *   workspace size (rodimus_scan_prefill_workspace_bytes with the same B, H,
 *   T, dk, dv, chunk and dtype).
 *
 * Precision: silu(z_g) is rounded to bf16 (the operand precision of this
 * path) and each logit is accumulated in fp32; everything after that is the
 * bf16 matrix-core prefill.  Supported: RODIMUS_BF16, dk = dv = 128,
 * rank = 16, chunk in {32, 64} (0 = 64), T < 2^23 (else
 * RODIMUS_ERR_UNSUPPORTED; rank <= 0 is RODIMUS_ERR_INVALID_ARG).  Every
 * pointer except S0, S_T and a NULL workspace must be 16-byte aligned and
 * non-NULL.  Other rules, launch limits and errors as for rodimus_scan_prefill.
 */
int rodimus_scan_prefill_lowrank(const void *q, const void *k, const void *v, const void *zg,
                                 const void *zt, const void *Ug, const float *bg, const void *Ut,
                                 const float *bt, const float *S0, void *o, float *S_T, int B, int H,
                                 int T, int dk, int dv, int rank, int chunk, int dtype, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * rodimus_scan_prefill without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, results (bit for bit)
 * and kernels as rodimus_scan_prefill, except that the segment-parallel
 * states live in a fixed array inside the library instead of a caller
 * workspace: 34 MiB of device memory per GPU, held from the first call on that
 * GPU until the process ends.  It is large enough for every prefill the
 * library accepts (the largest segment plan needs 33,684,480 bytes);
 * a plan beyond it would return RODIMUS_ERR_TOO_LARGE.  The call itself
 * allocates nothing (no hipMalloc, hipFree or allocating library routine);
 * its first call on a GPU looks up the array's device address there
 * (hipGetSymbolAddress, current device).  The caller passes inputs and
 * outputs as for rodimus_scan_prefill.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (the kernels write every element they read, so nothing needs
 * clearing): calls that may overlap on one GPU -- on different streams, or
 * from several host threads -- race and must be serialised by the caller.
 */
int rodimus_scan_prefill_noalloc(const void *q, const void *k, const void *v, const void *g,
                                 const void *tau, const float *S0, void *o, float *S_T,
                                 int B, int H, int T, int dk, int dv, int chunk, int dtype,
                                 void *stream);

/*
 * rodimus_scan_prefill over a packed batch of sequences of different lengths
 * (dynamic batching of short requests, each with its own small fixed-size
 * state: the Tupoi O(1)-memory practice guide, pwwt.cn/news/4131393,
 * section 4.2 on batching and resource management).  Per head, the N
 * sequences are concatenated:
 *
 *   q, k, g, tau : [H, total_T, dk]     v, o : [H, total_T, dv]   (dtype)
 *   cu_seqlens   : int32 [N + 1], device; sequence s occupies rows
 *                  cu_seqlens[s] .. cu_seqlens[s+1]-1 of every head
 *                  (non-decreasing, cu_seqlens[0] = 0, cu_seqlens[N] = total_T)
 *   S0, S_T      : [N, H, dk, dv] float, optional as in rodimus_scan_prefill
 *   max_seqlen   : at least the longest sequence; it sizes the segment plan
 *                  and the workspace (query with the _workspace_bytes call)
 *
 * The workspace also holds the order in which the sequences are processed
 * (longest first, computed on the device from the table: ranked by length up
 * to 4096 sequences, by 64-token chunk count beyond), so that long requests
 * do not start last; it never changes the results.
 *
 * Each sequence gives exactly what rodimus_scan_prefill gives for it alone
 * (same arithmetic; bitwise equal to a batched call of equal-length
 * sequences).  The table is read on the device only: the kernels clamp each
 * span to [0, total_T] and to max_seqlen, so a malformed table yields wrong
 * values but no access outside the tensors; rows of o that no span covers
 * are left untouched.  Sizes: N, H, total_T, max_seqlen >= 0; cu_seqlens
 * 4-byte aligned and non-NULL when N, H > 0; other rules as for
 * rodimus_scan_prefill.  max_seqlen = 0 or total_T = 0 copies S0 (or zeros)
 * to S_T.
 */
size_t rodimus_scan_prefill_varlen_workspace_bytes(int N, int H, int max_seqlen, int dk, int dv,
                                                   int chunk, int dtype);
int rodimus_scan_prefill_varlen(const void *q, const void *k, const void *v, const void *g,
                                const void *tau, const float *S0, void *o, float *S_T,
                                const int *cu_seqlens, int N, int H, int total_T, int max_seqlen,
                                int dk, int dv, int chunk, int dtype, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Backward of rodimus_scan_prefill: the gradients of
 *     L = sum(dO * o) + sum(dS_T * S_T)
 * with respect to q, k, v, g, tau and S0, for the same recurrence and gate map
 * (reverse-mode through the chunkwise form that the CodeFuse article's Rodimus
 * block paragraph trains with).  Inputs as for rodimus_scan_prefill, plus
 *   dO   : [B, H, T, dv] in the input dtype
 *   dS_T : [B, H, dk, dv] fp32, or NULL (no gradient of the final state)
 * Outputs, all fp32 and caller-allocated:
 *   grad_q, grad_k, grad_g, grad_tau : [B, H, T, dk]    grad_v : [B, H, T, dv]
 *   grad_S0 : [B, H, dk, dv], or NULL (not returned)
 * S0 NULL means zeros, as in the forward.  Supported: fp32 or bf16 inputs,
 * dk and dv multiples of 16 up to 128 (else RODIMUS_ERR_INVALID_ARG).
 * Launch size: the matrix-core path launches 8 work-items per token-head in
 * its gradient kernel (B*H*T < 2^29), the vector path 8 per token-head too
 * (256 threads per 32-token chunk); beyond that RODIMUS_ERR_INVALID_ARG.
 * Two paths, chosen from the arguments:
 *   - bf16 with dk = dv = 128: matrix cores (bf16 operands, fp32
 *     accumulation, bf16 checkpoints of the state and its gradient every 32
 *     tokens); same accuracy class as the bf16 forward;
 *   - otherwise: fp32 vector arithmetic over 32-token chunks with fp32
 *     checkpoints (workspace 2*B*H*ceil(T/32)*dk*dv fp32).
 * `workspace` must hold rodimus_scan_backward_workspace_bytes(...) bytes, else
 * RODIMUS_ERR_INVALID_ARG; its contents are overwritten (on the matrix-core
 * path: about 65 KiB per (b,h) per 32 tokens, plus per-segment edges and a
 * fixed 32 MiB).  T = 0 copies dS_T (or zeros) into grad_S0.  Calls that
 * share one workspace must not overlap.
 */
size_t rodimus_scan_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int dtype);
int rodimus_scan_backward(const void *q, const void *k, const void *v, const void *g,
                          const void *tau, const float *S0, const void *dO, const float *dS_T,
                          float *grad_q, float *grad_k, float *grad_v, float *grad_g,
                          float *grad_tau, float *grad_S0,
                          int B, int H, int T, int dk, int dv, int dtype,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * rodimus_scan_backward over the packed batch of rodimus_scan_prefill_varlen
 * (dynamic batching of short requests, Tupoi O(1)-memory practice guide,
 * pwwt.cn/news/4131393, section 4.2; trained chunkwise as in the CodeFuse
 * article's Rodimus block paragraph).  Layouts as for the packed prefill:
 *
 *   q, k, g, tau : [H, total_T, dk]     v, dO : [H, total_T, dv]   (dtype)
 *   grad_q, grad_k, grad_g, grad_tau : [H, total_T, dk]   grad_v : [H, total_T, dv]
 *                  (fp32, caller-allocated)
 *   cu_seqlens   : int32 [N + 1], device, as for rodimus_scan_prefill_varlen
 *   S0, dS_T, grad_S0 : [N, H, dk, dv] float, each optional (NULL) as in
 *                  rodimus_scan_backward
 *   max_seqlen   : at least the longest sequence; it sizes the plan, the
 *                  workspace (rodimus_scan_backward_varlen_workspace_bytes) and
 *                  selects the path exactly as T does for rodimus_scan_backward
 *
 * As for the packed prefill, the workspace also holds the longest-first order
 * of the sequences, which never changes the results.
 *
 * Each sequence gets exactly the gradients that rodimus_scan_backward gives
 * for it alone (bitwise equal to a batched call of equal-length sequences).
 * The table is read on the device only; each span is clamped to [0, total_T]
 * and to max_seqlen, so a malformed table yields wrong values but no access
 * outside the tensors.  Gradient rows that no span covers are left untouched.
 * An empty sequence gets grad_S0 = dS_T (or zeros).  Sizes: N, H, total_T,
 * max_seqlen >= 0; cu_seqlens 4-byte aligned and non-NULL when N, H > 0;
 * max_seqlen = 0 or total_T = 0 copies dS_T (or zeros) into grad_S0; other
 * rules as for rodimus_scan_backward.
 */
size_t rodimus_scan_backward_varlen_workspace_bytes(int N, int H, int max_seqlen, int dk, int dv,
                                                    int dtype);
int rodimus_scan_backward_varlen(const void *q, const void *k, const void *v, const void *g,
                                 const void *tau, const float *S0, const void *dO, const float *dS_T,
                                 float *grad_q, float *grad_k, float *grad_v, float *grad_g,
                                 float *grad_tau, float *grad_S0, const int *cu_seqlens, int N, int H,
                                 int total_T, int max_seqlen, int dk, int dv, int dtype,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * One recurrent (decode) step for N independent sequences (CodeFuse article,
 * Rodimus block paragraph: O(1)-size state at inference; the state stays
 * resident and is updated in place, MiniCPM-SALA blog section 3.3):
 *
 *   S' = diag(a) S + (beta * k)^T v,   o = q S'
 *
 *   q, k, g, tau : [N, H, dk]   v, o : [N, H, dv]   (dtype)
 *   S_in, S_out  : [N, H, dk, dv] float; S_out may equal S_in (in place) but
 *                  must not partially overlap it.
 *
 * Sizes: N, H >= 0; dk, dv multiples of 16 in [16, 128]; N*H < 2^24 (one
 * workgroup of up to 256 threads per sequence and head), else
 * RODIMUS_ERR_INVALID_ARG.
 */
int rodimus_decode_step(const void *q, const void *k, const void *v, const void *g,
                        const void *tau, const float *S_in, float *S_out, void *o,
                        int N, int H, int dk, int dv, int dtype, void *stream);

/*
 * Sliding-window shared-key attention (CodeFuse article, SKA and Rodimus+
 * paragraphs, Fig. 4; window semantics from the MiniCPM-SALA blog, sections
 * 1.1 and 2.1):
 *
 *   o[b,h,t] = sum_{s=max(0,t-window+1)}^{t} softmax_s(scale * q[b,h,t].k[b,s]) v[b,h,s]
 *
 *   q : [B, H, T, dk]   k_shared : [B, T, dk]   v, o : [B, H, T, dv]
 *   scale : usually 1/sqrt(dk); must be finite and > 0.
 *   window >= 1 (window >= T is causal attention over the whole prefix).
 *
 * No rotary embedding is applied: pass rotated q and k.  Supported:
 * RODIMUS_BF16 with dk = dv = 128 or dk = dv = 64, and T * dk * 2 < 2^31
 * (T <= 8388607 at dk = 128, T <= 16777215 at dk = 64); other combinations
 * return RODIMUS_ERR_UNSUPPORTED.  B, H, T >= 0.  Launch size: one workgroup
 * per (b,h) and block of 256 queries (512 threads; at dk = 64, 128 queries
 * and 256 threads), i.e. 2 work-items per query row: B*H*T below about
 * 2^31, else RODIMUS_ERR_INVALID_ARG.
 */
int sw_ska_attn(const void *q, const void *k_shared, const void *v, void *o,
                int B, int H, int T, int dk, int dv, int window, float scale, int dtype,
                void *stream);

/*
 * One decode step of SW-SKA for N independent sequences over ring-buffer
 * window caches (the KV cache that sharing the key shrinks: CodeFuse article,
 * SKA / Rodimus+ paragraphs and Fig. 4; window semantics as sw_ska_attn).
 *
 *   q     : [N, H, dk]   the new token's per-head queries
 *   k_new : [N, dk]      its key (shared by the heads)
 *   v_new : [N, H, dv]   its per-head values
 *   k_cache : [N, window, dk]      v_cache : [N, H, window, dv]
 *   pos   : [N] int32, device     tokens each sequence has seen (>= 0)
 *   o     : [N, H, dv]
 *
 * Position p of a sequence lives in slot p mod window of both caches.  With
 * t = pos[n], the step writes k_new / v_new into slot t mod window, computes
 *
 *   o[n,h] = sum_{s=max(0,t-window+1)}^{t} softmax_s(scale * q[n,h].k_s) v[n,h,s]
 *
 * (row t of sw_ska_attn over the sequence), and then increments pos[n]; all
 * in stream order.  Slots that hold no position of the window (t + 1 <
 * window) are never read.  A negative pos is treated as 0.
 *
 * Work split: the window is cut into splits of 256 slots, or of 1024 slots
 * when that still leaves at least 8 split workgroups per compute unit; a
 * split workgroup (256 threads) serves two heads when H is even, else one,
 * and a second kernel merges the splits' partial softmax results.
 *
 * Supported: RODIMUS_BF16 with dk = dv = 128 or 64 (else
 * RODIMUS_ERR_UNSUPPORTED); scale finite and > 0; 1 <= window <= 524288;
 * N * H < 2^24 and N * ceil(window / 256) * H below about 2^24 (else
 * RODIMUS_ERR_INVALID_ARG).  The second limit is a conservative bound: it
 * counts 256-slot splits and one head per workgroup, the most workgroups of
 * 256 threads the step can launch, so every launch stays below 2^32
 * work-items.  All buffers
 * are caller-owned device memory, 16-byte aligned (pos: 4-byte aligned).
 * `workspace` holds per-split partial results: at least
 * sw_ska_decode_workspace_bytes(N, H, dk, dv, window, dtype) bytes, else
 * RODIMUS_ERR_INVALID_ARG.  N = 0 or H = 0 is a no-op (pos unchanged).
 */
size_t sw_ska_decode_workspace_bytes(int N, int H, int dk, int dv, int window, int dtype);
int sw_ska_decode_step(const void *q, const void *k_new, const void *v_new, void *k_cache,
                       void *v_cache, int *pos, void *o, int N, int H, int dk, int dv, int window,
                       float scale, int dtype, void *workspace, size_t workspace_bytes,
                       void *stream);

/* Static, human-readable name of a status code (never NULL). */
const char *rodimus_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* RODIMUS_H */
