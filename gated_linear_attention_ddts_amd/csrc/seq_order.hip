// seq_order.hip -- longest-first order of the sequences of a packed ragged
// batch (the dynamic batching of short requests in the Tupoi O(1)-memory
// practice guide, section 4.2).
//
// The kernels that walk one sequence per workgroup (the prefill's output pass
// and segment-state pass, the backward's state passes) run far longer for a
// long request than for a short one.  Dispatched in table order, a long
// request that happens to come late runs alone at the end.  This kernel ranks
// the sequences by length, longest first (ties by index), and writes
// order[rank] = sequence; those kernels take their sequence through it, so
// the longest start first (list scheduling, longest job first).  All data is
// still addressed by the sequence's own index, so results do not change.
//
// Lengths are those the kernels use: each span clamped to [0, total] and to T.
// Up to kOrderMax sequences the comparison (length, then index) is a strict
// total order, so the ranks are a permutation whatever the table holds; cost
// O(N^2) compares, spread over one thread per sequence with the lengths staged
// through LDS (one workgroup up to 1024 sequences).  Larger batches are
// counted instead (O(N), one workgroup): the key is the number of 64-token
// chunks, clamped to kBuckets - 1, so the order is longest first at chunk
// granularity, and within a key in the order the slots were claimed.
#include "launch.h"

namespace rodimus {

namespace {

constexpr int kTile = 1024;
constexpr int kBuckets = 4096;  // chunk-count keys of the counting form (16 KiB of LDS)

__device__ __forceinline__ int span_len(const int *cu, int s, int total, int T) {
    const int a = min(max(cu[s], 0), total);
    const int b = min(max(cu[s + 1], a), total);
    return min(b - a, T);
}

// N <= kTile: one workgroup; every length is loaded once, by its own thread.
__global__ __launch_bounds__(kTile)
void seq_order_small_kernel(const int *__restrict__ cu, int N, int total, int T, int *__restrict__ order) {
    __shared__ int sl[kTile];
    const int i = threadIdx.x;
    const int li = i < N ? span_len(cu, i, total, T) : 0;
    sl[i] = li;
    __syncthreads();
    if (i < N) {
        int rank = 0;
        for (int j = 0; j < N; ++j) {
            const int lj = sl[j];
            rank += (lj > li) | ((lj == li) & (j < i));
        }
        order[rank] = i;
    }
}

__global__ __launch_bounds__(256)
void seq_order_kernel(const int *__restrict__ cu, int N, int total, int T, int *__restrict__ order) {
    __shared__ int sl[kTile];
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int li = i < N ? span_len(cu, i, total, T) : 0;
    int rank = 0;
    for (int j0 = 0; j0 < N; j0 += kTile) {
        const int m = min(kTile, N - j0);
        for (int k = threadIdx.x; k < m; k += 256) sl[k] = span_len(cu, j0 + k, total, T);
        __syncthreads();
        if (i < N) {
            for (int k = 0; k < m; ++k) {
                const int lj = sl[k], j = j0 + k;
                rank += (lj > li) | ((lj == li) & (j < i));
            }
        }
        __syncthreads();
    }
    if (i < N) order[rank] = i;
}

// N > kOrderMax: a counting sort by chunk count, longest first.  A histogram of
// the keys (LDS atomics), the start of each key's run of slots in descending
// key order (an exclusive scan of the histogram taken from the top key down),
// then every sequence claims the next slot of its key's run.  The slots of a
// key are claimed in a nondeterministic order, which changes only the order
// in which equally long sequences start, never a result.
__global__ __launch_bounds__(kTile)
void seq_order_count_kernel(const int *__restrict__ cu, int N, int total, int T, int *__restrict__ order) {
    __shared__ int cnt[kBuckets];
    __shared__ int part[kTile];
    const int tid = threadIdx.x;
    for (int b = tid; b < kBuckets; b += kTile) cnt[b] = 0;
    __syncthreads();
    auto key = [&](int s) { return min((span_len(cu, s, total, T) + 63) / 64, kBuckets - 1); };
    for (int s = tid; s < N; s += kTile) atomicAdd(&cnt[key(s)], 1);
    __syncthreads();
    // thread t scans the keys kBuckets-1-4t .. kBuckets-4-4t (4 per thread,
    // highest first); part[t] is their total
    constexpr int kPer = kBuckets / kTile;
    int c[kPer], run = 0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        c[u] = cnt[kBuckets - 1 - (kPer * tid + u)];
        run += c[u];
    }
    part[tid] = run;
    __syncthreads();
    // inclusive scan of part over the threads (Hillis-Steele in LDS)
    for (int off = 1; off < kTile; off <<= 1) {
        const int x = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += x;
        __syncthreads();
    }
    int start = part[tid] - run;  // slots taken by the higher keys of earlier threads
    __syncthreads();              // every thread has read the histogram
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        cnt[kBuckets - 1 - (kPer * tid + u)] = start;  // now the next free slot of the key
        start += c[u];
    }
    __syncthreads();
    for (int s = tid; s < N; s += kTile) order[atomicAdd(&cnt[key(s)], 1)] = s;
}

}  // namespace

size_t seq_order_bytes(int N) { return N > 0 ? ((size_t)N * 4 + 255) & ~(size_t)255 : 0; }

void launch_seq_order(const int *cu, int N, int total, int T, int *order, hipStream_t st) {
    if (N <= kTile)
        hipLaunchKernelGGL(seq_order_small_kernel, dim3(1), dim3(kTile), 0, st, cu, N, total, T, order);
    else if (N <= kOrderMax)
        hipLaunchKernelGGL(seq_order_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, cu, N, total, T,
                           order);
    else
        hipLaunchKernelGGL(seq_order_count_kernel, dim3(1), dim3(kTile), 0, st, cu, N, total, T, order);
}

}  // namespace rodimus
