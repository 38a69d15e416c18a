// Stable grouping of tokens by group id: a two-pass counting sort.
//
// The Focus pages group tokens by their assigned centroid (technical
// summaries §2.1-§2.2 of both pages); keeping each group's tokens in their
// sequence order makes a group's keys one contiguous, position-sorted segment,
// which is what lets the long-range attention pass skip other groups' tiles.
//
// Tokens of one batch element are cut into blocks of 2048 (256 threads x 8
// consecutive tokens).
//   pass 1 (hist):    each block counts its ids per group (LDS atomics; only
//                     counts, so the order of the increments does not matter)
//                     and writes hist[b][block][k].
//   pass 2 (scatter): each block derives the global start of its group-k run,
//                     offsets[k] + sum of hist[b][block' < block][k]; each
//                     thread counts its 8 tokens into its own LDS row, K
//                     threads scan those rows down the thread index
//                     (exclusive), and every thread replays its tokens in
//                     order, writing perm[start + rank] = token.
// Blocks, threads and the tokens of a thread are all visited in token order,
// so the result is the stable sort, and it is deterministic. A sequence of
// one block (n <= 2048) needs no counts from other blocks: the scatter pass
// alone runs, taking the group totals from its own scan.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "focus_internal.h"

namespace focus {
namespace {

constexpr int SORT_T = 256;
constexpr int SORT_PER = 8;
constexpr int MAXK = 64;

__device__ __forceinline__ int clamp_group(int g, int K) { return g < 0 ? 0 : (g >= K ? K - 1 : g); }

__global__ __launch_bounds__(SORT_T) void sort_hist_kernel(const int32_t* __restrict__ ids, int n,
                                                           int K, int nblk,
                                                           int32_t* __restrict__ hist) {
    __shared__ int h[MAXK];
    const int blk = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int32_t* g = ids + (int64_t)b * n;
    if (t < K) h[t] = 0;
    __syncthreads();
    const int x0 = blk * SORT_BLOCK_TOKENS + t * SORT_PER;
#pragma unroll
    for (int i = 0; i < SORT_PER; ++i) {
        const int x = x0 + i;
        if (x < n) atomicAdd(&h[clamp_group(g[x], K)], 1);
    }
    __syncthreads();
    if (t < K) hist[((int64_t)b * nblk + blk) * K + t] = h[t];
}

__global__ __launch_bounds__(SORT_T) void sort_scatter_kernel(const int32_t* __restrict__ ids,
                                                              int n, int K, int nblk,
                                                              const int32_t* __restrict__ hist,
                                                              int32_t* __restrict__ perm,
                                                              int32_t* __restrict__ offsets) {
    __shared__ int cnt[SORT_T * (MAXK + 1)];
    __shared__ int tot[MAXK + 1];
    __shared__ int before[MAXK];
    const int blk = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int32_t* g = ids + (int64_t)b * n;
    const int32_t* hb = hist + (int64_t)b * nblk * K;
    const int stride = K + 1;

    // Group totals of the batch element and the tokens of each group in
    // earlier blocks (one block: taken from the scan below).
    if (nblk > 1 && t < K) {
        int all = 0, pre = 0;
        for (int u = 0; u < nblk; ++u) {
            const int c = hb[(int64_t)u * K + t];
            all += c;
            if (u < blk) pre += c;
        }
        tot[t] = all;
        before[t] = pre;
    }
    // This thread's tokens, counted into its own row.
    int gid[SORT_PER];
    const int x0 = blk * SORT_BLOCK_TOKENS + t * SORT_PER;
    int* my = cnt + t * stride;
    for (int k = 0; k < K; ++k) my[k] = 0;
#pragma unroll
    for (int i = 0; i < SORT_PER; ++i) {
        const int x = x0 + i;
        gid[i] = x < n ? clamp_group(g[x], K) : -1;
        if (gid[i] >= 0) my[gid[i]] += 1;
    }
    __syncthreads();
    if (t < K) {   // exclusive scan down the thread index, per group
        int run = 0;
        for (int u = 0; u < SORT_T; ++u) {
            const int c = cnt[u * stride + t];
            cnt[u * stride + t] = run;
            run += c;
        }
        if (nblk == 1) {
            tot[t] = run;
            before[t] = 0;
        }
    }
    if (nblk == 1) __syncthreads();
    if (t == 0) {  // exclusive scan of the group totals -> group offsets
        int run = 0;
        for (int k = 0; k < K; ++k) {
            const int c = tot[k];
            tot[k] = run;
            run += c;
        }
        tot[K] = run;
    }
    __syncthreads();
    if (blk == 0 && t <= K) offsets[(int64_t)b * (K + 1) + t] = tot[t];
    int32_t* pb = perm + (int64_t)b * n;
#pragma unroll
    for (int i = 0; i < SORT_PER; ++i) {
        const int k = gid[i];
        if (k < 0) continue;
        pb[tot[k] + before[k] + my[k]] = x0 + i;
        my[k] += 1;
    }
}

}  // namespace

// The per-block group counts of focus_group_sort_noalloc live here instead of
// in a caller's workspace: a device array of the library, one copy on every
// GPU it runs on, held until the process ends. Every call on one GPU uses the
// same copy; the histogram pass writes every count the scatter pass reads, so
// nothing needs clearing between calls.
static __device__ __align__(256) int32_t scratch[kSortScratchBytes / 4];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t group_sort_scratch(int32_t** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        // The name `scratch` is only a host-side stand-in for the array; its
        // address on this device comes from the runtime, once per device.
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<int32_t*>(p);
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

size_t group_sort_workspace(int B, int n, int K) {
    const int nblk = (n + SORT_BLOCK_TOKENS - 1) / SORT_BLOCK_TOKENS;
    return align_up((size_t)B * nblk * K * 4);
}

hipError_t launch_group_sort(const int32_t* ids, int B, int n, int K, int32_t* perm,
                             int32_t* offsets, void* workspace, hipStream_t stream) {
    const int nblk = (n + SORT_BLOCK_TOKENS - 1) / SORT_BLOCK_TOKENS;
    int32_t* hist = static_cast<int32_t*>(workspace);
    const dim3 grid(nblk, B);
    if (nblk > 1) {
        hipLaunchKernelGGL(sort_hist_kernel, grid, dim3(SORT_T), 0, stream, ids, n, K, nblk, hist);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sort_scatter_kernel, grid, dim3(SORT_T), 0, stream, ids, n, K, nblk, hist,
                       perm, offsets);
    return hipGetLastError();
}

}  // namespace focus
