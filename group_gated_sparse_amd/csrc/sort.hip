// Stable grouping of tokens by group id: a counting sort per batch element.
//
// The Focus pages group tokens by their assigned centroid (technical
// summaries §2.1-§2.2 of both pages); keeping each group's tokens in their
// sequence order makes a group's keys one contiguous, position-sorted segment,
// which is what lets the long-range attention pass skip other groups' tiles.
//
// One workgroup of 256 threads per batch element:
//   1. thread t counts the ids of its contiguous chunk of tokens into its own
//      LDS column cnt[t][k] (no atomics: each counter has one owner; the row
//      stride K+1 spreads a wave's 64 columns over the banks);
//   2. K threads scan their group's column over t (exclusive), a single
//      thread scans the K totals -> group offsets;
//   3. each thread replays its chunk and scatters token indices to
//      offset[k] + (earlier tokens of k in lower chunks) + (earlier in chunk).
// Chunks are in token order and each chunk is replayed in order, so the sort
// is stable and deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "focus_internal.h"

namespace focus {
namespace {

constexpr int SORT_T = 256;
constexpr int MAXK = 64;

__device__ __forceinline__ int clamp_group(int g, int K) { return g < 0 ? 0 : (g >= K ? K - 1 : g); }

__global__ __launch_bounds__(SORT_T) void group_sort_kernel(const int32_t* __restrict__ ids, int n,
                                                            int K, int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ offsets) {
    __shared__ int cnt[SORT_T * (MAXK + 1)];
    __shared__ int tot[MAXK + 1];
    const int b = blockIdx.x, t = threadIdx.x;
    const int32_t* g = ids + (int64_t)b * n;
    int32_t* pb = perm + (int64_t)b * n;
    const int chunk = (n + SORT_T - 1) / SORT_T;
    const int beg = min(n, t * chunk), end = min(n, beg + chunk);
    const int stride = K + 1;
    int* my = cnt + t * stride;

    for (int k = 0; k < K; ++k) my[k] = 0;
    for (int i = beg; i < end; ++i) my[clamp_group(g[i], K)] += 1;
    __syncthreads();

    if (t < K) {
        int run = 0;
        for (int u = 0; u < SORT_T; ++u) {
            const int c = cnt[u * stride + t];
            cnt[u * stride + t] = run;
            run += c;
        }
        tot[t] = run;
    }
    __syncthreads();
    if (t == 0) {
        int run = 0;
        for (int k = 0; k < K; ++k) {
            const int c = tot[k];
            tot[k] = run;
            run += c;
        }
        tot[K] = run;
    }
    __syncthreads();
    if (t <= K) offsets[(int64_t)b * (K + 1) + t] = tot[t];
    for (int k = 0; k < K; ++k) my[k] += tot[k];
    for (int i = beg; i < end; ++i) {
        const int k = clamp_group(g[i], K);
        pb[my[k]] = i;
        my[k] += 1;
    }
}

}  // namespace

hipError_t launch_group_sort(const int32_t* ids, int B, int n, int K, int32_t* perm,
                             int32_t* offsets, hipStream_t stream) {
    hipLaunchKernelGGL(group_sort_kernel, dim3(B), dim3(SORT_T), 0, stream, ids, n, K, perm,
                       offsets);
    return hipGetLastError();
}

}  // namespace focus
