// Soft token-to-group assignment with Sinkhorn normalisation (the
// training-time step of Focus: Korean page "Why Attend to Everything? Focus
// is the Key", technical summary §2.2; Japanese page "Focus: Learning Which
// Attention Pairs Matter", §2.1 and §2.3): the n x K assignment matrix of
// each sequence is scaled to be doubly stochastic, every token's row summing
// to 1 and every group's column to n / K.
//
// With A = exp(scores / tau), G[t][k] = A[t][k] u[t] v[k]. Rows are
// normalised first (v = 1), then each round normalises the columns and then
// the rows again. The row step and the next round's column sums need the
// same row of A, so they share one pass over the scores:
//
//   pass p (p = 0 .. iters):  u[t] = 1 / sum_k A[t][k] v[k]     (v = 1 at p = 0)
//     p < iters:  column partial sums sum_t A[t][k] u[t] per workgroup; a
//                 small kernel then adds them (fixed order) and writes
//                 v[k] = (n / K) / column sum for the next pass, or, when
//                 there are few workgroups, each workgroup of the next pass
//                 adds them itself in the same fixed order
//     p = iters:  G[t][k] = A[t][k] u[t] v[k]
//
// A row's K scores sit in lpr lanes, four per lane when K is a multiple of
// 4 (one per lane otherwise), so a row is one coalesced read and its max
// and sum are a few in-lane steps plus lane-group reductions. A is recomputed from the scores on every pass with
// the row max subtracted (exp2((s - max) log2(e) / tau)); the per-row factor
// that this drops is absorbed by u exactly. Every sum is taken in a fixed
// order, so results are bitwise reproducible.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "focus_internal.h"

namespace focus {
namespace {

constexpr int NT = 256;
constexpr float kNegInf = -__builtin_inff();

// Value of the lane that mirrors this one inside the lane group of size
// 2s (s = 1, 2, 4, 8: DPP lane swizzles; 16: a cross-lane read; 32: swap of
// the wave halves). After the steps for s = 1 .. lpr/2, every lane of an
// aligned group of lpr lanes has combined all of the group's values.
template <int S>
__device__ __forceinline__ float partner(float x) {
    const int xi = __float_as_int(x);
    if (S == 1) return __int_as_float(__builtin_amdgcn_update_dpp(xi, xi, 0xB1, 0xF, 0xF, false));
    if (S == 2) return __int_as_float(__builtin_amdgcn_update_dpp(xi, xi, 0x4E, 0xF, 0xF, false));
    if (S == 4) return __int_as_float(__builtin_amdgcn_update_dpp(xi, xi, 0x141, 0xF, 0xF, false));
    if (S == 8) return __int_as_float(__builtin_amdgcn_update_dpp(xi, xi, 0x140, 0xF, 0xF, false));
    if (S == 16) return __shfl_xor(x, 16);
    auto r = __builtin_amdgcn_permlane32_swap((unsigned)xi, (unsigned)xi, false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
// quad_perm [1,0,3,2] (0xB1) and [2,3,0,1] (0x4E) pair lanes at distance 1
// and 2; row_half_mirror (0x141) maps lane i of 8 to 7 - i and row_mirror
// (0x140) lane i of 16 to 15 - i, which for max and sum is as good as a
// butterfly once the smaller groups are combined.
__device__ __forceinline__ float lane_group_max(float x, int lpr) {
    if (lpr > 1) x = fmaxf(x, partner<1>(x));
    if (lpr > 2) x = fmaxf(x, partner<2>(x));
    if (lpr > 4) x = fmaxf(x, partner<4>(x));
    if (lpr > 8) x = fmaxf(x, partner<8>(x));
    if (lpr > 16) x = fmaxf(x, partner<16>(x));
    if (lpr > 32) x = fmaxf(x, partner<32>(x));
    return x;
}
__device__ __forceinline__ float lane_group_sum(float x, int lpr) {
    if (lpr > 1) x += partner<1>(x);
    if (lpr > 2) x += partner<2>(x);
    if (lpr > 4) x += partner<4>(x);
    if (lpr > 8) x += partner<8>(x);
    if (lpr > 16) x += partner<16>(x);
    if (lpr > 32) x += partner<32>(x);
    return x;
}

struct SinkArgs {
    const float* S;      // scores [B][n][K]
    float* G;            // output [B][n][K]
    const float* v;      // column scales [B][K] from the previous round
    float* partial;      // column sums per workgroup, two buffers [2][B][nblk][K]
                         // (pass p writes buffer p % 2)
    int n, K, lpr, rpb, nblk, iters;
    int fused;           // each workgroup adds the previous pass's sums itself
    float sl2;           // log2(e) / tau
    float target;        // n / K
};

// Column totals of rows [0, J) of a [J][K] array in a fixed order: thread
// (g, k) of ng = 256 / K groups adds rows g, g + ng, ... into eight running
// sums (eight loads in flight), then the groups are added in order; returns
// the total of column tid for tid < K. Every caller gets the same bits.
__device__ float column_totals(const float* arr, int J, int K, float* gsum) {
    const int tid = threadIdx.x;
    const int ng = NT / K;
    const int g = tid / K, k = tid % K;
    float acc = 0.0f;
    if (g < ng) {
        float p8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        int j = g;
        for (; j + 7 * ng < J; j += 8 * ng) {
#pragma unroll
            for (int q = 0; q < 8; ++q) p8[q] += arr[(int64_t)(j + q * ng) * K + k];
        }
        float tail = 0.0f;
        for (; j < J; j += ng) tail += arr[(int64_t)j * K + k];
        acc = (((p8[0] + p8[1]) + (p8[2] + p8[3])) + ((p8[4] + p8[5]) + (p8[6] + p8[7]))) + tail;
    }
    gsum[tid] = acc;
    __syncthreads();
    float tot = 0.0f;
    if (tid < K)
        for (int j = 0; j < ng; ++j) tot += gsum[j * K + tid];
    return tot;
}

constexpr int UNROLL = 8;   // row chunks in flight per wave
// Per-workgroup column sums (workgroups x K) up to which each workgroup of
// the next pass adds them itself instead of a separate reduce launch.
constexpr int64_t kFuseMaxSums = 16384;

// VPL scores per lane: 1, or 4 (one 16-byte load) when K is a multiple of
// 4; a row then spans lpr = next power of two >= K / VPL lanes.
template <int VPL>
__global__ __launch_bounds__(NT) void sinkhorn_pass_kernel(SinkArgs a, int pass) {
    typedef float vecf __attribute__((ext_vector_type(VPL)));
    __shared__ float wsum[4][64 * VPL];
    const int b = blockIdx.y, blk = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lpr = a.lpr, rpw = 64 / lpr;
    const int c = lane & (lpr - 1);          // this lane's scores: columns VPL*c .. VPL*c + VPL-1
    const bool cvalid = VPL * c < a.K;
    const bool final_pass = pass == a.iters;
    const size_t pstride = (size_t)gridDim.y * a.nblk * a.K;   // one partial buffer
    const float* vsrc = a.v + (int64_t)b * a.K;
    if (a.fused && pass > 0) {
        // this workgroup adds the previous pass's per-workgroup sums itself
        // (same order in every workgroup, so every copy of v is identical)
        __shared__ float gsum[NT];
        __shared__ float vsh[64];
        const float* prev = a.partial + ((pass - 1) & 1) * pstride + (int64_t)b * a.nblk * a.K;
        const float tot = column_totals(prev, a.nblk, a.K, gsum);
        if (tid < a.K) vsh[tid] = tot > 0.0f ? a.target / tot : 0.0f;
        __syncthreads();
        vsrc = vsh;
    }
    float vc[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) vc[j] = (pass == 0 || !cvalid) ? 1.0f : vsrc[VPL * c + j];
    const float* Sb = a.S + (int64_t)b * a.n * a.K;
    const int r0 = blk * a.rpb, r1 = min(a.n, r0 + a.rpb);
    float colacc[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) colacc[j] = 0.0f;
    // wave-row chunks of rpw rows: chunk q of a trip covers rows
    // base + q * 4 * rpw + lane / lpr; a trip covers 4 * UNROLL * rpw rows
    for (int base = r0 + wave * rpw; base < r1; base += 4 * UNROLL * rpw) {
        vecf s[UNROLL];
#pragma unroll
        for (int q = 0; q < UNROLL; ++q) {
            const int t = base + q * 4 * rpw + lane / lpr;
            if (t < r1 && cvalid) {
                s[q] = *reinterpret_cast<const vecf*>(Sb + (int64_t)t * a.K + VPL * c);
            } else {
#pragma unroll
                for (int j = 0; j < VPL; ++j) s[q][j] = kNegInf;
            }
        }
#pragma unroll
        for (int q = 0; q < UNROLL; ++q) {
            const int t = base + q * 4 * rpw + lane / lpr;
            float m = s[q][0];
#pragma unroll
            for (int j = 1; j < VPL; ++j) m = fmaxf(m, s[q][j]);
            m = lane_group_max(m, lpr);
            float e[VPL], rs = 0.0f;
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                e[j] = (s[q][j] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f((s[q][j] - m) * a.sl2);
                rs += e[j] * vc[j];
            }
            rs = lane_group_sum(rs, lpr);
            const float u = rs > 0.0f ? 1.0f / rs : 0.0f;
            if (final_pass) {
                if (t < r1 && cvalid) {
                    vecf g;
#pragma unroll
                    for (int j = 0; j < VPL; ++j) g[j] = e[j] * u * vc[j];
                    *reinterpret_cast<vecf*>(a.G + ((int64_t)b * a.n + t) * a.K + VPL * c) = g;
                }
            } else {
#pragma unroll
                for (int j = 0; j < VPL; ++j) colacc[j] += e[j] * u;
            }
        }
    }
    if (final_pass) return;
    // Column sums of this workgroup: lanes of one column chunk (lane xor
    // multiples of lpr), then the four waves in order.
#pragma unroll
    for (int j = 0; j < VPL; ++j)
        for (int o = lpr; o < 64; o <<= 1) colacc[j] += __shfl_xor(colacc[j], o);
    if (lane < lpr) {
#pragma unroll
        for (int j = 0; j < VPL; ++j) wsum[wave][VPL * lane + j] = colacc[j];
    }
    __syncthreads();
    if (tid < a.K)
        a.partial[(pass & 1) * pstride + ((int64_t)b * a.nblk + blk) * a.K + tid] =
            ((wsum[0][tid] + wsum[1][tid]) + wsum[2][tid]) + wsum[3][tid];
}

// v[b][k] = (n / K) / (column k summed over the workgroups, in a fixed
// order): workgroup (k, b); thread j adds workgroups j, j + 256, ... into
// eight running sums (eight loads in flight), then a tree over the threads.
__global__ __launch_bounds__(NT) void sinkhorn_reduce_kernel(const float* __restrict__ partial,
                                                            int nblk, int K, float target,
                                                            float* __restrict__ v) {
    __shared__ float red[NT];
    const int k = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const float* pb = partial + (int64_t)b * nblk * K + k;
    float p8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int j = tid;
    for (; j + 7 * NT < nblk; j += 8 * NT) {
#pragma unroll
        for (int q = 0; q < 8; ++q) p8[q] += pb[(int64_t)(j + q * NT) * K];
    }
    float tail = 0.0f;
    for (; j < nblk; j += NT) tail += pb[(int64_t)j * K];
    red[tid] = (((p8[0] + p8[1]) + (p8[2] + p8[3])) + ((p8[4] + p8[5]) + (p8[6] + p8[7]))) + tail;
    __syncthreads();
    for (int h = NT / 2; h > 0; h >>= 1) {
        if (tid < h) red[tid] += red[tid + h];
        __syncthreads();
    }
    if (tid == 0) v[(int64_t)b * K + k] = red[0] > 0.0f ? target / red[0] : 0.0f;
}

}  // namespace

SinkhornLayout sinkhorn_layout(int B, int n, int K, int iters) {
    (void)iters;
    SinkhornLayout L{};
    // rows per workgroup: at least 128, and at most 2048 workgroups per sequence
    L.rpb = 128;
    while ((n + L.rpb - 1) / L.rpb > 2048) L.rpb <<= 1;
    L.nblk = (n + L.rpb - 1) / L.rpb;
    size_t off = 0;
    L.v = off;       off += align_up((size_t)B * K * 4);
    L.partial = off; off += 2 * align_up((size_t)B * L.nblk * K * 4);
    L.total = off;
    return L;
}

hipError_t launch_sinkhorn(const float* scores, int B, int n, int K, float tau, int iters,
                           float* G, void* workspace, hipStream_t stream) {
    const SinkhornLayout L = sinkhorn_layout(B, n, K, iters);
    char* base = static_cast<char*>(workspace);
    float* v = reinterpret_cast<float*>(base + L.v);
    SinkArgs a{};
    a.S = scores;
    a.G = G;
    a.v = v;
    a.partial = reinterpret_cast<float*>(base + L.partial);
    // four scores per lane (16-byte loads) when every row starts on 16 bytes
    const bool a16 = ((reinterpret_cast<uintptr_t>(scores) | reinterpret_cast<uintptr_t>(G)) & 15) == 0;
    const int vpl = (K % 4 == 0 && a16) ? 4 : 1;
    int lpr = 1;
    while (lpr * vpl < K) lpr <<= 1;
    a.n = n;
    a.K = K;
    a.lpr = lpr;
    a.rpb = L.rpb;
    a.nblk = L.nblk;
    a.iters = iters;
    a.sl2 = 1.44269504088896340736f / tau;
    const float target = (float)n / (float)K;
    a.target = target;
    // few enough per-workgroup sums: every workgroup of the next pass adds
    // them itself, which saves the reduce launch of each round
    a.fused = (int64_t)L.nblk * K <= kFuseMaxSums;
    const size_t pstride = (size_t)B * L.nblk * K;
    const dim3 grid((unsigned)L.nblk, (unsigned)B);
    for (int p = 0; p <= iters; ++p) {
        if (vpl == 4)
            hipLaunchKernelGGL(sinkhorn_pass_kernel<4>, grid, dim3(NT), 0, stream, a, p);
        else
            hipLaunchKernelGGL(sinkhorn_pass_kernel<1>, grid, dim3(NT), 0, stream, a, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (p == iters || a.fused) continue;
        hipLaunchKernelGGL(sinkhorn_reduce_kernel, dim3((unsigned)K, (unsigned)B), dim3(NT), 0,
                           stream, a.partial + (p & 1) * pstride, L.nblk, K, target, v);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace focus
