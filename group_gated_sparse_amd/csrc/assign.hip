// Hard group assignment: group_ids[t] = argmax_k (h_t · P) · C_k + bias_k.
//
// Focus ("Focus: Learning Which Attention Pairs Matter", technical summary
// §2.1: the hidden state is projected and compared with K centroids in
// centroid space; §2.2: a hard top-k assignment at inference, k = 1 here).
//
// (h P) C^T is regrouped as h (P C^T): a tiny prologue forms W^T = C P^T
// (K x d_model, fp32) once per call, so the streaming pass does d_model*K
// multiply-adds per token instead of d_model*d_proj + d_proj*K.
//
// The streaming pass is a dense contraction S^T = W^T H^T (K x tokens) that
// must keep up with HBM: at K = 32 it needs 16 flop per byte of hidden state,
// near the fp32 vector ridge, so it runs on bf16 MFMA with fp32-accurate
// operands: x = hi + lo with hi = bf16(x), lo = bf16(x - hi) for both h and
// W, and hi*hi + hi*lo + lo*hi accumulated in fp32 (the lo*lo term is below
// fp32 rounding of the products that are kept).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "focus_internal.h"

namespace focus {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kNegInf = -__builtin_inff();

// W^T[k][m] = sum_j P[m][j] C[k][j] for a block of 64 rows m, split into
// bf16 hi/lo tables of shape [KP][dpad]; padding rows/columns are zero.
// P is staged through LDS in 128-column slabs (row stride 129 floats, so the
// 64 lanes of a wave, one row each, hit 64 different banks); C is read with a
// wave-uniform address (one group k per wave at a time).
constexpr int PREP_ROWS = 64;
constexpr int PREP_COLS = 128;

__global__ __launch_bounds__(256) void assign_prep_kernel(const float* __restrict__ P,
                                                          const float* __restrict__ C,
                                                          int d_model, int d_proj, int K,
                                                          int KP, int dpad,
                                                          __bf16* __restrict__ whi,
                                                          __bf16* __restrict__ wlo) {
    __shared__ float Ps[PREP_ROWS * (PREP_COLS + 1)];
    const int m0 = blockIdx.x * PREP_ROWS;
    const int r = threadIdx.x % PREP_ROWS, wv = threadIdx.x / PREP_ROWS;
    const int m = m0 + r;
    float acc[16];
#pragma unroll
    for (int it = 0; it < 16; ++it) acc[it] = 0.0f;
    for (int j0 = 0; j0 < d_proj; j0 += PREP_COLS) {
        const int jc = min(PREP_COLS, d_proj - j0);
        __syncthreads();
        for (int x = threadIdx.x; x < PREP_ROWS * jc; x += blockDim.x) {
            const int rr = x / jc, j = x % jc;
            const int mm = m0 + rr;
            Ps[rr * (PREP_COLS + 1) + j] = (mm < d_model) ? P[(int64_t)mm * d_proj + j0 + j] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int k = wv + 4 * it;
            if (k < K) {
                const float* cr = C + (int64_t)k * d_proj + j0;
                const float* pr = Ps + r * (PREP_COLS + 1);
                float a = acc[it];
                for (int j = 0; j < jc; ++j) a = __builtin_fmaf(pr[j], cr[j], a);
                acc[it] = a;
            }
        }
    }
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int k = wv + 4 * it;
        if (k >= KP || m >= dpad) continue;
        const float a = (m < d_model && k < K) ? acc[it] : 0.0f;
        const __bf16 hi = (__bf16)a;
        const __bf16 lo = (__bf16)(a - (float)hi);
        whi[(int64_t)k * dpad + m] = hi;
        wlo[(int64_t)k * dpad + m] = lo;
    }
}

__device__ __forceinline__ float other_half(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ int other_half_i(int x) {
    auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return (int)((threadIdx.x & 32) ? r[0] : r[1]);
}

// One workgroup = 32 tokens; its 4 waves split d_model into quarters and
// their partial score tiles are summed in a fixed order (deterministic).
// Lane (rl, hh): token t0+rl; in each 64-wide step s it owns hidden columns
// s*64 + 32*hh .. +32 (one 128-byte run) and feeds them to 4 MFMA k-steps.
template <int NB>  // number of 32-group blocks: 1 (K <= 32) or 2 (K <= 64)
__global__ __launch_bounds__(256) void assign_argmax_kernel(
    const float* __restrict__ hidden, const __bf16* __restrict__ whi,
    const __bf16* __restrict__ wlo, const float* __restrict__ bias, int64_t ntok,
    int d_model, int dpad, int K, int32_t* __restrict__ ids, float* __restrict__ margin) {
    __shared__ float red[3][NB][16][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rl = lane & 31, hh = lane >> 5;
    const int64_t tok = (int64_t)blockIdx.x * 32 + rl;
    const bool tvalid = tok < ntok;
    const float* hrow = hidden + (tvalid ? tok : 0) * (int64_t)d_model;

    const int NS = dpad / 64;
    const int s_beg = (NS * wave) / 4, s_end = (NS * (wave + 1)) / 4;

    f32x16 acc[NB];
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
        for (int e = 0; e < 16; ++e) acc[mb][e] = 0.0f;

    for (int s = s_beg; s < s_end; ++s) {
        const int d0 = s * 64 + hh * 32;
        float4 hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = d0 + 4 * e;
            hv[e] = (tvalid && d < d_model) ? *reinterpret_cast<const float4*>(hrow + d)
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x[8] = {hv[2 * e].x,     hv[2 * e].y,     hv[2 * e].z,     hv[2 * e].w,
                                hv[2 * e + 1].x, hv[2 * e + 1].y, hv[2 * e + 1].z, hv[2 * e + 1].w};
            bf16x8 bh, bl;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                bh[t] = (__bf16)x[t];
                bl[t] = (__bf16)(x[t] - (float)bh[t]);
            }
#pragma unroll
            for (int mb = 0; mb < NB; ++mb) {
                const int64_t woff = (int64_t)(mb * 32 + rl) * dpad + d0 + 8 * e;
                const bf16x8 ah = *reinterpret_cast<const bf16x8*>(whi + woff);
                const bf16x8 al = *reinterpret_cast<const bf16x8*>(wlo + woff);
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc[mb], 0, 0, 0);
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc[mb], 0, 0, 0);
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc[mb], 0, 0, 0);
            }
        }
    }

    if (wave > 0) {
#pragma unroll
        for (int mb = 0; mb < NB; ++mb)
            for (int e = 0; e < 16; ++e) red[wave - 1][mb][e][lane] = acc[mb][e];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
        for (int e = 0; e < 16; ++e)
            acc[mb][e] = ((acc[mb][e] + red[0][mb][e][lane]) + red[1][mb][e][lane]) +
                         red[2][mb][e][lane];

    // Lane holds scores of groups k = mb*32 + 8*i + 4*hh + j (e = 4*i + j),
    // visited in increasing k. Top-2 with exact ties resolved to the lowest k.
    float b1 = kNegInf, b2 = kNegInf;
    int i1 = 0x7fffffff;
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
        for (int e = 0; e < 16; ++e) {
            const int k = mb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
            if (k >= K) continue;
            const float sc = bias ? acc[mb][e] + bias[k] : acc[mb][e];
            if (sc > b1) {
                b2 = b1;
                b1 = sc;
                i1 = k;
            } else if (sc > b2) {
                b2 = sc;
            }
        }
    const float ob1 = other_half(b1), ob2 = other_half(b2);
    const int oi1 = other_half_i(i1);
    float m1, m2;
    int mi;
    if (b1 > ob1 || (b1 == ob1 && i1 < oi1)) {
        m1 = b1; mi = i1; m2 = fmaxf(b2, ob1);
    } else {
        m1 = ob1; mi = oi1; m2 = fmaxf(ob2, b1);
    }
    if (hh == 0 && tvalid) {
        ids[tok] = mi;
        if (margin) margin[tok] = m1 - m2;
    }
}

}  // namespace

hipError_t launch_assign(const float* hidden, const float* P, const float* C, const float* bias,
                         int B, int n, int d_model, int d_proj, int K, int32_t* ids,
                         float* margin, void* workspace, hipStream_t stream) {
    const int KP = assign_kpad(K), dpad = assign_dpad(d_model);
    __bf16* whi = static_cast<__bf16*>(workspace);
    __bf16* wlo = reinterpret_cast<__bf16*>(static_cast<char*>(workspace) +
                                            align_up((size_t)KP * dpad * 2));
    hipLaunchKernelGGL(assign_prep_kernel, dim3(dpad / PREP_ROWS), dim3(256), 0, stream, P,
                       C, d_model, d_proj, K, KP, dpad, whi, wlo);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t ntok = (int64_t)B * n;
    const dim3 grid((unsigned)((ntok + 31) / 32));
    if (KP == 32)
        hipLaunchKernelGGL(assign_argmax_kernel<1>, grid, dim3(256), 0, stream, hidden, whi, wlo,
                           bias, ntok, d_model, dpad, K, ids, margin);
    else
        hipLaunchKernelGGL(assign_argmax_kernel<2>, grid, dim3(256), 0, stream, hidden, whi, wlo,
                           bias, ntok, d_model, dpad, K, ids, margin);
    return hipGetLastError();
}

}  // namespace focus
