// Hard group assignment: the top-M groups of each token by the scores
// s_k = (h_t · P) · C_k + bias_k (M = 1: group_ids[t] = argmax_k s_k).
//
// Focus ("Focus: Learning Which Attention Pairs Matter", technical summary
// §2.1: the hidden state is projected and compared with K centroids in
// centroid space; §2.2: a hard top-k assignment at inference, k = 1 or 2
// here; the Korean page §2.3 and §3.4 give the k = 2 variant).
//
// (h P) C^T is regrouped as h (P C^T): a tiny prologue forms W^T = C P^T
// (K x d_model, fp32) once per call, so the streaming pass does d_model*K
// multiply-adds per token instead of d_model*d_proj + d_proj*K.
//
// The streaming pass is a dense contraction S^T = W^T H^T (K x tokens) that
// must keep up with HBM: at K = 32 it needs 16 flop per byte of hidden state,
// beyond what scalar fp32 FMA sustains at 8 TB/s, so it runs on bf16 MFMA
// with fp32-accurate operands: x = hi + lo with hi = bf16(x), lo =
// bf16(x - hi) for both h and W, and hi*hi + hi*lo + lo*hi accumulated in
// fp32 (the dropped lo*lo term is ~2^-16 of each product).
//
// Memory layout for coalescing: the hidden slice of a stage (32 tokens x 256
// columns, 32 KB) is copied HBM -> LDS with global_load_lds_dwordx4, each
// copy one contiguous 1 KB of one token row (shorter runs per row, e.g. 256
// bytes, measured about 15 % slower on gfx950); the four waves share the
// stage and each multiplies its own 64 of the 256 columns. The W^T operand
// is stored by the prologue in MFMA fragment order, so every fragment load is
// also one contiguous 1 KB.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "focus_internal.h"

namespace focus {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();

// Fragment order of the split W^T tables. For 64-column step s, 32-group
// block mb, k-step e (8 columns) and table (0 = hi, 1 = lo), lane l = 32*hh +
// rl holds W^T[mb*32 + rl][64*s + 32*hh + 8*e .. +8] as 8 bf16 (16 bytes):
//   fragment index f = ((s * NB + mb) * 4 + e) * 2 + table,  bytes [f*1024 + 16*l, +16)
__device__ __forceinline__ int64_t wfrag_elem(int s, int NB, int mb, int e, int table, int lane) {
    return ((((int64_t)s * NB + mb) * 4 + e) * 2 + table) * 512 + lane * 8;
}

// W^T[k][m] = sum_j P[m][j] C[k][j]. One thread per output: a workgroup
// covers 256/KP columns m and all KP groups; P rows and C are staged through
// LDS in slabs of 128 values of j, C with a row stride of 129 floats so the
// KP groups read by one wave sit in distinct banks. Outputs are split into
// hi/lo bf16 and scattered into fragment order; padding groups (k >= K) and
// columns (m >= d_model) are zero.
constexpr int PREP_COLS = 128;
constexpr int PREP_CS = PREP_COLS + 1;

__global__ __launch_bounds__(256) void assign_prep_kernel(const float* __restrict__ P,
                                                          const float* __restrict__ C,
                                                          int d_model, int d_proj, int K,
                                                          int KP, int dpad,
                                                          __bf16* __restrict__ wfrag) {
    __shared__ float Cs[64 * PREP_CS];
    __shared__ float Ps[8 * PREP_COLS];
    const int rows = 256 / KP;                  // 8 (KP = 32) or 4 (KP = 64)
    const int m0 = blockIdx.x * rows;
    const int k = threadIdx.x % KP, r = threadIdx.x / KP;
    const int m = m0 + r;
    float acc = 0.0f;
    for (int j0 = 0; j0 < d_proj; j0 += PREP_COLS) {
        const int jc = min(PREP_COLS, d_proj - j0);
        __syncthreads();
        for (int x = threadIdx.x; x < KP * jc; x += 256) {
            const int kk = x / jc, j = x % jc;
            Cs[kk * PREP_CS + j] = (kk < K) ? C[(int64_t)kk * d_proj + j0 + j] : 0.0f;
        }
        for (int x = threadIdx.x; x < rows * jc; x += 256) {
            const int rr = x / jc, j = x % jc;
            const int mm = m0 + rr;
            Ps[rr * PREP_COLS + j] = (mm < d_model) ? P[(int64_t)mm * d_proj + j0 + j] : 0.0f;
        }
        __syncthreads();
        const float* pr = Ps + r * PREP_COLS;
        const float* cr = Cs + k * PREP_CS;
        for (int j = 0; j < jc; ++j) acc = __builtin_fmaf(pr[j], cr[j], acc);
    }
    if (m >= dpad) return;
    const float a = (m < d_model && k < K) ? acc : 0.0f;
    const __bf16 hi = (__bf16)a;
    const __bf16 lo = (__bf16)(a - (float)hi);
    const int NB = KP / 32;
    const int s = m / 64, within = m % 64;
    const int hh = within / 32, e = (within % 32) / 8, t = within % 8;
    const int mb = k / 32, rl = k % 32;
    const int lane = hh * 32 + rl;
    wfrag[wfrag_elem(s, NB, mb, e, 0, lane) + t] = hi;
    wfrag[wfrag_elem(s, NB, mb, e, 1, lane) + t] = lo;
}

__device__ __forceinline__ float other_half(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ int other_half_i(int x) {
    auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return (int)((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// LDS stage: 32 token rows x 256 fp32 columns (1 KB per row); 16-byte chunk
// c of row r sits in slot c ^ (r & 15), so the 16 rows read by one
// quarter-wave at the same logical chunk hit 16 distinct bank groups.
constexpr int HROWB = 1024;
constexpr int HSTAGEB = 32 * HROWB;  // 32 KB

template <int NB>
struct WRegs {
    bf16x8 f[NB][4][2];
};

// Running top list of (score, group), best first; the order is score
// descending, then group ascending, so exact ties go to the lowest index.
template <int M>
struct TopList {
    float v[M + 1];
    int g[M + 1];
};
__device__ __forceinline__ bool ranks_before(float a, int ga, float b, int gb) {
    return a > b || (a == b && ga < gb);
}
template <int M>
__device__ __forceinline__ void top_insert(TopList<M>& t, float x, int gx) {
#pragma unroll
    for (int p = 0; p <= M; ++p) {
        if (ranks_before(x, gx, t.v[p], t.g[p])) {
            const float tv = t.v[p];
            const int tg = t.g[p];
            t.v[p] = x;
            t.g[p] = gx;
            x = tv;
            gx = tg;
        }
    }
}

// M >= 1: top-M groups (ids, margin); M == 0: the raw scores [ntok][K].
template <int NB, int M>
__global__ __launch_bounds__(256, 2) void assign_argmax_kernel(
    const float* __restrict__ hidden, const __bf16* __restrict__ wfrag,
    const float* __restrict__ bias, int64_t ntok, int d_model, int dpad, int K,
    int32_t* __restrict__ ids, float* __restrict__ margin, float* __restrict__ scores) {
    // Two 32 KB stages; reused for the cross-wave reduction at the end.
    __shared__ __attribute__((aligned(1024))) unsigned char hbuf[2 * HSTAGEB];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rl = lane & 31, hh = lane >> 5;
    const int64_t t0 = (int64_t)blockIdx.x * 32;
    const int64_t tok = t0 + rl;
    const bool tvalid = tok < ntok;

    // Stage st holds columns [256 st, 256 st + 256); wave w multiplies its
    // 64-column step s = 4 st + w (when s < NS, the 64-column steps of dpad).
    const int NS = dpad / 64;
    const int NSTG = (NS + 3) / 4;

    // Copies of a stage: wave w copies rows 8w .. 8w+7, one 1 KB run each;
    // lane l fills slot l of the row, i.e. logical chunk l ^ (row & 15). The
    // hidden states are read once, so the copies are non-temporal (cache
    // policy nt), which leaves the caches to W and lifts the read rate.
    auto issue = [&](int st, unsigned char* dst, WRegs<NB>& wr) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 8 * wave + i;
            const int c = lane ^ (r & 15);
            const int64_t trow = min(t0 + r, ntok - 1);
            const int d = min(256 * st + 4 * c, d_model - 4);  // past d_model: W^T is zero there
            __builtin_amdgcn_global_load_lds(hidden + trow * d_model + d,
                                             (__attribute__((address_space(3))) void*)(dst + r * HROWB),
                                             16, 0, 2);
        }
        const int s = min(4 * st + wave, NS - 1);
#pragma unroll
        for (int mb = 0; mb < NB; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
                    wr.f[mb][e][tb] = *reinterpret_cast<const bf16x8*>(
                        wfrag + wfrag_elem(s, NB, mb, e, tb, lane));
    };

    f32x16 acc[NB];
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mb][e] = 0.0f;

    auto compute = [&](const unsigned char* src, const WRegs<NB>& wr) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // columns 64*wave + 32*hh + 8*e .. +8 of token rl: logical chunks c, c+1
            const int c = 16 * wave + 8 * hh + 2 * e;
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(src + rl * HROWB + ((c ^ (rl & 15)) << 4));
            const f32x4 x1 =
                *reinterpret_cast<const f32x4*>(src + rl * HROWB + (((c + 1) ^ (rl & 15)) << 4));
            const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            bf16x8 bh, bl;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                bh[t] = (__bf16)x[t];
                bl[t] = (__bf16)(x[t] - (float)bh[t]);
            }
#pragma unroll
            for (int mb = 0; mb < NB; ++mb) {
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr.f[mb][e][0], bl, acc[mb], 0, 0, 0);
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr.f[mb][e][1], bh, acc[mb], 0, 0, 0);
                acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wr.f[mb][e][0], bh, acc[mb], 0, 0, 0);
            }
        }
    };

    // Two stages; the copy of stage st+1 is in flight while stage st
    // computes. The barrier after each stage's copies have landed also
    // tells every wave that the other buffer's previous stage is done.
    WRegs<NB> wa, wb;
    issue(0, hbuf, wa);
    for (int st = 0; st < NSTG; st += 2) {
        wait_vm();
        __syncthreads();
        if (st + 1 < NSTG) issue(st + 1, hbuf + HSTAGEB, wb);
        if (4 * st + wave < NS) compute(hbuf, wa);
        if (st + 1 >= NSTG) break;
        wait_vm();
        __syncthreads();
        if (st + 2 < NSTG) issue(st + 2, hbuf, wa);
        if (4 * (st + 1) + wave < NS) compute(hbuf + HSTAGEB, wb);
    }

    // Cross-wave sum in a fixed order (deterministic), through LDS.
    __syncthreads();
    float* red = reinterpret_cast<float*>(hbuf);   // [3][NB][16][64]
    if (wave > 0) {
#pragma unroll
        for (int mb = 0; mb < NB; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) red[(((wave - 1) * NB + mb) * 16 + e) * 64 + lane] = acc[mb][e];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            acc[mb][e] = ((acc[mb][e] + red[((0 * NB + mb) * 16 + e) * 64 + lane]) +
                          red[((1 * NB + mb) * 16 + e) * 64 + lane]) +
                         red[((2 * NB + mb) * 16 + e) * 64 + lane];

    // Lane holds scores of groups k = mb*32 + 8*i + 4*hh + j (e = 4*i + j).
    if constexpr (M == 0) {
        if (tvalid) {
#pragma unroll
            for (int mb = 0; mb < NB; ++mb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int k = mb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
                    if (k < K) scores[tok * K + k] = bias ? acc[mb][e] + bias[k] : acc[mb][e];
                }
        }
        return;
    }
    // Each lane half keeps the top M+1 of its groups; the halves then swap
    // lists and both merge them, so both hold the top M+1 over all groups.
    TopList<(M > 0 ? M : 1)> top;
#pragma unroll
    for (int p = 0; p <= M; ++p) {
        top.v[p] = kNegInf;
        top.g[p] = 0x7fffffff;
    }
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int k = mb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
            if (k >= K) continue;
            top_insert(top, bias ? acc[mb][e] + bias[k] : acc[mb][e], k);
        }
    float ov[M + 1];
    int og[M + 1];
#pragma unroll
    for (int p = 0; p <= M; ++p) {
        ov[p] = other_half(top.v[p]);
        og[p] = other_half_i(top.g[p]);
    }
#pragma unroll
    for (int p = 0; p <= M; ++p) top_insert(top, ov[p], og[p]);
    if (hh == 0 && tvalid) {
#pragma unroll
        for (int c = 0; c < M; ++c) ids[tok * M + c] = top.g[c];
        // score gap deciding the M-th membership (+inf when K == M)
        if (margin) margin[tok] = top.v[M - 1] - top.v[M];
    }
}

}  // namespace

hipError_t launch_assign(const float* hidden, const float* P, const float* C, const float* bias,
                         int B, int n, int d_model, int d_proj, int K, int M, int32_t* ids,
                         float* margin, float* scores, void* workspace, hipStream_t stream) {
    const int KP = assign_kpad(K), dpad = assign_dpad(d_model);
    __bf16* wfrag = static_cast<__bf16*>(workspace);
    hipLaunchKernelGGL(assign_prep_kernel, dim3(dpad / (256 / KP)), dim3(256), 0, stream, P, C,
                       d_model, d_proj, K, KP, dpad, wfrag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t ntok = (int64_t)B * n;
    const dim3 grid((unsigned)((ntok + 31) / 32));
#define FOCUS_ASSIGN_LAUNCH(NB_, M_)                                                          \
    hipLaunchKernelGGL((assign_argmax_kernel<NB_, M_>), grid, dim3(256), 0, stream, hidden,   \
                       wfrag, bias, ntok, d_model, dpad, K, ids, margin, scores)
    if (KP == 32 && M == 0) FOCUS_ASSIGN_LAUNCH(1, 0);
    else if (KP == 32 && M == 1) FOCUS_ASSIGN_LAUNCH(1, 1);
    else if (KP == 32 && M == 2) FOCUS_ASSIGN_LAUNCH(1, 2);
    else if (M == 0) FOCUS_ASSIGN_LAUNCH(2, 0);
    else if (M == 1) FOCUS_ASSIGN_LAUNCH(2, 1);
    else if (M == 2) FOCUS_ASSIGN_LAUNCH(2, 2);
    else return hipErrorInvalidValue;
#undef FOCUS_ASSIGN_LAUNCH
    return hipGetLastError();
}

}  // namespace focus
