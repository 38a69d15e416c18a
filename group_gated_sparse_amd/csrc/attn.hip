// Exact-softmax attention over the Focus pattern, and the dense causal
// baseline, as bf16 MFMA flash-style kernels for gfx950.
//
// The pattern (Korean page "Why Attend to Everything? Focus is the Key",
// technical summary §2.1 and §2.3; Japanese page "Focus: Learning Which
// Attention Pairs Matter", §2.1-§2.2): row i keeps every key of the causal
// window 0 <= i-j <= w, and beyond the window only keys of its own group;
// the softmax is exact over the kept keys. The Korean page §2.3 splits the
// work into a local-window attention and an intra-group long-range
// attention; here those are two kernels joined by a log-sum-exp merge:
//
//   long-range pass (group-sorted order): for each tile of 128/G sorted
//     tokens x G query heads that share one kv head, visit only the key
//     tiles of the groups present in the tile, and inside a group only keys
//     whose position is below (largest query position) - w. Keys are
//     gathered through perm, so every visited tile is dense in one group.
//     Writes the normalised partial output and its log2-sum-exp per row.
//   window pass (sequence order): for each tile of tokens, the key band
//     [q0 - w, q0 + TT - 1]. The long-range partial is merged by starting
//     the online softmax from it (log-sum-exp merge, exact).
//   dense causal (baseline): the window pass with the band [0, q0 + TT - 1].
//
// The two key sets {i-j <= w} and {i-j > w, same group} are disjoint, so
// every allowed pair is counted exactly once.
//
// Per workgroup: 4 waves x 32 query rows. Per 64-key tile:
//   S^T (keys x rows) = K Q^T   : A = K from LDS, B = Q^T held in registers
//   online softmax per row in registers (one row per lane pair, exp2 domain)
//   O^T (d x rows)  += V^T P^T  : A = V^T via LDS transposing reads
//                                 (ds_read_b64_tr_b16), B = P^T in registers
// with v_mfma_f32_32x32x16_bf16 and fp32 accumulation. K and V tiles are
// copied HBM -> LDS by global_load_lds_dwordx4 into two LDS buffers: the copy
// of tile t+1 runs while tile t is computed, one barrier per tile. The
// running max is only moved (and the accumulator rescaled) when a row's max
// grows by more than 2^8, so probabilities stay <= 256 and the rescale is
// rare; the final normalisation is exact either way.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "focus_internal.h"

namespace focus {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 64;       // keys per tile
constexpr int NT = 256;      // threads per workgroup
constexpr int ROWS = 128;    // query rows per workgroup (4 waves x 32)
constexpr int MAXSEG = 64;   // groups present in one sorted query tile (K <= 64)
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;  // log2 units the running max may lag
constexpr int SEGCAP = 6;    // group segments stored per planned query tile
constexpr int PLAN_INTS = 16;

enum { kWindow = 0, kLongRange = 1, kDense = 2 };

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* ids;
    const int32_t* perm;
    const int32_t* offsets;
    const int* plan;  // long-range tile plan [B][ntiles][PLAN_INTS] or null
    float* og;     // long-range partial output [B][Hq][n][D] (normalised)
    float* lseg;   // long-range partial log2-sum-exp [B][Hq][n] (-inf: no key)
    void* out;
    float* lse;
    int B, Hq, Hkv, n, K, w;
    int hpk;       // Hq / Hkv
    int G;         // query heads packed per workgroup
    int TT;        // tokens per workgroup tile (ROWS / G)
    int nslices;   // hpk / G
    int ntiles;    // ceil(n / TT)
    int total;     // workgroups
    float sl2;     // scale * log2(e)
    int out_f32;
    int merge;
};

template <int D>
struct Geom {
    static constexpr int NCH = D / 8;                         // 16-byte chunks per row
    static constexpr int ROWB = D * 2;                        // bytes per row
    static constexpr int RPL = ROWB >= 256 ? 1 : 256 / ROWB;  // rows per 256-byte bank line
    static constexpr int TILEB = BN * ROWB;                   // bytes of one K or V tile
    static constexpr int NI = TILEB / (4 * 1024);             // 1 KB copies per wave per tile
    static constexpr int KS = D / 16;                         // k-steps of S^T = K Q^T
    static constexpr int DB = D / 32;                         // 32-wide blocks of O^T
};

// LDS tile layout: row r (one key) is ROWB contiguous bytes; its 16-byte
// chunk c is stored in slot c ^ swz(r). The LDS serves 256 bytes (64 banks)
// per cycle; a read is conflict-free when the lanes served together hit
// distinct 16-byte bank groups (address / 16 mod 16). Measured on gfx950, the
// patterns that matter are
//   K operand (16-byte reads): 16 consecutive rows, one logical chunk;
//   V operand (transposing 8-byte reads, 32 lanes together): 4 consecutive
//     rows (aligned to 4) x logical chunks c0..c0+3 (c0 a multiple of 4),
// and the swizzles below make both conflict-free. They depend on row bits
// 0-3 only, so row + 16*j keeps the same swizzle.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);          // 16 chunks per row
    if (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);    // 8 chunks, 2 rows per 256 B
    return (r >> 2) & 3;                                           // 4 chunks, 4 rows per 256 B
}
template <int D>
__device__ __forceinline__ int lds_off(int row, int ch) {
    return row * Geom<D>::ROWB + ((ch ^ swz<D>(row)) << 4);
}
// Inverse for the copy: chunk slot `pc` of row `row` holds logical chunk pc ^ swz.
template <int D>
__device__ __forceinline__ int logical_chunk(int row, int pc) {
    return pc ^ swz<D>(row);
}

__device__ __forceinline__ float other_half(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16-byte global -> LDS copy; lane l lands at lds_base + 16*l.
__device__ __forceinline__ void copy16(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0,
                                     0);
}

// Workgroups are dealt round-robin to the 8 XCDs; renumber them so each XCD
// works through one contiguous range of work items (neighbouring tiles of one
// head share keys in that XCD's L2).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int per = total / 8, rem = total % 8;
    const int x = bid % 8, local = bid / 8;
    return x * per + (x < rem ? x : rem) + local;
}

// Key slots [ob, kend) that group g contributes to the long-range pass of
// the sorted query slots [s0, s1): the group's segment [ob, oe) of perm, cut
// at the first slot whose position is >= (largest query position of g in the
// tile) - w. Positions increase inside a segment, so that cut is a binary
// search, and no later slot of the segment can pair with any query of g here.
__device__ __forceinline__ void segment_range(const int32_t* perm_b, const int32_t* offb, int n,
                                              int w, int s0, int s1, int g, int& ob, int& kend) {
    ob = clampi(offb[g], 0, n);
    const int oe = clampi(offb[g + 1], ob, n);
    const int qlo = max(s0, ob), qhi = min(s1, oe);
    kend = ob;
    if (qlo < qhi) {
        const int maxpos = clampi(perm_b[qhi - 1], 0, n - 1);
        int lo = ob, hi = qhi;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (perm_b[mid] < maxpos - w) lo = mid + 1; else hi = mid;
        }
        kend = lo;
    }
}

// Tile plan of the long-range pass, once per (batch, sorted query tile) and
// shared by every kv head: record = {nseg (-1: more than SEGCAP groups, the
// attention kernel then derives its segments itself), first group, all query
// rows in one group, smallest query position, (ob, kend) per group}.
__global__ __launch_bounds__(256) void attn_plan_kernel(const int32_t* __restrict__ ids,
                                                        const int32_t* __restrict__ perm,
                                                        const int32_t* __restrict__ offsets,
                                                        int n, int K, int w, int TT, int ntiles,
                                                        int32_t* __restrict__ plan) {
    const int b = blockIdx.y;
    const int tile = blockIdx.x * 256 + threadIdx.x;
    if (tile >= ntiles) return;
    const int64_t bn = (int64_t)b * n;
    const int32_t* perm_b = perm + bn;
    const int32_t* offb = offsets + (int64_t)b * (K + 1);
    const int s0 = tile * TT, s1 = min(n, s0 + TT);
    const int gf = clampi(ids[bn + clampi(perm_b[s0], 0, n - 1)], 0, K - 1);
    const int gl = clampi(ids[bn + clampi(perm_b[s1 - 1], 0, n - 1)], gf, K - 1);
    const int nseg = gl - gf + 1;
    int32_t* rec = plan + ((int64_t)b * ntiles + tile) * PLAN_INTS;
    if (nseg > SEGCAP) {
        rec[0] = -1;
        return;
    }
    for (int t = 0; t < nseg; ++t) {
        int ob, kend;
        segment_range(perm_b, offb, n, w, s0, s1, gf + t, ob, kend);
        rec[4 + 2 * t] = ob;
        rec[5 + 2 * t] = kend;
    }
    const int ob0 = clampi(offb[gf], 0, n), oe0 = clampi(offb[gf + 1], ob0, n);
    rec[0] = nseg;
    rec[1] = gf;
    rec[2] = (s0 >= ob0 && s1 <= oe0) ? 1 : 0;
    rec[3] = clampi(perm_b[s0], 0, n - 1);
}

template <int D, int PHASE>
__global__ __launch_bounds__(NT, 2) void attn_kernel(AttnArgs a) {
    using G = Geom<D>;
    constexpr bool SORTED = PHASE == kLongRange;
    __shared__ __attribute__((aligned(1024))) unsigned char buf0[2 * G::TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char buf1[2 * G::TILEB];
    __shared__ int kpos0[BN], kpos1[BN];
    __shared__ int seg_ob[MAXSEG], seg_kend[MAXSEG], seg_t0[MAXSEG + 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = lane & 31, hh = lane >> 5;

    const int L = xcd_remap(blockIdx.x, a.total);
    int tile = L % a.ntiles;
    int rest = L / a.ntiles;
    const int slice = rest % a.nslices;
    rest /= a.nslices;
    const int kvh = rest % a.Hkv;
    const int b = rest / a.Hkv;
    if (SORTED) tile = a.ntiles - 1 - tile;  // heavier sorted tiles first

    const int R = wave * 32 + rl;
    const int hslot = R / a.TT, tok = R % a.TT;
    const int h = kvh * a.hpk + slice * a.G + hslot;
    const int64_t bn = (int64_t)b * a.n;
    const int s_row = tile * a.TT + tok;
    const bool rvalid = s_row < a.n;
    int pos_i = rvalid ? s_row : 0;
    int g_i = -1;
    if (SORTED && rvalid) {
        pos_i = clampi(a.perm[bn + s_row], 0, a.n - 1);
        g_i = clampi(a.ids[bn + pos_i], 0, a.K - 1);
    }

    const uint16_t* kbase = a.k + ((int64_t)b * a.Hkv + kvh) * a.n * D;
    const uint16_t* vbase = a.v + ((int64_t)b * a.Hkv + kvh) * a.n * D;

    // ---- the key tiles this workgroup visits: ntl tiles, tile tau at
    // ---- key slot kt0(tau), valid slots below kend(tau).
    int ntl = 0;
    int kstart = 0, kend0 = 0;               // sequence-order passes
    int gfirst = 0, minpos = 0;              // long-range pass
    bool rows_one_group = false;
    if (!SORTED) {
        const int q0 = tile * a.TT;
        const int qlast = min(a.n, q0 + a.TT) - 1;
        kstart = (PHASE == kDense) ? 0 : max(0, q0 - a.w);
        kend0 = qlast + 1;
        ntl = (kend0 - kstart + BN - 1) / BN;
    } else {
        const int s0 = tile * a.TT;
        const int s1 = min(a.n, s0 + a.TT);
        const int32_t* offb = a.offsets + (int64_t)b * (a.K + 1);
        const int32_t* rec = a.plan ? a.plan + ((int64_t)b * a.ntiles + tile) * PLAN_INTS : nullptr;
        int nseg = rec ? rec[0] : -1;
        if (nseg >= 0) {
            nseg = min(nseg, SEGCAP);
            gfirst = clampi(rec[1], 0, a.K - 1);
            rows_one_group = rec[2] != 0;
            minpos = clampi(rec[3], 0, a.n - 1);
            if (tid < nseg) {
                seg_ob[tid] = clampi(rec[4 + 2 * tid], 0, a.n);
                seg_kend[tid] = clampi(rec[5 + 2 * tid], seg_ob[tid], a.n);
            }
        } else {
            gfirst = clampi(a.ids[bn + clampi(a.perm[bn + s0], 0, a.n - 1)], 0, a.K - 1);
            const int glast =
                clampi(a.ids[bn + clampi(a.perm[bn + s1 - 1], 0, a.n - 1)], gfirst, a.K - 1);
            nseg = glast - gfirst + 1;
            if (tid < nseg) {
                int ob, kend;
                segment_range(a.perm + bn, offb, a.n, a.w, s0, s1, gfirst + tid, ob, kend);
                seg_ob[tid] = ob;
                seg_kend[tid] = kend;
            }
            const int ob0 = clampi(offb[gfirst], 0, a.n);
            const int oe0 = clampi(offb[gfirst + 1], ob0, a.n);
            rows_one_group = (s0 >= ob0) && (s1 <= oe0);
            minpos = clampi(a.perm[bn + s0], 0, a.n - 1);
        }
        __syncthreads();
        if (tid == 0) {
            int run = 0;
            for (int t = 0; t < nseg; ++t) {
                seg_t0[t] = run;
                run += (seg_kend[t] - seg_ob[t] + BN - 1) / BN;
            }
            seg_t0[nseg] = run;
        }
        __syncthreads();
        ntl = seg_t0[nseg];
    }

    // Tile tau -> (segment, first key slot, end of valid slots).
    int seg_cur = 0;
    auto locate = [&](int tau, int& seg, int& kt0, int& kend) {
        if (!SORTED) {
            seg = 0;
            kt0 = kstart + tau * BN;
            kend = kend0;
        } else {
            while (seg_t0[seg + 1] <= tau) ++seg;
            kt0 = seg_ob[seg] + (tau - seg_t0[seg]) * BN;
            kend = seg_kend[seg];
        }
    };

    // This lane's share of a tile copy: NI rows (one per 1 KB copy) and the
    // logical chunk it fetches from each.
    int crow[G::NI], cch[G::NI];
#pragma unroll
    for (int i = 0; i < G::NI; ++i) {
        const int o = (wave * G::NI + i) * 1024 + 16 * lane;
        crow[i] = o / G::ROWB;
        cch[i] = logical_chunk<D>(crow[i], (o % G::ROWB) / 16);
    }
    int cpos[G::NI];  // sorted pass: positions of the rows of the next copy

    auto fetch_pos = [&](int tau) {
        int seg = seg_cur, kt0, kend;
        locate(tau, seg, kt0, kend);
#pragma unroll
        for (int i = 0; i < G::NI; ++i)
            cpos[i] = a.perm[bn + min(kt0 + crow[i], kend - 1)];
    };
    auto issue = [&](int tau, unsigned char* bufp, int* kposp) {
        int seg = seg_cur, kt0, kend;
        locate(tau, seg, kt0, kend);
#pragma unroll
        for (int i = 0; i < G::NI; ++i) {
            int pos;
            if (SORTED) {
                pos = clampi(cpos[i], 0, a.n - 1);
                if ((16 * lane) % G::ROWB == 0)
                    kposp[crow[i]] = (kt0 + crow[i] < kend) ? pos : 0x7fffffff;
            } else {
                pos = min(kt0 + crow[i], kend - 1);
            }
            const int64_t go = (int64_t)pos * D + cch[i] * 8;
            copy16(kbase + go, bufp + (wave * G::NI + i) * 1024);
            copy16(vbase + go, bufp + G::TILEB + (wave * G::NI + i) * 1024);
        }
    };

    // LDS offsets of this lane's operand reads (tile-relative).
    int koff[G::KS];
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) koff[ks] = lds_off<D>(rl, 2 * ks + hh);
    const int m16 = lane & 15;
    const int colbase = 16 * ((lane >> 4) & 1) + 4 * (m16 & 3);
    int voff[G::DB][2];
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int col = db * 32 + colbase;
            voff[db][s] = G::TILEB + lds_off<D>(4 * hh + (m16 >> 2) + 8 * s, col >> 3) + (col & 7) * 2;
        }

    f32x16 acc[G::DB];
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;
    float m_ref = kNegInf, l_run = 0.0f;
    bf16x8 qf[G::KS];  // Q^T fragments, loaded once the first key tile is in flight

    auto compute = [&](int tau, const unsigned char* bufp, const int* kposp) {
        int kt0, kend;
        locate(tau, seg_cur, kt0, kend);
        // S^T = K Q^T for two 32-key blocks.
        f32x16 st[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) st[kb][e] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < G::KS; ++ks) {
                const bf16x8 kf =
                    *reinterpret_cast<const bf16x8*>(bufp + kb * 32 * G::ROWB + koff[ks]);
                st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], st[kb], 0, 0, 0);
            }
        }

        // Mask (boundary tiles only). Lane holds keys kidx = kb*32 +
        // 8*(e>>2) + 4*hh + (e&3) of its row.
        bool full;
        if (!SORTED) {
            const int q0 = tile * a.TT;
            const int qlast = kend - 1;
            full = (kt0 + BN - 1 <= q0) && (kt0 + BN <= kend) &&
                   (PHASE == kDense || qlast - kt0 <= a.w);
        } else {
            full = rows_one_group && seg_cur == 0 && (kt0 + BN <= kend) &&
                   (minpos - kposp[BN - 1] > a.w);
        }
        if (!full) {
            const int seg_g = gfirst + seg_cur;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int kidx = kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
                    const int key = kt0 + kidx;
                    bool ok;
                    if (!SORTED) {
                        ok = key < kend && key <= pos_i && pos_i - key <= a.w;
                    } else {
                        ok = g_i == seg_g && key < kend && pos_i - kposp[kidx] > a.w;
                    }
                    if (!ok) st[kb][e] = kNegInf;
                }
        }

        // Online softmax with a lagging reference max.
        float tmax = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, st[kb][e]);
        tmax = fmaxf(tmax, other_half(tmax)) * a.sl2;
        const bool grow = tmax > m_ref + kRescaleSlack;
        if (__any(grow)) {
            // growing rows: alpha = 2^(m_ref - tmax) (0 when m_ref = -inf);
            // the other rows of the wave keep their reference (alpha = 1).
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - tmax) : 1.0f;
            const float m_new = grow ? tmax : m_ref;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < G::DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
            m_ref = m_new;
        }
        const float m_use = (m_ref == kNegInf) ? 0.0f : m_ref;
        float psum = 0.0f;
        bf16x8 pf[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][e], a.sl2, -m_use));
                psum += p;
                pf[kb][e >> 3][e & 7] = (__bf16)p;
            }
        l_run += psum;

        // O^T += V^T P^T. For k-step (kb, sp) the B slots 0..3 / 4..7 of lane
        // half hh hold keys kb*32+16*sp+4*hh+{0..3} / +8+{0..3}; the A operand
        // gets the same keys through two transposing reads, lane m of each
        // 16-lane group addressing row key0 + m/4, columns 4*(m%4) .. +3 of
        // its 16-column half.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                const unsigned char* vb = bufp + (kb * 32 + 16 * sp) * G::ROWB;
#pragma unroll
                for (int db = 0; db < G::DB; ++db) {
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4*)(vb + voff[db][0]));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4*)(vb + voff[db][1]));
                    const s16x8 vv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, vv), pf[kb][sp], acc[db], 0, 0, 0);
                }
            }
    };

    // ---- main loop: two LDS buffers, the copy of tile tau+1 overlaps the
    // ---- compute of tile tau; one barrier per tile.
    if (ntl > 0) {
        if (SORTED) {
            fetch_pos(0);
            wait_vm();
        }
        issue(0, buf0, kpos0);
        if (SORTED && ntl > 1) fetch_pos(1);
    }
    // Window pass: start the online softmax from the long-range partial. A
    // normalised partial O_g with log2-sum-exp L_g is exactly the state
    // (acc = O_g, l = 1, reference max = L_g), so the window keys accumulate
    // on top of it and the final normalisation merges both parts; the loads
    // share the round trip of the Q rows and the first K/V tile.
    if (PHASE == kWindow && a.merge && rvalid) {
        const int64_t row = ((int64_t)b * a.Hq + h) * a.n + pos_i;
        const float lg = a.lseg[row];
        if (lg != kNegInf) {
            const float* grow_p = a.og + row * D;
#pragma unroll
            for (int db = 0; db < G::DB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4 gv = *reinterpret_cast<const f32x4*>(grow_p + db * 32 + 8 * i + 4 * hh);
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[db][4 * i + j] = gv[j];
                }
            m_ref = lg;
            l_run = (hh == 0) ? 1.0f : 0.0f;  // halves are summed at the end
        }
    }
    // Q^T fragments: lane holds Q[row][16*ks + 8*hh .. +8] for every k-step.
    const int64_t qrow_off = (((int64_t)b * a.Hq + h) * a.n + pos_i) * D;
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
        if (rvalid) {
            qf[ks] = *reinterpret_cast<const bf16x8*>(a.q + qrow_off + 16 * ks + 8 * hh);
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) qf[ks][t] = (__bf16)0.0f;
        }
    }

    if (ntl > 0) {
        for (int tau = 0; tau < ntl; tau += 2) {
            wait_vm();
            __syncthreads();
            if (tau + 1 < ntl) {
                issue(tau + 1, buf1, kpos1);
                if (SORTED && tau + 2 < ntl) fetch_pos(tau + 2);
            }
            compute(tau, buf0, kpos0);
            if (tau + 1 >= ntl) break;
            wait_vm();
            __syncthreads();
            if (tau + 2 < ntl) {
                issue(tau + 2, buf0, kpos0);
                if (SORTED && tau + 3 < ntl) fetch_pos(tau + 3);
            }
            compute(tau + 1, buf1, kpos1);
        }
    }

    // Epilogue. Lane holds rows' O^T entries d = db*32 + 8*i + 4*hh + j at
    // acc[db][4*i + j]; l_run covers this lane half's keys.
    const float l_tot = l_run + other_half(l_run);
    const int64_t row = ((int64_t)b * a.Hq + h) * a.n + pos_i;
    if (!rvalid) return;
    if (SORTED) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        float* orow = a.og + row * D;
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 o = {acc[db][4 * i] * inv, acc[db][4 * i + 1] * inv,
                           acc[db][4 * i + 2] * inv, acc[db][4 * i + 3] * inv};
                *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * i + 4 * hh) = o;
            }
        if (hh == 0) a.lseg[row] = l_tot > 0.0f ? m_ref + __log2f(l_tot) : kNegInf;
        return;
    }
    const float lse2 = m_ref + __log2f(l_tot);
    const float cw = 1.0f / l_tot;
#pragma unroll
    for (int db = 0; db < G::DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d0 = db * 32 + 8 * i + 4 * hh;
            const f32x4 o = {acc[db][4 * i] * cw, acc[db][4 * i + 1] * cw, acc[db][4 * i + 2] * cw,
                             acc[db][4 * i + 3] * cw};
            if (a.out_f32) {
                *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * D + d0) = o;
            } else {
                const bf16x4 ob = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
                *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.out) + row * D + d0) = ob;
            }
        }
    if (hh == 0 && a.lse) a.lse[row] = lse2 * kLn2;
}

// Query heads packed into one workgroup: the largest power of two <= 8 that
// divides Hq/Hkv. All packed heads share the kv head, the token set and the
// mask, so each K/V tile staged in LDS serves G*TT = 128 query rows.
int heads_per_wg(int hpk) {
    int g = 1;
    while (g < 8 && hpk % (2 * g) == 0) g *= 2;
    return g;
}

AttnArgs make_args(const AttnProblem& p) {
    AttnArgs a{};
    a.q = p.q;
    a.k = p.k;
    a.v = p.v;
    a.ids = p.ids;
    a.perm = p.perm;
    a.offsets = p.offsets;
    a.out = p.out;
    a.lse = p.lse;
    a.B = p.B;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.n = p.n;
    a.K = p.K;
    a.w = p.w;
    a.hpk = p.Hq / p.Hkv;
    a.G = heads_per_wg(a.hpk);
    a.TT = ROWS / a.G;
    a.nslices = a.hpk / a.G;
    a.ntiles = (p.n + a.TT - 1) / a.TT;
    a.total = p.B * p.Hkv * a.nslices * a.ntiles;
    a.sl2 = p.scale * 1.44269504088896340736f;
    a.out_f32 = p.out_f32;
    if (p.workspace) {
        char* ws = static_cast<char*>(p.workspace);
        const size_t og_bytes = align_up((size_t)p.B * p.Hq * p.n * p.d * 4);
        const size_t lse_bytes = align_up((size_t)p.B * p.Hq * p.n * 4);
        a.og = reinterpret_cast<float*>(ws);
        a.lseg = reinterpret_cast<float*>(ws + og_bytes);
        a.plan = reinterpret_cast<const int32_t*>(ws + og_bytes + lse_bytes);
    }
    return a;
}

template <int PHASE>
hipError_t launch(const AttnArgs& a, int d, hipStream_t stream) {
    const dim3 grid((unsigned)a.total), block(NT);
    switch (d) {
        case 32: hipLaunchKernelGGL((attn_kernel<32, PHASE>), grid, block, 0, stream, a); break;
        case 64: hipLaunchKernelGGL((attn_kernel<64, PHASE>), grid, block, 0, stream, a); break;
        case 128: hipLaunchKernelGGL((attn_kernel<128, PHASE>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_long_range(const AttnProblem& p, hipStream_t stream) {
    if (!attn_has_long_range(p.n, p.w)) return hipSuccess;
    AttnArgs a = make_args(p);
    hipLaunchKernelGGL(attn_plan_kernel, dim3((a.ntiles + 255) / 256, p.B), dim3(256), 0, stream,
                       p.ids, p.perm, p.offsets, p.n, p.K, p.w, a.TT, a.ntiles,
                       const_cast<int32_t*>(a.plan));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch<kLongRange>(a, p.d, stream);
}

hipError_t launch_attn_window(const AttnProblem& p, bool merge, hipStream_t stream) {
    AttnArgs a = make_args(p);
    a.plan = nullptr;
    a.merge = merge && attn_has_long_range(p.n, p.w) ? 1 : 0;
    return launch<kWindow>(a, p.d, stream);
}

hipError_t launch_attn_dense(const AttnProblem& p, hipStream_t stream) {
    AttnArgs a = make_args(p);
    a.plan = nullptr;
    a.merge = 0;
    a.w = p.n;
    return launch<kDense>(a, p.d, stream);
}

}  // namespace focus
