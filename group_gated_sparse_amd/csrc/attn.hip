// Exact-softmax attention over the Focus pattern, and the dense causal
// baseline, as bf16 MFMA flash-style kernels for gfx950.
//
// The pattern (Korean page "Why Attend to Everything? Focus is the Key",
// technical summary §2.1 and §2.3; Japanese page "Focus: Learning Which
// Attention Pairs Matter", §2.1-§2.2): row i keeps every key of the causal
// window 0 <= i-j <= w, and beyond the window only keys of its own group;
// the softmax is exact over the kept keys. The Korean page §2.3 splits the
// work into a local-window attention and an intra-group long-range
// attention; here those are two passes joined by a log-sum-exp merge:
//
//   window pass (sequence order): for each tile of tokens, the key band
//     [q0 - w, q0 + TT - 1]. It needs no group data, so it can run while the
//     groups are being assigned and sorted. It writes the normalised partial
//     output as 16 bits per element (fp16 with a per-row power-of-two scale)
//     and its log2-sum-exp per row.
//   long-range pass (group-sorted order): key slot s is key row perm[s],
//     read in place (one group per token: each tile copy takes its rows'
//     positions from perm, loaded a tile ahead) or from group-sorted copies
//     of K and V (two groups per token); a plan kernel lists, per
//     sorted query tile, the key-slot range of each group present (keys of
//     the group with position below (largest query position) - w). The
//     attention kernel, for each tile of 128/G sorted tokens x G query heads
//     sharing one kv head, visits only those key tiles, so every visited
//     tile is dense in one group. The window partial is merged by starting
//     the online softmax from it (log-sum-exp merge, exact), and the final
//     rows are written to their original positions.
//   dense causal (baseline): the window pass with the band [0, q0 + TT - 1].
//
// The two key sets {i-j <= w} and {i-j > w, same group} are disjoint, so
// every allowed pair is counted exactly once.
//
// Per workgroup: 4 waves x 32 query rows. Per key tile (32 or 64 keys):
//   S^T (keys x rows) = K Q^T   : A = K from LDS, B = Q^T held in registers
//   online softmax per row in registers (one row per lane pair, exp2 domain)
//   O^T (d x rows)  += V^T P^T  : A = V^T via LDS transposing reads
//                                 (ds_read_b64_tr_b16), B = P^T in registers
// with v_mfma_f32_32x32x16_bf16 and fp32 accumulation. K and V tiles are
// copied HBM -> LDS by buffer_load_dwordx4 ... lds into two LDS buffers: the
// copy of tile t+1 runs while tile t is computed, one barrier per tile. A
// wave skips a tile none of its rows keeps. The
// probabilities are taken against a reference max that is only moved (and
// the accumulator rescaled) when a lane's probability sum for a tile exceeds
// 2^8, so no per-tile max is computed on the common path, probabilities stay
// <= 256, and the final normalisation is exact either way. Each row keeps two
// sums: that of the probabilities as the PV product takes them (rounded to
// bf16), which normalises the output, so the weights applied to V sum to one
// exactly; and that of the fp32 probabilities, which gives the log-sum-exp.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "focus_internal.h"

namespace focus {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;      // threads per workgroup
constexpr int ROWS = 128;    // query rows per workgroup (4 waves x 32)
constexpr int MAXSEG = 64;   // groups present in one sorted query tile (K <= 64)
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kProbSumCap = 256.0f;  // a lane's probability sum that triggers a rescale
constexpr int kNoPos = 0x7fffffff;      // position of a padding key slot

// kLongMulti: the long-range pass over membership entries, two groups per
// token (K >= 5): launched once per membership index, over the tokens' first
// then second group.
// kLongSets: the long-range pass with two groups per token and few groups
// (K <= 4), over tokens sorted by their membership set.
// kSoftGate + s (s = 0, 1, 2): the training-time soft-gated pass over every
// causal pair, with soft assignments of KG = 16 << s columns (zero-padded).
enum { kWindow = 0, kLongRange = 1, kDense = 2, kLongMulti = 3, kSoftGate = 4, kLongSets = 7 };
constexpr bool attn_gated(int PHASE) { return PHASE >= kSoftGate && PHASE < kLongSets; }

// Division by a divisor fixed for the launch (the work decode's tile, slice
// and head counts): floor(x / d) for any 32-bit x as a multiply-high, an add
// and two shifts, with the multiplier m = floor(2^32 (2^l - d) / d) + 1,
// l = ceil(log2 d), computed on the host (division by invariant integers,
// Granlund and Montgomery, PLDI 1994). d = 1 takes x itself.
struct FastDiv {
    uint32_t mul, shr, d;
};
inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f{0u, 0u, d};
    if (d <= 1) return f;
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    f.mul = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
    f.shr = l;
    return f;
}
__device__ __forceinline__ uint32_t fast_div(uint32_t x, const FastDiv& f) {
    if (f.d <= 1) return x;
    const uint32_t t = __umulhi(x, f.mul);
    return (t + ((x - t) >> 1)) >> (f.shr - 1);
}

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k;      // sequence order (window / dense) or sorted copy (long-range)
    const uint16_t* v;
    const int32_t* ids;
    const int32_t* perm;    // sorted key order (long-range passes)
    const int32_t* offsets;
    const int32_t* qperm;   // entry passes: the query order's entries [B][2n]
    int half;               // entry passes: membership index of this launch's query rows
    const int32_t* plan;    // long-range tile plan [B][tiles][PLAN_INTS] (entry passes:
                            // [B][2][ntiles][PLAN_INTS], one half per membership index)
    const int32_t* order;   // long-range pass: sorted query tiles, most work first [B][ntiles]
    const int32_t* pack;    // long-range pass (one group per token): a record per ordered tile
    int pack_ints;          // ints per packed record
    int32_t* spos;          // positions of sorted slots, [B][n + KPOS_PAD], padded kNoPos
    int set_lut;            // set pass: group mask of membership set s in bits 4s .. 4s+3
    _Float16* og;           // window partial [B][Hq][n][D]: O * 2^-e in fp16 (|.| < 1)
    f32x2* lseg;            // per row (log2-sum-exp L or -inf: no key, e)
    _Float16* og_dst;       // where a partial is written (og, except in the first entry
    f32x2* lseg_dst;        // pass, which must not overwrite the partial it merges)
    void* out;
    float* lse;
    int B, Hq, Hkv, n, K, w;
    int ne;        // slots of the sorted key order: n, or n*2 entries in the entry passes
    int hpk;       // Hq / Hkv
    int G;         // query heads packed per workgroup
    int TT;        // tokens per workgroup tile (ROWS / G, a power of two)
    int tt_log;    // log2(TT)
    int nslices;   // hpk / G
    int ntiles;    // ceil(n / TT): query tiles (of one launch)
    FastDiv fd_ntiles, fd_nslices, fd_hkv;   // the work decode's divisors
    int total;     // workgroups
    float sl2;     // scale * log2(e)
    const uint16_t* gs;   // soft-gated pass: bf16 hi/lo split of the soft assignments,
                          // [B][n][2][KG] (hi row, then lo row)
    float nl2;            // soft-gated pass: -lambda * log2(e)
    int out_f32;
    int merge;     // start from the partial in og/lseg (row of the original position)
    int direct;    // long-range pass, one group per token: k and v are the sequence-order
                   // tensors and key rows are read at their positions (perm), not copied
    int partial;   // write the normalised partial to og/lseg instead of out/lse
};

// Workgroups per CU each attention kernel is built for: three (one can
// wait on memory while two compute) wherever the registers fit, i.e. all but
// the dense pass at d = 128. Keys per tile: 32 at three workgroups per CU
// for d = 64/128 (LDS and registers), 64 otherwise.
constexpr int attn_occupancy(int D, int PHASE) {
    return attn_gated(PHASE) ? 2 : ((D == 128 && PHASE == kDense) ? 2 : 3);
}
constexpr int attn_tile_keys(int D, int PHASE) {
    if (attn_gated(PHASE)) return D == 32 ? 64 : 32;   // registers for the gate operands
    return (D != 32 && attn_occupancy(D, PHASE) == 3) ? 32 : 64;
}

template <int D, int BN_ = 64>
struct Geom {
    static constexpr int BN = BN_;                            // keys per tile
    static constexpr int KB = BN / 32;                        // 32-key MFMA blocks per tile
    static constexpr int NCH = D / 8;                         // 16-byte chunks per row
    static constexpr int ROWB = D * 2;                        // bytes per row
    static constexpr int TILEB = BN * ROWB;                   // bytes of one K or V tile
    static constexpr int NI = TILEB / (4 * 1024);             // 1 KB copies per wave per tile
    static constexpr int KS = D / 16;                         // k-steps of S^T = K Q^T
    static constexpr int DB = D / 32;                         // 32-wide blocks of O^T
    static constexpr bool QSTAGE = 128 * ROWB <= 2 * TILEB;   // Q tile fits buffer 1
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

// Swizzle of the soft-gated pass's assignment rows in LDS (GNCH 16-byte
// chunks per row): the 16 consecutive rows that one quarter-wave reads at
// the same logical chunk land in 16 distinct bank groups.
template <int GNCH>
__device__ __forceinline__ int gswz(int r) {
    return GNCH >= 16 ? (r & 15) : ((r * GNCH / 16) & (GNCH - 1));
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

// 16-byte buffer -> LDS copy: lane l reads base + soff + voff (a 32-bit
// per-lane offset) and lands at lds_base + 16*l. The buffer resource holds
// the base and the byte size in scalar registers; reads past the size
// return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ void copy16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                           void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, soff, 0, 0);
}

// Workgroups are dealt round-robin to the 8 XCDs; renumber them so each XCD
// works through one contiguous range of work items (neighbouring tiles of one
// head share keys in that XCD's L2).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int per = total / 8, rem = total % 8;
    const int x = bid % 8, local = bid / 8;
    return x * per + (x < rem ? x : rem) + local;
}

// ---------------------------------------------------------------------------
// Sorted copies for the long-range pass: k_s[b][h][s] = k[b][h][pos(s)]
// (same for v), one 16-byte chunk per thread, and spos[b][s] followed by
// KPOS_PAD padding slots (kNoPos), written by the kv-head-0 grid row. Slot s
// holds entry e = perm[b][s] of token pos(s) = e / m. With one group per
// token spos is the position; with two it is position * 64 + the token's
// other group (the pair rule needs both).
__global__ __launch_bounds__(256) void attn_gather_kernel(const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const int32_t* __restrict__ perm,
                                                          const int32_t* __restrict__ ids,
                                                          int n, int ne, int m, int K, int Hkv,
                                                          int D, uint16_t* __restrict__ ks,
                                                          uint16_t* __restrict__ vs,
                                                          int32_t* __restrict__ spos) {
    const int nch = D / 8;
    const int bh = blockIdx.y, b = bh / Hkv, h = bh % Hkv;
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t s = x / nch;
    const int c = (int)(x % nch);
    if (s >= ne + KPOS_PAD) return;
    if (s >= ne) {
        if (h == 0 && c == 0) spos[(int64_t)b * (ne + KPOS_PAD) + s] = kNoPos;
        return;
    }
    const int e = clampi(perm[(int64_t)b * ne + s], 0, ne - 1);
    const int pos = e / m;
    if (h == 0 && c == 0) {
        int val = pos;
        if (m == 2) val = (pos << 6) | clampi(ids[(int64_t)b * ne + (e ^ 1)], 0, K - 1);
        spos[(int64_t)b * (ne + KPOS_PAD) + s] = val;
    }
    const int64_t src = (int64_t)bh * n * D + (int64_t)pos * D + c * 8;
    const int64_t dst = ((int64_t)bh * ne + s) * D + c * 8;
    *reinterpret_cast<u32x4*>(ks + dst) = *reinterpret_cast<const u32x4*>(k + src);
    *reinterpret_cast<u32x4*>(vs + dst) = *reinterpret_cast<const u32x4*>(v + src);
}

// Key slots [ob, kend) that group g contributes to the long-range pass of
// the sorted query slots [s0, s1): the group's segment [ob, oe) of perm, cut
// at the first slot whose position is >= (largest query position of g in the
// tile) - w. Positions increase inside a segment, so that cut is a binary
// search, and no later slot of the segment can pair with any query of g here.
// kfull: slots below it pair with every query of g in the tile (position
// below (smallest query position) - w).
__device__ __forceinline__ int first_slot_at_or_above(const int32_t* perm_b, int lo, int hi,
                                                      int bound) {
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (perm_b[mid] < bound) lo = mid + 1; else hi = mid;
    }
    return lo;
}
__device__ __forceinline__ void segment_range(const int32_t* perm_b, const int32_t* offb, int ne,
                                              int w, int s0, int s1, int g, int& ob, int& kend,
                                              int& kfull) {
    ob = clampi(offb[g], 0, ne);
    const int oe = clampi(offb[g + 1], ob, ne);
    const int qlo = max(s0, ob), qhi = min(s1, oe);
    kend = ob;
    kfull = ob;
    if (qlo < qhi) {
        const int maxpos = clampi(perm_b[qhi - 1], 0, ne - 1);
        const int minpos = clampi(perm_b[qlo], 0, ne - 1);
        kend = first_slot_at_or_above(perm_b, ob, qhi, maxpos - w);
        kfull = first_slot_at_or_above(perm_b, ob, kend, minpos - w);
    }
}

// Entry passes (two groups per token, K >= 5). The key order is the sort
// of the n*2 membership entries e = t*2 + c by group (position t = e / 2,
// increasing inside a group's segment); the query rows of a tile are
// entries of one membership index c, taken in key order, so the rows of
// one group are consecutive there too. Group g's key slots for the tile's
// rows of g, at positions minpos .. maxpos: [ob, kend), kend the first slot
// of the segment at a position >= maxpos - w; kfull: the slots below
// position minpos - w, kept by every such row (up to the pair rule). An
// entry is below 2 * bound exactly when its position is below bound.
__device__ __forceinline__ void entry_segment(const int32_t* perm_b, const int32_t* offb, int ne,
                                              int w, int g, bool rows, int minpos, int maxpos,
                                              int& ob, int& kend, int& kfull) {
    ob = clampi(offb[g], 0, ne);
    const int oe = clampi(offb[g + 1], ob, ne);
    kend = ob;
    kfull = ob;
    if (rows) {
        kend = first_slot_at_or_above(perm_b, ob, oe, 2 * (maxpos - w));
        kfull = first_slot_at_or_above(perm_b, ob, kend, 2 * (minpos - w));
    }
}

// Entry passes: the membership index of each key slot (okey[b][s] = the
// entry's c), to sort the key slots stably by it into the query order.
__global__ __launch_bounds__(256) void attn_entry_index_kernel(const int32_t* __restrict__ perm,
                                                               int64_t slots,
                                                               int32_t* __restrict__ okey) {
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (x < slots) okey[x] = perm[x] & 1;
}

// Entry passes: the query order's entries, qent[b][u] = perm[b][operm[b][u]]
// (operm: the key slots stably sorted by membership index).
__global__ __launch_bounds__(256) void attn_entry_query_kernel(const int32_t* __restrict__ perm,
                                                               const int32_t* __restrict__ operm,
                                                               int ne, int64_t slots,
                                                               int32_t* __restrict__ qent) {
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (x >= slots) return;
    const int64_t b = x / ne;
    qent[x] = perm[b * ne + clampi(operm[x], 0, ne - 1)];
}

// Entry passes: one plan record per query tile of each half (tile j of
// half c holds query slots c*n + j*TT .. c*n + min(n, (j+1)*TT) - 1),
// shared by every kv head, laid out as attn_plan_kernel's records over
// [B][2][T] tiles: the groups gf .. gl of the tile's rows, each with its key
// slots (entry_segment), its first tile index and kfull.
__global__ __launch_bounds__(256) void attn_entry_plan_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ qent, int n, int K, int w,
    int TT, int T, int bn_keys, int32_t* __restrict__ plan) {
    const int b = blockIdx.y;
    const int u = blockIdx.x * 256 + threadIdx.x;
    if (u >= 2 * T) return;
    const int c = u / T, j = u % T;
    const int ne = 2 * n;
    const int64_t bne = (int64_t)b * ne;
    const int32_t* perm_b = perm + bne;
    const int32_t* qb = qent + bne;
    const int32_t* offb = offsets + (int64_t)b * (K + 1);
    const int s0 = c * n + j * TT, s1 = c * n + min(n, (j + 1) * TT);
    auto entry = [&](int s) { return clampi(qb[s], 0, ne - 1); };
    auto group = [&](int e) { return clampi(ids[bne + e], 0, K - 1); };
    const int gf = group(entry(s0));
    const int gl = max(gf, group(entry(s1 - 1)));
    const int nseg = gl - gf + 1;
    int32_t* rec = plan + ((int64_t)b * 2 * T + u) * PLAN_INTS;
    int run = 0;
    int s = s0;   // first row of the current group
    for (int t = 0; t < nseg; ++t) {
        const int g = gf + t;
        int se = s;
        while (se < s1 && group(entry(se)) == g) ++se;
        const bool rows = se > s;
        int ob, kend, kfull;
        entry_segment(perm_b, offb, ne, w, g, rows, rows ? entry(s) >> 1 : 0,
                      rows ? entry(se - 1) >> 1 : 0, ob, kend, kfull);
        if (nseg <= SEGCAP) {
            rec[4 + 4 * t] = ob;
            rec[5 + 4 * t] = kend;
            rec[6 + 4 * t] = run;
            rec[7 + 4 * t] = kfull;
        }
        run += (kend - ob + bn_keys - 1) / bn_keys;
        s = se;
    }
    // more groups than a record holds: the attention kernel derives them
    rec[0] = nseg <= SEGCAP ? nseg : -1;
    rec[1] = gf;
    rec[2] = gf == gl ? 1 : 0;
    rec[3] = run;
}

// Long-range pass with one group per token: one record per ordered query
// tile j (the tile order[j]), so that the attention kernel finds at a fixed
// address everything its prologue needs before the first key tile, in one
// round trip rather than a chain of dependent loads (order, then perm, plan
// and row ends, then the first key tile's positions):
//   [0, 32)             the tile's plan record
//   [32]                the tile's index
//   [64, 64+TT)         its rows' entries (sorted slot -> position)
//   [64+TT, 64+2TT)     each row's key-slot end: the first slot of its
//                       group's segment whose position is >= its position -
//                       w (positions increase inside a segment, so this is a
//                       binary search over [segment start, slot)); a partial
//                       key tile is then masked by comparing slot indices
//   [64+2TT, 64+2TT+BN) the positions of the rows of the first key tile the
//                       tile visits (the first non-empty segment's first BN
//                       slots, clamped to its valid slots)
// Rows past the sequence end take the last slot's values.
__global__ __launch_bounds__(256) void attn_pack_kernel(
    const int32_t* __restrict__ plan, const int32_t* __restrict__ order,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, int n, int K, int w, int TT, int BN, int ntiles, int pi,
    int32_t* __restrict__ pack) {
    const int j = blockIdx.x, b = blockIdx.y;
    const int tile = clampi(order[(int64_t)b * ntiles + j], 0, ntiles - 1);
    const int32_t* src = plan + ((int64_t)b * ntiles + tile) * PLAN_INTS;
    int32_t* dst = pack + ((int64_t)b * ntiles + j) * pi;
    const int32_t* perm_b = perm + (int64_t)b * n;
    int ob0 = 0, kend0 = 0;   // the first segment with key tiles (none: ob0 = kend0)
    const int nseg = min(src[0], SEGCAP);
    for (int t = 0; t < nseg; ++t) {
        const int ob = src[4 + 4 * t], ke = src[5 + 4 * t];
        if (ke > ob) {
            ob0 = ob;
            kend0 = ke;
            break;
        }
    }
    for (int i = threadIdx.x; i < pi; i += 256) {
        int val = 0;
        if (i < PLAN_INTS) {
            val = src[i];
        } else if (i == PLAN_INTS) {
            val = tile;
        } else if (i >= 64 && i < 64 + TT) {
            val = perm_b[min(tile * TT + (i - 64), n - 1)];
        } else if (i >= 64 + TT && i < 64 + 2 * TT) {
            const int slot = min(tile * TT + (i - 64 - TT), n - 1);
            const int pos = clampi(perm_b[slot], 0, n - 1);
            const int g = clampi(ids[(int64_t)b * n + pos], 0, K - 1);
            const int ob = clampi(offsets[(int64_t)b * (K + 1) + g], 0, slot);
            val = first_slot_at_or_above(perm_b, ob, slot, pos - w);
        } else if (i >= 64 + 2 * TT && i < 64 + 2 * TT + BN && kend0 > ob0) {
            val = perm_b[clampi(min(ob0 + (i - 64 - 2 * TT), kend0 - 1), 0, n - 1)];
        }
        dst[i] = val;
    }
}

// ---------------------------------------------------------------------------
// Two groups per token with few groups (K <= 4, at most 6 membership sets):
// tokens are sorted by their membership set {a, b}, and a query tile of set
// S visits the key segments of every set that shares a group with S. Each
// kept pair then meets exactly once, in the query's tile, and the pass can
// merge the window partial and write the result itself.
//
// Set id of the unordered pair a < b of K groups: the pairs in lexicographic
// order, (0,1) = 0, (0,2) = 1, ...
__device__ __forceinline__ int pair_set_id(int a, int b, int K) {
    return a * K - a * (a + 1) / 2 + (b - a - 1);
}
__device__ __forceinline__ int token_group_mask(const int32_t* ids_t, int K) {
    return (1 << clampi(ids_t[0], 0, K - 1)) | (1 << clampi(ids_t[1], 0, K - 1));
}
// sid[t] = set id of token t's two groups (ids [B*n][2]), clamped to [0, S).
__global__ __launch_bounds__(256) void attn_set_id_kernel(const int32_t* __restrict__ ids,
                                                          int64_t ntok, int K, int S,
                                                          int32_t* __restrict__ sid) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= ntok) return;
    const int g0 = clampi(ids[2 * t], 0, K - 1), g1 = clampi(ids[2 * t + 1], 0, K - 1);
    sid[t] = clampi(pair_set_id(min(g0, g1), max(g0, g1), K), 0, S - 1);
}
// Per set-sorted slot s: (position << 6) | the token's group mask, then
// KPOS_PAD padding slots (kNoPos): the keys' data for masking partial tiles.
__global__ __launch_bounds__(256) void attn_set_spos_kernel(const int32_t* __restrict__ perm,
                                                            const int32_t* __restrict__ ids,
                                                            int n, int K,
                                                            int32_t* __restrict__ spos) {
    const int b = blockIdx.y;
    const int s = blockIdx.x * 256 + threadIdx.x;
    if (s >= n + KPOS_PAD) return;
    int val = kNoPos;
    if (s < n) {
        const int pos = clampi(perm[(int64_t)b * n + s], 0, n - 1);
        val = (pos << 6) | token_group_mask(ids + ((int64_t)b * n + pos) * 2, K);
    }
    spos[(int64_t)b * (n + KPOS_PAD) + s] = val;
}
// Plan record of a set-sorted query tile (same layout as attn_plan_kernel's):
// one segment per membership set t (so nseg = S and segment t is set t), with
// the key slots [ob, kend) of set t whose positions lie below (largest query
// position of the tile) - w when set t shares a group with some row of the
// tile, and none otherwise; kfull: slots below it pair with every row (all
// rows of one set, positions below (smallest query position) - w).
__global__ __launch_bounds__(256) void attn_set_plan_kernel(
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ ids, int n, int K, int S, int w, int TT, int ntiles,
    int bn_keys, int set_lut, int32_t* __restrict__ plan) {
    const int b = blockIdx.y;
    const int tile = blockIdx.x * 256 + threadIdx.x;
    if (tile >= ntiles) return;
    const int32_t* perm_b = perm + (int64_t)b * n;
    const int32_t* offb = offsets + (int64_t)b * (S + 1);
    const int s0 = tile * TT, s1 = min(n, s0 + TT);
    int umask = 0, mask0 = -1, minpos = n, maxpos = 0;
    bool one_set = true;
    for (int sl = s0; sl < s1; ++sl) {
        const int pos = clampi(perm_b[sl], 0, n - 1);
        const int mk = token_group_mask(ids + ((int64_t)b * n + pos) * 2, K);
        if (mask0 < 0) mask0 = mk;
        one_set = one_set && mk == mask0;
        umask |= mk;
        minpos = min(minpos, pos);
        maxpos = max(maxpos, pos);
    }
    int32_t* rec = plan + ((int64_t)b * ntiles + tile) * PLAN_INTS;
    int run = 0;
    for (int t = 0; t < S; ++t) {
        const int ob = clampi(offb[t], 0, n);
        const int oe = clampi(offb[t + 1], ob, n);
        int kend = ob, kfull = ob;
        if (((set_lut >> (4 * t)) & 15) & umask) {
            kend = first_slot_at_or_above(perm_b, ob, oe, maxpos - w);
            kfull = first_slot_at_or_above(perm_b, ob, kend, minpos - w);
        }
        rec[4 + 4 * t] = ob;
        rec[5 + 4 * t] = kend;
        rec[6 + 4 * t] = run;
        rec[7 + 4 * t] = kfull;
        run += (kend - ob + bn_keys - 1) / bn_keys;
    }
    rec[0] = S;
    rec[1] = 0;
    rec[2] = one_set ? 1 : 0;
    rec[3] = run;
}

// Tile plan of the long-range pass with one group per token, once per
// (batch, sorted query tile) and shared by every kv head: record = {nseg
// (-1: more than SEGCAP groups, the attention kernel then derives its
// segments itself), first group, all query rows in one group, key tiles in
// total, then per group (ob, kend, first tile index, kfull)}.
__global__ __launch_bounds__(256) void attn_plan_kernel(const int32_t* __restrict__ ids,
                                                        const int32_t* __restrict__ perm,
                                                        const int32_t* __restrict__ offsets,
                                                        int ne, int K, int w, int TT,
                                                        int ntiles, int bn_keys,
                                                        int32_t* __restrict__ plan) {
    const int b = blockIdx.y;
    const int tile = blockIdx.x * 256 + threadIdx.x;
    if (tile >= ntiles) return;
    const int64_t bne = (int64_t)b * ne;
    const int32_t* perm_b = perm + bne;
    const int32_t* offb = offsets + (int64_t)b * (K + 1);
    const int s0 = tile * TT, s1 = min(ne, s0 + TT);
    const int gf = clampi(ids[bne + clampi(perm_b[s0], 0, ne - 1)], 0, K - 1);
    const int gl = clampi(ids[bne + clampi(perm_b[s1 - 1], 0, ne - 1)], gf, K - 1);
    const int nseg = gl - gf + 1;
    int32_t* rec = plan + ((int64_t)b * ntiles + tile) * PLAN_INTS;
    if (nseg > SEGCAP) {
        // too many groups for the record: the attention kernel derives the
        // segments itself; only the tile's total work is kept (for the order)
        int run = 0;
        for (int t = 0; t < nseg; ++t) {
            int ob, kend, kfull;
            segment_range(perm_b, offb, ne, w, s0, s1, gf + t, ob, kend, kfull);
            run += (kend - ob + bn_keys - 1) / bn_keys;
        }
        rec[0] = -1;
        rec[3] = run;
        return;
    }
    int run = 0;
    for (int t = 0; t < nseg; ++t) {
        int ob, kend, kfull;
        segment_range(perm_b, offb, ne, w, s0, s1, gf + t, ob, kend, kfull);
        rec[4 + 4 * t] = ob;
        rec[5 + 4 * t] = kend;
        rec[6 + 4 * t] = run;
        rec[7 + 4 * t] = kfull;
        run += (kend - ob + bn_keys - 1) / bn_keys;
    }
    const int ob0 = clampi(offb[gf], 0, ne), oe0 = clampi(offb[gf + 1], ob0, ne);
    rec[0] = nseg;
    rec[1] = gf;
    rec[2] = (s0 >= ob0 && s1 <= oe0) ? 1 : 0;
    rec[3] = run;
}

// Order in which the long-range pass takes the sorted query tiles of one
// batch element: by decreasing work class (1 + floor(log2(key tiles)), 0 for
// none), then by tile index; so the longest tiles start first and the
// grid's tail is made of short ones. One workgroup per batch element: each
// thread counts the classes of a contiguous chunk of tiles, the counts are
// scanned per class, and every thread writes its chunk in order (stable,
// deterministic).
constexpr int ORDER_CLASSES = 17;
__device__ __forceinline__ int work_class(int work) {
    return work <= 0 ? 0 : min(ORDER_CLASSES - 1, 32 - __clz(work));
}
__global__ __launch_bounds__(256) void attn_order_kernel(const int32_t* __restrict__ plan,
                                                         int ntiles,
                                                         int32_t* __restrict__ order) {
    __shared__ int cnt[ORDER_CLASSES][256];
    __shared__ int base[ORDER_CLASSES];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int chunk = (ntiles + 255) / 256;
    const int t0 = min(ntiles, tid * chunk), t1 = min(ntiles, t0 + chunk);
    const int32_t* pb = plan + (int64_t)b * ntiles * PLAN_INTS;
    for (int c = 0; c < ORDER_CLASSES; ++c) cnt[c][tid] = 0;
    for (int t = t0; t < t1; ++t) ++cnt[work_class(pb[(int64_t)t * PLAN_INTS + 3])][tid];
    __syncthreads();
    if (tid < ORDER_CLASSES) {
        // exclusive prefix over threads, per class
        int run = 0;
        for (int j = 0; j < 256; ++j) {
            const int x = cnt[tid][j];
            cnt[tid][j] = run;
            run += x;
        }
        base[tid] = run;   // class total for now
    }
    __syncthreads();
    if (tid == 0) {
        // classes from the highest down
        int run = 0;
        for (int c = ORDER_CLASSES - 1; c >= 0; --c) {
            const int tot = base[c];
            base[c] = run;
            run += tot;
        }
    }
    __syncthreads();
    int32_t* ob = order + (int64_t)b * ntiles;
    for (int t = t0; t < t1; ++t) {
        const int c = work_class(pb[(int64_t)t * PLAN_INTS + 3]);
        ob[base[c] + cnt[c][tid]++] = t;
    }
}

// ---------------------------------------------------------------------------
template <int D, int PHASE>
__global__ __launch_bounds__(NT, attn_occupancy(D, PHASE)) void attn_kernel(AttnArgs a) {
    using G = Geom<D, attn_tile_keys(D, PHASE)>;
    constexpr int BN = G::BN;
    constexpr bool SORTED = PHASE == kLongRange || PHASE == kLongMulti || PHASE == kLongSets;
    constexpr bool MULTI = PHASE == kLongMulti;   // entries of two groups per token
    constexpr bool SETS = PHASE == kLongSets;     // tokens sorted by membership set
    constexpr bool KPOS = MULTI || SETS;          // partial tiles masked by staged key data
    // single-group long-range pass: work item = ordered slot of a packed record
    constexpr bool PACKED = PHASE == kLongRange;
    static_assert(!PACKED || BN == attn_long_range_tile_keys(D), "packed record tile size");
    constexpr bool GATED = attn_gated(PHASE);
    constexpr bool CAUSAL_ALL = PHASE == kDense || GATED;   // key range [0, last row]
    // soft-gated pass: assignment columns (padded), bytes per key row of the
    // hi/lo split, 16-byte chunks per row, 1 KB copies per key tile
    constexpr int KG = GATED ? (16 << (PHASE - kSoftGate)) : 16;
    constexpr int GROWB = 4 * KG;
    constexpr int GNCH = GROWB / 16;
    constexpr int GNC = BN * GROWB / 1024;
    // slots of the sorted key order (n except in the entry passes: n*2)
    const int ne = MULTI ? a.ne : a.n;
    // Two K/V buffers, [K tile | V tile] each. In the sorted passes they are
    // two LDS variables: the compiler then sees that reads of one buffer
    // never meet the copies into the other and does not wait for those
    // copies before the reads (in the single-group pass, which copies no key
    // positions, this takes the wait for the next tile's copy out of every
    // tile; the other passes measured no gain from it and keep one variable).
    // Buffer 1 also stages the Q tile in the prologue; the epilogue stages
    // output rows in both (the first half of the rows in buffer 0).
    constexpr bool SPLIT = SORTED;
    __shared__ __attribute__((aligned(1024))) unsigned char buf0[(SPLIT ? 2 : 4) * G::TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char buf1_split[SPLIT ? 2 * G::TILEB : 16];
    unsigned char* const buf1 = SPLIT ? buf1_split : buf0 + 2 * G::TILEB;
    // multi pass: positions (and other groups) of the key slots of a partial tile
    __shared__ __attribute__((aligned(1024))) int kpos0[KPOS ? KPOS_PAD : 4],
        kpos1[KPOS ? KPOS_PAD : 4];
    // soft-gated pass: the key tile's assignment rows, one buffer per K/V buffer
    __shared__ __attribute__((aligned(1024))) unsigned char gk_lds[GATED ? 2 * BN * GROWB : 16];
    __shared__ int seg_ob[MAXSEG], seg_kend[MAXSEG], seg_t0[MAXSEG + 1], seg_kfull[MAXSEG];
    __shared__ int rowpos[ROWS];  // entry (= position with one group) of each query row (sorted pass)
    __shared__ int excl_any;      // multi pass: some row can meet a pair shared twice

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = lane & 31, hh = lane >> 5;

    // Work item of this workgroup. The indices are uniform; readfirstlane
    // keeps them (and every address derived from them) in scalar registers.
    const int L = xcd_remap(blockIdx.x, a.total);
    // Sequence-order passes take their query tiles last to first: the later
    // tiles have the most keys (causal passes) or the full window, so the
    // grid's last round is made of the short first tiles (longest first).
    const uint32_t q1 = fast_div((uint32_t)L, a.fd_ntiles);
    const uint32_t q2 = fast_div(q1, a.fd_nslices);
    const uint32_t q3 = fast_div(q2, a.fd_hkv);
    int tile = (int)((uint32_t)L - q1 * (uint32_t)a.ntiles);
    if (!SORTED) tile = a.ntiles - 1 - tile;
    int slice = (int)(q1 - q2 * (uint32_t)a.nslices);
    int kvh = (int)(q2 - q3 * (uint32_t)a.Hkv);
    int b = (int)q3;
    slice = __builtin_amdgcn_readfirstlane(slice);
    kvh = __builtin_amdgcn_readfirstlane(kvh);
    b = __builtin_amdgcn_readfirstlane(b);
    // plan and order rows of this launch: per batch element, or per (batch
    // element, half) in the entry passes
    const int pbi = MULTI ? 2 * b + a.half : b;
    const int R = wave * 32 + rl;
    const int hslot = R >> a.tt_log, tok = R & (a.TT - 1);
    // Packed pass: every load the prologue needs before the first key tile
    // is at a fixed address in the item's record, so they form one round
    // trip: lanes 0-15 of every wave hold record ints 4l .. 4l+3 (lane 0 the
    // header, lane t + 1 segment t, lane 8 the tile index), every lane its
    // row's entry and key-slot end and its rows of the first key tile.
    const int32_t* rec = nullptr;
    i32x4 prec = {0, 0, 0, 0};
    int ent_pk = 0, kend_pk = 0;
    int pos0_pk[G::NI];
    if (PACKED) {
        rec = a.pack + ((int64_t)b * a.ntiles + tile) * a.pack_ints;
        prec = *reinterpret_cast<const i32x4*>(rec + 4 * (lane & 15));
        ent_pk = rec[64 + tok];
        kend_pk = rec[64 + a.TT + tok];
#pragma unroll
        for (int i = 0; i < G::NI; ++i)
            pos0_pk[i] = rec[64 + 2 * a.TT + ((wave * G::NI + i) * 1024 + 16 * lane) / G::ROWB];
        tile = clampi(__builtin_amdgcn_readlane(prec[0], 8), 0, a.ntiles - 1);
    } else if (SORTED) {
        tile = clampi(a.order[(int64_t)pbi * a.ntiles + tile], 0, a.ntiles - 1);
    }
    tile = __builtin_amdgcn_readfirstlane(tile);

    const int h = kvh * a.hpk + slice * a.G + hslot;
    const int64_t bne = (int64_t)b * ne;
    // the tile's query slots [qs0, qs1) (entry passes: in the half of this
    // launch's membership index)
    const int qs0 = (MULTI ? a.half * a.n : 0) + tile * a.TT;
    const int qs1 = MULTI ? a.half * a.n + min(a.n, (tile + 1) * a.TT) : min(ne, qs0 + a.TT);
    const int s_row = qs0 + tok;
    const bool rvalid = s_row < qs1;
    // entry of the row (sorted passes: perm holds entries t*m + c; m = 1
    // makes the entry the position) and its sequence position
    int ent_i = rvalid ? s_row : 0;
    // Sorted passes: every row has an entry (rows past the end take the last
    // slot's, a valid position they never store to).
    if (PACKED) ent_i = clampi(ent_pk, 0, ne - 1);
    else if (MULTI) ent_i = clampi(a.qperm[bne + min(s_row, qs1 - 1)], 0, ne - 1);
    else if (SORTED) ent_i = clampi(a.perm[bne + min(s_row, ne - 1)], 0, ne - 1);
    // long-range pass: the end of the row's key slots (a partial tile is
    // masked by slot index)
    int kend_row = 0;
    if (PACKED) kend_row = clampi(kend_pk, 0, ne);
    // Multi and set passes: the tile's plan record, loaded beside the perm
    // entry so that the two round trips overlap. Lane l < 8 of every wave
    // holds ints 4l .. 4l+3: lane 0 the header, lane t + 1 segment t.
    if (MULTI || SETS)
        prec = *reinterpret_cast<const i32x4*>(a.plan + ((int64_t)pbi * a.ntiles + tile) * PLAN_INTS +
                                              4 * (lane & 7));
    const int pos_i = MULTI ? (ent_i >> 1) : ent_i;
    // Sequence-order passes: the positions of the wave's valid rows form one
    // run [wpmin, wpmax] (32 consecutive tokens of the tile, or all TT
    // tokens when the wave spans several heads), so whether the wave keeps
    // any key of a tile is a scalar test.
    int wpmin = 0, wpmax = -1;
    if constexpr (!SORTED) {
        const int w0 = a.TT >= 32 ? ((__builtin_amdgcn_readfirstlane(wave) * 32) & (a.TT - 1)) : 0;
        wpmin = qs0 + w0;
        wpmax = min(qs1 - 1, qs0 + w0 + min(32, a.TT) - 1);
    }
    // multi pass: the row token's other group
    const int oth_i = (MULTI && rvalid) ? clampi(a.ids[bne + (ent_i ^ 1)], 0, a.K - 1) : 0;
    // set pass: the row token's group mask (a key is kept when it shares one)
    const int gmask_i = SETS ? token_group_mask(a.ids + ((int64_t)b * a.n + pos_i) * 2, a.K) : 0;

    const uint16_t* kbase = a.k + ((int64_t)b * a.Hkv + kvh) * ne * D;
    const uint16_t* vbase = a.v + ((int64_t)b * a.Hkv + kvh) * ne * D;

    // ---- the key tiles this workgroup visits: ntl tiles, tile tau at key
    // ---- slot kt0(tau), valid slots below kend(tau).
    int ntl = 0;
    int kstart = 0, kend0 = 0;               // sequence-order passes
    int gfirst = 0, g_i = -1;                // long-range pass
    int nseg_tile = 1;                       // long-range pass: group segments of this tile
    int x_i = -1;                            // multi pass: excluded key group, or -1
    bool rows_one_group = false, rows_excl = false;
    if (!SORTED) {
        const int q0 = tile * a.TT;
        const int qlast = min(a.n, q0 + a.TT) - 1;
        kstart = CAUSAL_ALL ? 0 : max(0, q0 - a.w);
        kend0 = qlast + 1;
        ntl = (kend0 - kstart + BN - 1) / BN;
    } else {
        const int s0 = qs0, s1 = qs1;
        if (hh == 0) rowpos[R] = ent_i;  // published by the barrier below
        if (MULTI && tid == 0) excl_any = 0;
        // the header is uniform: readlane keeps it in scalar registers
        int nseg = __builtin_amdgcn_readlane(prec[0], 0);
        if (nseg >= 0) {
            nseg = min(nseg, SEGCAP);
            gfirst = clampi(__builtin_amdgcn_readlane(prec[1], 0), 0, a.K - 1);
            rows_one_group = __builtin_amdgcn_readlane(prec[2], 0) != 0;
            const int t = lane - 1;   // segment held by this lane
            if (wave == 0 && t >= 0 && t < nseg) {
                const int ob = clampi(prec[0], 0, ne);
                const int kend = clampi(prec[1], ob, ne);
                seg_ob[t] = ob;
                seg_kend[t] = kend;
                seg_t0[t] = prec[2];
                seg_kfull[t] = clampi(prec[3], ob, kend);
            }
            if (tid == 0) seg_t0[nseg] = prec[3];
            __syncthreads();
        } else {
            // More groups in this tile than a plan record holds: derive the
            // segments here (every tile of them is treated as partial).
            const int32_t* offb = a.offsets + (int64_t)b * (a.K + 1);
            const int32_t* qord = MULTI ? a.qperm : a.perm;
            gfirst = __builtin_amdgcn_readfirstlane(
                clampi(a.ids[bne + clampi(qord[bne + s0], 0, ne - 1)], 0, a.K - 1));
            const int glast = __builtin_amdgcn_readfirstlane(
                clampi(a.ids[bne + clampi(qord[bne + s1 - 1], 0, ne - 1)], gfirst, a.K - 1));
            nseg = glast - gfirst + 1;
            if (MULTI) __syncthreads();   // rowpos: the rows' entries
            if (tid < nseg) {
                int ob, kend, kfull;
                if (MULTI) {
                    // this group's rows (consecutive) and their position range
                    const int g = gfirst + tid;
                    int lo = -1, hi = -1;
                    for (int r = 0; r < s1 - s0; ++r) {
                        const int e = rowpos[r];
                        if (clampi(a.ids[bne + e], 0, a.K - 1) == g) {
                            if (lo < 0) lo = e >> 1;
                            hi = e >> 1;
                        }
                    }
                    entry_segment(a.perm + bne, offb, ne, a.w, g, lo >= 0, lo, hi, ob, kend,
                                  kfull);
                } else {
                    segment_range(a.perm + bne, offb, ne, a.w, s0, s1, gfirst + tid, ob, kend,
                                  kfull);
                }
                seg_ob[tid] = ob;
                seg_kend[tid] = kend;
                seg_kfull[tid] = ob;
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
        }
        // Key tiles in total, bounded by what nseg segments of at most ne
        // slots each can hold, and the segment count kept for the cursor:
        // a plan that does not match the data gives wrong numbers, but the
        // loops below still end.
        nseg_tile = __builtin_amdgcn_readfirstlane(nseg);
        ntl = __builtin_amdgcn_readfirstlane(
            clampi(seg_t0[nseg], 0, nseg * ((ne + BN - 1) / BN)));
        // the row's group: its own (entry passes: the entry's group; else
        // the segment holding its slot, segments being consecutive in sorted
        // order), within the tile's segments
        if (rvalid) {
            if (MULTI) {
                g_i = clampi(a.ids[bne + ent_i], gfirst, gfirst + nseg - 1);
            } else {
                int t = 0;
                while (t + 1 < nseg && seg_ob[t + 1] <= s_row) ++t;
                g_i = gfirst + t;
            }
        }
        if (MULTI) {
            // A pair of tokens sharing both their groups meets in both
            // segments; it is kept only in the segment of the lower group.
            // Row i in segment g skips keys whose other group equals its own
            // other group when that group is below g.
            x_i = (rvalid && oth_i < g_i) ? oth_i : -1;
            if (x_i >= 0) excl_any = 1;
            __syncthreads();
            rows_excl = __builtin_amdgcn_readfirstlane(excl_any) != 0;
        }
    }
    // Set pass: the groups the wave's valid rows hold, a scalar bit mask
    // taken once per work item, so that the per-tile test of whether the
    // wave keeps any key of a segment is scalar.
    uint32_t wave_groups = 0;
    if constexpr (SETS) {
#pragma unroll
        for (int bit = 0; bit < 4; ++bit)
            if (__any(rvalid && ((gmask_i >> bit) & 1))) wave_groups |= 1u << bit;
    }

    // Sorted passes: a cursor over the segments, with the current segment's
    // values held in scalar registers (first and end tile, first key slot,
    // end of valid slots, end of the slots every row keeps); it is reloaded
    // from LDS only when a tile crosses into the next segment.
    struct SegCursor {
        int seg, t0, t1, ob, kend, kfull;
    };
    auto seg_load = [&](SegCursor& c) {
        // segment values are uniform (LDS, written by one thread each)
        c.t0 = __builtin_amdgcn_readfirstlane(seg_t0[c.seg]);
        c.t1 = __builtin_amdgcn_readfirstlane(seg_t0[c.seg + 1]);
        c.ob = __builtin_amdgcn_readfirstlane(seg_ob[c.seg]);
        c.kend = __builtin_amdgcn_readfirstlane(seg_kend[c.seg]);
        c.kfull = __builtin_amdgcn_readfirstlane(seg_kfull[c.seg]);
    };
    // Tile tau -> (segment, first key slot, end of valid slots, all pairs kept).
    auto locate = [&](int tau, SegCursor& c, int& kt0, int& kend, bool& full) {
        if (!SORTED) {
            kt0 = kstart + tau * BN;
            kend = kend0;
            const int q0 = tile * a.TT;
            full = (kt0 + BN - 1 <= q0) && (kt0 + BN <= kend) &&
                   (CAUSAL_ALL || kend - 1 - kt0 <= a.w);
        } else {
            while (c.t1 <= tau && c.seg + 1 < nseg_tile) {
                ++c.seg;
                seg_load(c);
            }
            kt0 = c.ob + (tau - c.t0) * BN;
            kend = c.kend;
            full = rows_one_group && !rows_excl && (kt0 + BN <= c.kfull);
        }
    };

    // This lane's share of a tile copy: NI rows (one per 1 KB copy) and the
    // logical chunk it fetches from each.
    // lane_off = byte offset of this lane's 16 bytes within a tile
    // (row * ROWB + 16 * logical chunk); unsigned, so a copy addresses
    // memory as a scalar tile base plus a 32-bit lane offset.
    uint32_t lane_off[G::NI];
#pragma unroll
    for (int i = 0; i < G::NI; ++i) {
        const int o = (wave * G::NI + i) * 1024 + 16 * lane;
        const int crow = o / G::ROWB;
        lane_off[i] = crow * G::ROWB + logical_chunk<D>(crow, (o % G::ROWB) / 16) * 16;
    }
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // wave index in a scalar register
    SegCursor seg_issue = {0, 0, 0, 0, 0, 0};
    if (SORTED && ntl > 0) seg_load(seg_issue);
    SegCursor seg_cur = seg_issue;
    // Long-range pass reading K and V rows in place (direct): the position
    // of each of this lane's NI rows of the next tile to copy, loaded from
    // perm one tile ahead (so the copy never waits for it), and a buffer
    // resource over the head's n rows.
    const bool direct = SORTED && !MULTI && a.direct;
    SegCursor seg_pref = seg_issue;
    int pnext[G::NI];
    const __amdgpu_buffer_rsrc_t krs_head =
        make_rsrc(kbase, direct ? (uint32_t)a.n * G::ROWB : 0u);
    const __amdgpu_buffer_rsrc_t vrs_head =
        make_rsrc(vbase, direct ? (uint32_t)a.n * G::ROWB : 0u);
    // The positions come through a buffer resource over the tile's valid
    // slots of the batch element's perm row (scalar base and size, built per
    // tile), so each lane's read is a fixed 32-bit offset; a slot past the
    // segment's valid end reads 0, a valid row, which the mask drops.
    auto prefetch = [&](int tau) {
        int kt0, kend;
        bool full;
        locate(tau, seg_pref, kt0, kend, full);
        const int s0 = min(max(kt0, 0), kend);
        const __amdgpu_buffer_rsrc_t prs =
            make_rsrc(a.perm + bne + s0, direct ? (uint32_t)(kend - s0) * 4u : 0u);
#pragma unroll
        for (int i = 0; i < G::NI; ++i)
            pnext[i] = __builtin_amdgcn_raw_buffer_load_b32(prs, (lane_off[i] / G::ROWB) * 4u, 0, 0);
    };
    // the first key tile's positions: from the packed record when the plan
    // record holds the segments (otherwise the kernel derived them itself)
    if (direct && ntl > 0) {
        if (PACKED && __builtin_amdgcn_readlane(prec[0], 0) >= 0) {
#pragma unroll
            for (int i = 0; i < G::NI; ++i) pnext[i] = pos0_pk[i];
        } else {
            prefetch(0);
        }
    }
    // soft-gated pass: this lane's share of the assignment-row copies (1 KB
    // copies wave, wave + 4, ...): key row within the tile and logical chunk
    constexpr int GCPW = (GNC + 3) / 4;
    int g_row[GCPW], g_chunk[GCPW];
#pragma unroll
    for (int i = 0; i < GCPW; ++i) {
        const int o = (wave + 4 * i) * 1024 + 16 * lane;
        g_row[i] = o / GROWB;
        g_chunk[i] = ((o % GROWB) / 16) ^ gswz<GNCH>(g_row[i]);
    }
    auto issue = [&](int tau, unsigned char* bufp, int* kposp) {
        int kt0, kend;
        bool full;
        locate(tau, seg_issue, kt0, kend, full);
        unsigned char* dst = bufp + wave_s * G::NI * 1024;
        // multi and set passes: the key slots' positions and group data, for
        // the mask of a partial tile (a scalar base plus a 32-bit lane offset,
        // like the tile copies: a per-lane 64-bit pointer here would be kept
        // across the loop, spilled, and its reload would wait for the copies
        // issued just before it). The single-group pass masks by slot index.
        if (KPOS && !full && wave == 0) {
            const char* sp = reinterpret_cast<const char*>(a.spos + (int64_t)b * (ne + KPOS_PAD));
            copy16(sp + (uint32_t)(4 * kt0 + 16 * lane), kposp);
        }
        if (direct) {
#pragma unroll
            for (int i = 0; i < G::NI; ++i) {
                // no clamp: the offset is 32-bit and the resource spans the
                // head's n rows, so no position reads outside them (one
                // outside [0, n) reads zeros, or another row if it wraps)
                const uint32_t vo = (uint32_t)pnext[i] * G::ROWB + lane_off[i] % G::ROWB;
                copy16_buf(krs_head, vo, 0, dst + i * 1024);
                copy16_buf(vrs_head, vo, 0, dst + G::TILEB + i * 1024);
            }
            if (tau + 1 < ntl) prefetch(tau + 1);
            return;
        }
        // The tile's K and V rows through buffer resources whose base is the
        // tile's first row (scalar registers) and whose size stops at the
        // sequence end; each lane adds its fixed 32-bit offset. In a tile that
        // runs past the sequence end, rows from kend on re-read row kend - 1
        // (they are masked).
        const int64_t tb = (int64_t)kt0 * D;
        const uint32_t nbytes = __builtin_amdgcn_readfirstlane(clampi(ne - kt0, 0, BN) * G::ROWB);
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase + tb, nbytes);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase + tb, nbytes);
        if (kt0 + BN <= ne) {
#pragma unroll
            for (int i = 0; i < G::NI; ++i) {
                copy16_buf(krs, lane_off[i], 0, dst + i * 1024);
                copy16_buf(vrs, lane_off[i], 0, dst + G::TILEB + i * 1024);
            }
        } else {
#pragma unroll
            for (int i = 0; i < G::NI; ++i) {
                const uint32_t r = min(lane_off[i] / G::ROWB, (uint32_t)max(kend - 1 - kt0, 0));
                const uint32_t vo = r * G::ROWB + lane_off[i] % G::ROWB;
                copy16_buf(krs, vo, 0, dst + i * 1024);
                copy16_buf(vrs, vo, 0, dst + G::TILEB + i * 1024);
            }
        }
        if constexpr (GATED) {
            // the key tile's assignment rows (hi and lo), row-clamped at the end
            unsigned char* gd = gk_lds + (bufp == buf0 ? 0 : BN * GROWB);
            const char* gbase = reinterpret_cast<const char*>(a.gs) + (int64_t)b * a.n * GROWB;
#pragma unroll
            for (int i = 0; i < GCPW; ++i) {
                if (wave_s + 4 * i < GNC) {
                    const int key = min(kt0 + g_row[i], a.n - 1);
                    copy16(gbase + (int64_t)key * GROWB + g_chunk[i] * 16,
                           gd + (wave_s + 4 * i) * 1024);
                }
            }
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

    // soft-gated pass: LDS offsets of this lane's assignment-row reads
    // (key rl, columns 16*ks + 8*hh .. +8 of the hi (part 0) or lo (part 1) half)
    int goff[KG / 16][2];
#pragma unroll
    for (int ks = 0; ks < KG / 16; ++ks)
#pragma unroll
        for (int part = 0; part < 2; ++part)
            goff[ks][part] = rl * GROWB + (((part * KG / 8) + 2 * ks + hh) ^ gswz<GNCH>(rl)) * 16;

    f32x16 acc[G::DB];   // the sorted passes set it from the partial they merge
    if constexpr (!SORTED) {
#pragma unroll
        for (int db = 0; db < G::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;
    }
    // l_run: sum of the fp32 probabilities (log-sum-exp); l_pv: sum of the
    // bf16-rounded probabilities the PV MFMAs multiply (output normaliser)
    float m_ref = kNegInf, l_run = 0.0f, l_pv = 0.0f;
    bf16x8 qf[G::KS];  // Q^T fragments, loaded once the first key tile is in flight
    bf16x8 gq[KG / 16][2];  // soft-gated pass: the row's assignment (hi, lo) fragments

    // Tile tau, located before the next tile's copy is issued (between the
    // copy and the tile's first LDS reads there is then no segment-cursor
    // loop, across which the compiler would wait for the copy to land).
    auto compute = [&](int tau, int kt0, int kend, bool full, const unsigned char* bufp,
                       const int* kposp) {
        // A wave none of whose rows keeps a key of this tile skips it (all
        // its products would be masked). With one query head per kv head
        // the four waves hold different tokens, so near either end of the
        // workgroup's key range, or in a segment of another group, some
        // waves have nothing to do; their SIMD serves the other workgroups.
        {
            bool needs;
            if (!SORTED) {
                if (!(wpmin <= wpmax && kt0 <= wpmax && (CAUSAL_ALL || kt0 + BN - 1 + a.w >= wpmin)))
                    return;
                needs = true;
            } else if (SETS) {
                // the segment's set shares a group with one of the wave's rows
                if ((wave_groups & (uint32_t)(a.set_lut >> (4 * seg_cur.seg)) & 15u) == 0) return;
                needs = true;
            } else if (!MULTI) {
                needs = rvalid && g_i == gfirst + seg_cur.seg && kt0 < kend_row;
            } else {
                needs = rvalid && g_i == gfirst + seg_cur.seg;
            }
            if (!__any(needs)) return;
        }
        // S^T = K Q^T for the tile's 32-key blocks.
        f32x16 st[G::KB];
#pragma unroll
        for (int kb = 0; kb < G::KB; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) st[kb][e] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < G::KS; ++ks) {
                const bf16x8 kf =
                    *reinterpret_cast<const bf16x8*>(bufp + kb * 32 * G::ROWB + koff[ks]);
                st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], st[kb], 0, 0, 0);
            }
        }
        // Schedule (DS-read group 0x100, MFMA group 0x008): keep three K
        // fragment reads in flight ahead of the S MFMAs, otherwise each MFMA
        // waits out a full LDS round trip.
        {
            constexpr int NS = G::KB * G::KS;
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (j + 3 < NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }

        // Mask (partial tiles only). Lane holds keys kidx = kb*32 +
        // 8*(e>>2) + 4*hh + (e&3) of its row, i.e. key kt0 + 4*hh + c with a
        // compile-time c; each test is one subtraction or compare against c.
        // (branch-free: every condition is evaluated, combined with &)
        // Entry passes: a tile whose keys every row keeps by position (below
        // the segment's kfull, rows of one group) needs only the pair rule,
        // one compare per key against the row's excluded group.
        const bool excl_only = MULTI && rows_one_group && (kt0 + BN <= seg_cur.kfull);
        if (!full && excl_only) {
#pragma unroll
            for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int4 kp = *reinterpret_cast<const int4*>(kposp + kb * 32 + 8 * e4 + 4 * hh);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        st[kb][4 * e4 + j] =
                            (kp[j] & 63) != x_i ? st[kb][4 * e4 + j] : kNegInf;
                }
        } else if (!full) {
            const bool row_ok = !SORTED || SETS || g_i == gfirst + seg_cur.seg;
            // sequence-order passes: kept keys are those with 0 <= pos_i - key
            // <= w (keys past the last row then fail too: pos_i < kend for
            // every stored row; the dense pass runs with w = n, the gated
            // pass keeps far keys and gates them instead)
            const int dpos = pos_i - kt0 - 4 * hh;   // pos_i - key = dpos - c
            // single-group pass: kept keys are the slots below kend_row
            const int dend = row_ok ? kend_row - kt0 - 4 * hh : -1;   // key < kend_row: c < dend
#pragma unroll
            for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int k0 = kb * 32 + 8 * e4 + 4 * hh;   // keys k0 .. k0+3
                    int4 kp = {0, 0, 0, 0};
                    if (KPOS) kp = *reinterpret_cast<const int4*>(kposp + k0);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int c = kb * 32 + 8 * e4 + j;
                        bool ok;
                        if (!SORTED) {
                            ok = GATED ? c <= dpos : (uint32_t)(dpos - c) <= (uint32_t)a.w;
                        } else if (SETS) {   // kp = position * 64 + the key token's group mask
                            const int key = kt0 + k0 + j;
                            ok = (key < kend) & (pos_i - (kp[j] >> 6) > a.w) &
                                 ((kp[j] & gmask_i) != 0);
                        } else if (!MULTI) {
                            ok = c < dend;
                        } else {   // kp = position * 64 + the key token's other group
                            const int key = kt0 + k0 + j;
                            ok = row_ok & (key < kend) & (pos_i - (kp[j] >> 6) > a.w) &
                                 ((kp[j] & 63) != x_i);
                        }
                        st[kb][4 * e4 + j] = ok ? st[kb][4 * e4 + j] : kNegInf;
                    }
                }
        }

        // Soft-gated pass: for a tile with some pair further apart than the
        // window, the group affinity a = g_key . g_row of every pair comes
        // from three MFMAs on the bf16 hi/lo split (hi*hi + hi*lo + lo*hi),
        // and far pairs get the gate sigmoid(lambda a) = 1 / (1 + 2^(-lambda
        // log2(e) a)), the row side's fragments carrying the factor -lambda
        // log2(e); pairs inside the window keep gate 1.
        float gate[G::KB][16];
        bool gated_tile = false;
        if constexpr (GATED) {
            const int q0 = tile * a.TT;
            const int qlast = min(a.n, q0 + a.TT) - 1;
            gated_tile = qlast - kt0 > a.w;
            if (gated_tile) {
                const bool all_far = q0 - (kt0 + BN - 1) > a.w;
                const unsigned char* gkb = gk_lds + (bufp == buf0 ? 0 : BN * GROWB);
#pragma unroll
                for (int kb = 0; kb < G::KB; ++kb) {
                    f32x16 at;
#pragma unroll
                    for (int e = 0; e < 16; ++e) at[e] = 0.0f;
#pragma unroll
                    for (int ks = 0; ks < KG / 16; ++ks) {
                        const bf16x8 ghi =
                            *reinterpret_cast<const bf16x8*>(gkb + kb * 32 * GROWB + goff[ks][0]);
                        const bf16x8 glo =
                            *reinterpret_cast<const bf16x8*>(gkb + kb * 32 * GROWB + goff[ks][1]);
                        at = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ghi, gq[ks][0], at, 0, 0, 0);
                        at = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ghi, gq[ks][1], at, 0, 0, 0);
                        at = __builtin_amdgcn_mfma_f32_32x32x16_bf16(glo, gq[ks][0], at, 0, 0, 0);
                    }
                    if (all_far) {   // the common case: every pair of the tile is far
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            gate[kb][e] = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(at[e]));
                    } else {
                        // pos_i - key = dpos - c with a compile-time c per slot
                        const int dpos = pos_i - kt0 - kb * 32 - 4 * hh;
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int c = 8 * (e >> 2) + (e & 3);
                            gate[kb][e] = dpos - c > a.w
                                              ? __builtin_amdgcn_rcpf(
                                                    1.0f + __builtin_amdgcn_exp2f(at[e]))
                                              : 1.0f;
                        }
                    }
                }
            }
        }

        // Online softmax with a lagging reference max m_ref. Probabilities
        // are taken against m_ref as it stands; only when a lane's sum of
        // them exceeds 2^8 (some score grew more than 8 in log2 units past
        // m_ref), or a row has no reference yet, is the reference moved to
        // the tile max, the accumulator rescaled and the tile recomputed.
        // Either way every probability is <= 2^8. The PV product takes them
        // rounded to bf16; the output normaliser adds exactly those rounded
        // values (two per v_dot2c_f32_bf16 against (1, 1)), so the weights
        // applied to V sum to one and a row whose weight sits on few keys
        // carries no normalisation bias; the log-sum-exp adds the fp32 values.
        bf16x8 pf[G::KB][2];
        float psum;
        auto probs = [&](float m_use) {
            float ps2[2] = {0.0f, 0.0f};
#pragma unroll
            for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][e], a.sl2, -m_use));
                    if constexpr (GATED) {
                        if (gated_tile) p *= gate[kb][e];
                    }
                    if (kb == 0 && e < 2) {
                        ps2[e] = p;   // no add to zero (it is not folded: -0 + 0 = +0)
                    } else {
                        ps2[e & 1] += p;
                    }
                    pf[kb][e >> 3][e & 7] = (__bf16)p;
                }
            psum = ps2[0] + ps2[1];
        };
        // (the tests are wave-wide: the decision stays in scalar registers)
        bool redo = __any(m_ref == kNegInf);
        if (!redo) {
            probs(m_ref);
            redo = __any(psum > kProbSumCap);
        }
        if (redo) {
            float tmax = kNegInf;
#pragma unroll
            for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, st[kb][e]);
            tmax = fmaxf(tmax, other_half(tmax)) * a.sl2;
            // every row may move its reference up to the tile max
            const float m_new = fmaxf(m_ref, tmax);
            const float alpha = (m_new == m_ref) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
            l_run *= alpha;
            l_pv *= alpha;
            // rows with no reference yet hold nothing to rescale (the first
            // key tile of every sequence-order item)
            if (__any(m_ref != kNegInf)) {
#pragma unroll
                for (int db = 0; db < G::DB; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
            }
            m_ref = m_new;
            probs(m_ref == kNegInf ? 0.0f : m_ref);
        }
        l_run += psum;
        {
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int kb = 0; kb < G::KB; ++kb)
#pragma unroll
                for (int sp = 0; sp < 2; ++sp)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bf16x2 pair = {pf[kb][sp][2 * j], pf[kb][sp][2 * j + 1]};
                        l_pv = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, l_pv, false);
                    }
        }

        // O^T += V^T P^T. For k-step (kb, sp) the B slots 0..3 / 4..7 of lane
        // half hh hold keys kb*32+16*sp+4*hh+{0..3} / +8+{0..3}; the A operand
        // gets the same keys through two transposing reads, lane m of each
        // 16-lane group addressing row key0 + m/4, columns 4*(m%4) .. +3 of
        // its 16-column half.
#pragma unroll
        for (int kb = 0; kb < G::KB; ++kb)
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
        // Same for the PV MFMAs: V^T reads for three MFMAs ahead.
        {
            constexpr int NP = G::KB * 2 * G::DB;
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * 3, 1);
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                if (j + 3 < NP) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
            }
        }
    };

    // ---- prologue: first K/V copy in flight, then the row data.
    if (ntl > 0) issue(0, buf0, kpos0);
    // A merging pass starts the online softmax from a partial result. The
    // partial is stored as O~ = O * 2^-e (fp16, |O~| < 1) with the row's
    // log2-sum-exp L and e; (acc = O~, l = 2^-e, reference max = L + e) is
    // exactly the state that result stands for, so this pass's keys
    // accumulate on top of it and the final normalisation merges both parts.
    // The sorted passes always merge (every row; rows past the end take a
    // valid row's partial, never stored): they load the partial rows whatever
    // (L, e) holds (the window pass writes every row, zeros with L = -inf for
    // a row without keys, which is then the empty state), so their round trip
    // overlaps that of (L, e), the Q rows and the first K/V tile, and they
    // take them into the state once the loads are back; their accumulator
    // needs no zeroing. (The window pass never merges, but keeping the plain
    // form of this code in it gives it a far better register allocation at
    // three workgroups per CU.)
    const bool merging = SORTED || (!CAUSAL_ALL && a.merge && rvalid);
    f32x2 le_in = {kNegInf, 0.0f};
    f16x4 part_in[G::DB][4];
    auto set_state = [&](int db, int i, f16x4 gv) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[db][4 * i + j] = (float)gv[j];
    };
    auto set_scale = [&]() {
        m_ref = le_in[0] + le_in[1];
        // halves are summed at the end; the partial's weight enters both sums
        l_run = (hh == 0) ? __builtin_ldexpf(1.0f, -(int)le_in[1]) : 0.0f;
        l_pv = l_run;
    };
    if (merging) {
        const int64_t row = ((int64_t)b * a.Hq + h) * a.n + pos_i;
        le_in = a.lseg[row];
        const _Float16* grow_p = a.og + row * D;
        if (SORTED || le_in[0] != kNegInf) {
#pragma unroll
            for (int db = 0; db < G::DB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f16x4 gv =
                        *reinterpret_cast<const f16x4*>(grow_p + db * 32 + 8 * i + 4 * hh);
                    if (SORTED) {
                        part_in[db][i] = gv;
                    } else {
                        set_state(db, i, gv);
                    }
                }
            if (!SORTED) set_scale();
        }
    }
    auto take_partial = [&]() {
        if constexpr (SORTED) {
#pragma unroll
            for (int db = 0; db < G::DB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) set_state(db, i, part_in[db][i]);
            set_scale();
        }
    };
    // query row r -> (head, entry); the entry is the position except in
    // the multi pass (position = entry / 2)
    auto row_of = [&](int r, int& hr, int& pr) {
        hr = kvh * a.hpk + slice * a.G + (r >> a.tt_log);
        if (SORTED) {
            pr = rowpos[r];
        } else {
            pr = min(tile * a.TT + (r & (a.TT - 1)), a.n - 1);
        }
    };
    if (G::QSTAGE) {
        // Q tile (128 rows x ROWB bytes) -> buffer 1 with 1 KB copies, each row
        // one contiguous run in HBM (rows past n copy a valid row; never stored).
#pragma unroll
        for (int c = 0; c < 2 * G::NI; ++c) {
            const int o = (wave * 2 * G::NI + c) * 1024 + 16 * lane;
            const int r = o / G::ROWB;
            int hr, pr;
            row_of(r, hr, pr);
            const int ch = logical_chunk<D>(r, (o % G::ROWB) / 16);
            copy16(a.q + (((int64_t)b * a.Hq + hr) * a.n + (MULTI ? pr >> 1 : pr)) * D + ch * 8,
                   buf1 + (wave * 2 * G::NI + c) * 1024);
        }
        wait_vm();
        __syncthreads();
        // Q^T fragments: lane holds Q[row][16*ks + 8*hh .. +8] for every k-step.
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks)
            qf[ks] = *reinterpret_cast<const bf16x8*>(buf1 + lds_off<D>(R, 2 * ks + hh));
        // buffer 1 is refilled right after the next barrier: the reads must be done
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    } else {
        // Q^T fragments straight from HBM: Q[row][16*ks + 8*hh .. +8].
        const int64_t qrow_off = (((int64_t)b * a.Hq + h) * a.n + pos_i) * D;
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks)
            qf[ks] = *reinterpret_cast<const bf16x8*>(a.q + qrow_off + 16 * ks + 8 * hh);
    }

    if constexpr (GATED) {
        // the row's assignment fragments: columns 16*ks + 8*hh .. +8 of hi and
        // lo, scaled by -lambda log2(e) and split again (hi = bf16 of the
        // scaled value, lo = bf16 of the rest), so the affinity MFMAs return
        // the gate's exponent directly
        const uint16_t* gr = a.gs + ((int64_t)b * a.n + pos_i) * 2 * KG;
#pragma unroll
        for (int ks = 0; ks < KG / 16; ++ks) {
            const bf16x8 hi = *reinterpret_cast<const bf16x8*>(gr + 16 * ks + 8 * hh);
            const bf16x8 lo = *reinterpret_cast<const bf16x8*>(gr + KG + 16 * ks + 8 * hh);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float g = ((float)hi[j] + (float)lo[j]) * a.nl2;
                const __bf16 gh = (__bf16)g;
                gq[ks][0][j] = gh;
                gq[ks][1][j] = (__bf16)(g - (float)gh);
            }
        }
    }

    take_partial();

    // ---- main loop: two LDS buffers, the copy of tile tau+1 overlaps the
    // ---- compute of tile tau; one barrier per tile.
    for (int tau = 0; tau < ntl; tau += 2) {
        int kt0, kend;
        bool full;
        wait_vm();
        __syncthreads();
        locate(tau, seg_cur, kt0, kend, full);
        if (tau + 1 < ntl) issue(tau + 1, buf1, kpos1);
        compute(tau, kt0, kend, full, buf0, kpos0);
        if (tau + 1 >= ntl) break;
        wait_vm();
        __syncthreads();
        locate(tau + 1, seg_cur, kt0, kend, full);
        if (tau + 2 < ntl) issue(tau + 2, buf0, kpos0);
        compute(tau + 1, kt0, kend, full, buf1, kpos1);
    }

    // Epilogue. Lane holds rows' O^T entries d = db*32 + 8*i + 4*hh + j at
    // acc[db][4*i + j]; l_run and l_pv cover this lane half's keys. O is
    // normalised by l_pv (the weights it was accumulated with), the
    // log-sum-exp comes from l_run. The rows are written to LDS (chunk slots
    // XOR-swizzled by row) and stored as whole contiguous rows; each output
    // kind has its own straight-line path (sizes known at compile time).
    const float l_tot = l_run + other_half(l_run);
    const float l_pv_tot = l_pv + other_half(l_pv);
    const int64_t row = ((int64_t)b * a.Hq + h) * a.n + pos_i;   // output row
    const float inv_l = l_pv_tot > 0.0f ? __builtin_amdgcn_rcpf(l_pv_tot) : 0.0f;
    // kind 0: fp16 partial O * 2^-e; 1: bf16 output; 2: fp32 output
    auto epilogue = [&](auto kind_tag) {
        constexpr int KIND = decltype(kind_tag)::value;
        constexpr int ESZ = KIND == 2 ? 4 : 2;
        constexpr int RB = D * ESZ;                          // bytes per output row
        constexpr int NCHK = RB / 16;                        // 16-byte chunks per row
        constexpr int CMASK = (NCHK < 16 ? NCHK : 16) - 1;
        constexpr int RPP = ROWS < 4 * G::TILEB / RB ? ROWS : 4 * G::TILEB / RB;   // rows per pass
        constexpr int HROWS = 2 * G::TILEB / RB;             // rows staged per buffer
        float scale_o = inv_l;
        if constexpr (KIND == 0) {
            // 16-bit partial with a per-row power-of-two scale: O~ = O * 2^-e
            // with e the exponent of max |O| (so |O~| < 1), kept in fp16, whose
            // 11-bit significand keeps the merge as precise as the final output
            float mx = 0.0f;
#pragma unroll
            for (int db = 0; db < G::DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, __builtin_fabsf(acc[db][e]));
            mx = fmaxf(mx, other_half(mx)) * scale_o;
            const int ex = mx > 0.0f ? __builtin_amdgcn_frexp_expf(mx) : 0;
            scale_o = __builtin_ldexpf(scale_o, -ex);
            if (rvalid && hh == 0) {
                const f32x2 le = {l_tot > 0.0f ? m_ref + __log2f(l_tot) : kNegInf, (float)ex};
                a.lseg_dst[row] = le;
            }
        } else {
            if (rvalid && hh == 0 && a.lse) a.lse[row] = (m_ref + __log2f(l_tot)) * kLn2;
        }
        auto stage = [&](int rs) -> unsigned char* {
            return rs < HROWS ? buf0 + rs * RB : buf1 + (rs - HROWS) * RB;
        };
        char* dst = KIND == 0 ? reinterpret_cast<char*>(a.og_dst) : static_cast<char*>(a.out);
        // Stores: each thread writes one fixed 16-byte chunk c of every
        // RSTEP-th staged row. Row r of the tile is token (or entry) slot
        // r & (TT-1) of head slot r >> tt_log; the head's rows start at
        // dbase + (r >> tt_log) * n * RB.
        constexpr int RSTEP = NT / NCHK;
        const int c_t = tid % NCHK, rs_t = tid / NCHK;
        const int64_t hstride = (int64_t)a.n * RB;
        char* const dbase =
            dst + ((int64_t)b * a.Hq + kvh * a.hpk + slice * a.G) * hstride + c_t * 16;
#pragma unroll
        for (int r0 = 0; r0 < ROWS; r0 += RPP) {
            // K/V buffers (or the previous pass) are free
            __syncthreads();
            if (R >= r0 && R < r0 + RPP) {
                const int rs = R - r0;
#pragma unroll
                for (int db = 0; db < G::DB; ++db)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int qd = db * 8 + 2 * i + hh;   // quad index: d = 4*qd .. +3
                        const f32x4 o = {acc[db][4 * i] * scale_o, acc[db][4 * i + 1] * scale_o,
                                         acc[db][4 * i + 2] * scale_o, acc[db][4 * i + 3] * scale_o};
                        if constexpr (KIND == 2) {
                            *reinterpret_cast<f32x4*>(stage(rs) + ((qd ^ (rs & CMASK)) << 4)) = o;
                        } else {
                            const int half = (qd & 1) ^ ((rs >> 4) & 1);
                            unsigned char* sp =
                                stage(rs) + (((qd >> 1) ^ (rs & CMASK)) << 4) + half * 8;
                            if constexpr (KIND == 0) {
                                const f16x4 oh = {(_Float16)o[0], (_Float16)o[1], (_Float16)o[2],
                                                  (_Float16)o[3]};
                                *reinterpret_cast<f16x4*>(sp) = oh;
                            } else {
                                const bf16x4 ob = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2],
                                                   (__bf16)o[3]};
                                *reinterpret_cast<bf16x4*>(sp) = ob;
                            }
                        }
                    }
            }
            __syncthreads();
            static_assert(RPP % RSTEP == 0, "whole store rounds");
#pragma unroll
            for (int k = 0; k < RPP / RSTEP; ++k) {
                const int rs = rs_t + k * RSTEP;
                const int r = r0 + rs;
                const int tk = r & (a.TT - 1);
                if (qs0 + tk >= qs1) continue;   // rows past the sequence end
                // the row's position (sorted passes: from its entry; entry passes: entry / 2)
                int pr = qs0 + tk;
                if (SORTED) pr = MULTI ? rowpos[r] >> 1 : rowpos[r];
                u32x4 val =
                    *reinterpret_cast<const u32x4*>(stage(rs) + ((c_t ^ (rs & CMASK)) << 4));
                if (ESZ == 2 && ((rs >> 4) & 1)) val = __builtin_shufflevector(val, val, 2, 3, 0, 1);
                // non-temporal: written once, read (if at all) by a later pass
                __builtin_nontemporal_store(
                    val, reinterpret_cast<u32x4*>(dbase + (int64_t)(r >> a.tt_log) * hstride +
                                                  (int64_t)pr * RB));
            }
        }
    };
    // partials: the window pass ahead of a long-range pass, the first entry
    // pass
    if ((MULTI || PHASE == kWindow) && a.partial) {
        epilogue(std::integral_constant<int, 0>{});
    } else if (a.out_f32) {
        epilogue(std::integral_constant<int, 2>{});
    } else {
        epilogue(std::integral_constant<int, 1>{});
    }
}

// Soft-gated pass operand: gs[t][0][k] = bf16(G[t][k]) (round to nearest
// even), gs[t][1][k] = bf16(G[t][k] - gs[t][0][k]), zero for k >= K; one
// thread per (token, column of KG).
__global__ __launch_bounds__(256) void gate_split_kernel(const float* __restrict__ G,
                                                         int64_t ntok, int K, int KG,
                                                         uint16_t* __restrict__ gs) {
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (x >= ntok * KG) return;
    const int64_t t = x / KG;
    const int k = (int)(x % KG);
    const float g = k < K ? G[t * K + k] : 0.0f;
    const __bf16 hi = (__bf16)g;
    const __bf16 lo = (__bf16)(g - (float)hi);
    gs[t * 2 * KG + k] = __builtin_bit_cast(uint16_t, hi);
    gs[t * 2 * KG + KG + k] = __builtin_bit_cast(uint16_t, lo);
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
    a.G = attn_heads_per_wg(a.hpk);
    a.TT = ROWS / a.G;
    a.tt_log = 31 - __builtin_clz((unsigned)a.TT);
    a.nslices = a.hpk / a.G;
    a.ne = p.n;
    a.ntiles = (p.n + a.TT - 1) / a.TT;
    a.total = p.B * p.Hkv * a.nslices * a.ntiles;
    a.fd_ntiles = make_fastdiv((uint32_t)a.ntiles);
    a.fd_nslices = make_fastdiv((uint32_t)a.nslices);
    a.fd_hkv = make_fastdiv((uint32_t)p.Hkv);
    a.sl2 = p.scale * 1.44269504088896340736f;
    a.out_f32 = p.out_f32;
    if (p.workspace) {
        const AttnWorkspace ws = attn_workspace_layout(p);
        char* base = static_cast<char*>(p.workspace);
        a.og = reinterpret_cast<_Float16*>(base + ws.og);
        a.lseg = reinterpret_cast<f32x2*>(base + ws.lseg);
        a.og_dst = a.og;
        a.lseg_dst = a.lseg;
        a.plan = reinterpret_cast<const int32_t*>(base + ws.plan);
        a.order = reinterpret_cast<const int32_t*>(base + ws.order);
        a.spos = reinterpret_cast<int32_t*>(base + ws.spos);
        a.pack = reinterpret_cast<const int32_t*>(base + ws.pack);
        a.pack_ints = attn_pack_ints(a.TT, attn_long_range_tile_keys(p.d));
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

// Long-range pass arguments: the sorted key order lists n*m entries. K and
// V rows are read in place at the positions perm gives, or from sorted
// copies made by the prepare call (attn_sorted_copies: two groups per token,
// a head's rows beyond a buffer resource's 2^31-byte reach, or asked for).
// The choice depends only on the problem, so prepare and apply agree. With
// two groups per token each of the two entry passes takes ceil(n / TT)
// query tiles of its half of the query order.
AttnArgs long_range_args(const AttnProblem& p) {
    AttnArgs a = make_args(p);
    a.ne = p.n * p.m;
    a.direct = attn_sorted_copies(p.n, p.d, p.m, p.K, p.force_copies != 0) ? 0 : 1;
    const AttnWorkspace ws = attn_workspace_layout(p);
    char* base = static_cast<char*>(p.workspace);
    if (!a.direct) {
        a.k = reinterpret_cast<const uint16_t*>(base + ws.ks);
        a.v = reinterpret_cast<const uint16_t*>(base + ws.vs);
    }
    if (p.m == 2) a.qperm = reinterpret_cast<const int32_t*>(base + ws.qent);
    return a;
}

}  // namespace

int attn_heads_per_wg(int hpk) {
    // Query heads packed into one workgroup: the largest power of two <= 8
    // that divides Hq/Hkv. All packed heads share the kv head, the token set
    // and the mask, so each K/V tile staged in LDS serves G*TT = 128 rows.
    int g = 1;
    while (g < 8 && hpk % (2 * g) == 0) g *= 2;
    return g;
}

// Set pass (two groups per token, K <= 4): the group masks of the membership
// sets, 4 bits each (set s in bits 4s .. 4s+3).
int set_mask_table(int K) {
    int lut = 0, s = 0;
    for (int x = 0; x < K; ++x)
        for (int y = x + 1; y < K; ++y) lut |= ((1 << x) | (1 << y)) << (4 * s++);
    return lut;
}

// Set pass arguments: the sorted order lists the n tokens by membership set;
// key rows come from set-sorted copies of K and V (contiguous key tiles).
AttnArgs set_pass_args(const AttnProblem& p) {
    AttnArgs a = make_args(p);
    const AttnWorkspace ws = attn_workspace_layout(p);
    char* base = static_cast<char*>(p.workspace);
    a.perm = reinterpret_cast<const int32_t*>(base + ws.operm);
    a.offsets = reinterpret_cast<const int32_t*>(base + ws.ooffs);
    a.k = reinterpret_cast<const uint16_t*>(base + ws.ks);
    a.v = reinterpret_cast<const uint16_t*>(base + ws.vs);
    a.direct = 0;
    a.set_lut = set_mask_table(p.K);
    return a;
}

hipError_t launch_attn_set_prepare(const AttnProblem& p, hipStream_t stream) {
    const AttnArgs a = set_pass_args(p);
    const AttnWorkspace ws = attn_workspace_layout(p);
    char* base = static_cast<char*>(p.workspace);
    int32_t* sid = reinterpret_cast<int32_t*>(base + ws.okey);
    const int S = attn_membership_sets(p.K);
    const int64_t ntok = (int64_t)p.B * p.n;
    hipLaunchKernelGGL(attn_set_id_kernel, dim3((unsigned)((ntok + 255) / 256)), dim3(256), 0,
                       stream, p.ids, ntok, p.K, S, sid);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_group_sort(sid, p.B, p.n, S, const_cast<int32_t*>(a.perm),
                          const_cast<int32_t*>(a.offsets), base + ws.ohist, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_set_plan_kernel, dim3((a.ntiles + 255) / 256, p.B), dim3(256), 0,
                       stream, a.perm, a.offsets, p.ids, p.n, p.K, S, p.w, a.TT, a.ntiles,
                       attn_tile_keys(p.d, kLongSets), a.set_lut, const_cast<int32_t*>(a.plan));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_order_kernel, dim3(p.B), dim3(256), 0, stream, a.plan, a.ntiles,
                       const_cast<int32_t*>(a.order));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // set-sorted K and V (the gather also writes plain positions into spos,
    // which the next kernel replaces by the (position, group mask) words)
    const int64_t chunks = (int64_t)(p.n + KPOS_PAD) * (p.d / 8);
    hipLaunchKernelGGL(attn_gather_kernel, dim3((unsigned)((chunks + 255) / 256), p.B * p.Hkv),
                       dim3(256), 0, stream, p.k, p.v, a.perm, p.ids, p.n, p.n, 1, p.K, p.Hkv,
                       p.d, const_cast<uint16_t*>(a.k), const_cast<uint16_t*>(a.v), a.spos);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_set_spos_kernel, dim3((p.n + KPOS_PAD + 255) / 256, p.B), dim3(256),
                       0, stream, a.perm, p.ids, p.n, p.K, a.spos);
    return hipGetLastError();
}

// Entry passes (two groups per token, K >= 5): the query order (the key
// slots stably sorted by membership index: first-group entries, then
// second-group entries, each half in key order), its plan over [B][2][T]
// tiles and the LPT order of each half.
hipError_t launch_attn_entry_prepare(const AttnProblem& p, const AttnArgs& a,
                                     hipStream_t stream) {
    const AttnWorkspace ws = attn_workspace_layout(p);
    char* base = static_cast<char*>(p.workspace);
    int32_t* okey = reinterpret_cast<int32_t*>(base + ws.okey);
    int32_t* operm = reinterpret_cast<int32_t*>(base + ws.operm);
    int32_t* ooffs = reinterpret_cast<int32_t*>(base + ws.ooffs);
    int32_t* qent = const_cast<int32_t*>(a.qperm);
    const int64_t slots = (int64_t)p.B * a.ne;
    const dim3 sgrid((unsigned)((slots + 255) / 256));
    hipLaunchKernelGGL(attn_entry_index_kernel, sgrid, dim3(256), 0, stream, p.perm, slots, okey);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_group_sort(okey, p.B, a.ne, 2, operm, ooffs, base + ws.ohist, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_entry_query_kernel, sgrid, dim3(256), 0, stream, p.perm, operm, a.ne,
                       slots, qent);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int T = a.ntiles;
    hipLaunchKernelGGL(attn_entry_plan_kernel, dim3((2 * T + 255) / 256, p.B), dim3(256), 0, stream,
                       p.ids, p.perm, p.offsets, qent, p.n, p.K, p.w, a.TT, T,
                       attn_tile_keys(p.d, kLongMulti), const_cast<int32_t*>(a.plan));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // one order row per (batch element, half)
    hipLaunchKernelGGL(attn_order_kernel, dim3(2 * p.B), dim3(256), 0, stream, a.plan, T,
                       const_cast<int32_t*>(a.order));
    return hipGetLastError();
}

hipError_t launch_attn_long_range_prepare(const AttnProblem& p, hipStream_t stream) {
    if (!attn_has_long_range(p.n, p.w)) return hipSuccess;
    if (p.m != 1 && p.m != 2) return hipErrorInvalidValue;
    if (attn_uses_sets(p.n, p.d, p.m, p.K)) return launch_attn_set_prepare(p, stream);
    const AttnArgs a = long_range_args(p);
    hipError_t e = hipSuccess;
    if (!a.direct) {
        const int64_t chunks = (int64_t)(a.ne + KPOS_PAD) * (p.d / 8);
        hipLaunchKernelGGL(attn_gather_kernel,
                           dim3((unsigned)((chunks + 255) / 256), p.B * p.Hkv), dim3(256), 0,
                           stream, p.k, p.v, p.perm, p.ids, p.n, a.ne, p.m, p.K, p.Hkv, p.d,
                           const_cast<uint16_t*>(a.k), const_cast<uint16_t*>(a.v), a.spos);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (p.m == 2) return launch_attn_entry_prepare(p, a, stream);
    hipLaunchKernelGGL(attn_plan_kernel, dim3((a.ntiles + 255) / 256, p.B), dim3(256), 0, stream,
                       p.ids, p.perm, p.offsets, a.ne, p.K, p.w, a.TT, a.ntiles,
                       attn_tile_keys(p.d, kLongRange), const_cast<int32_t*>(a.plan));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_order_kernel, dim3(p.B), dim3(256), 0, stream, a.plan, a.ntiles,
                       const_cast<int32_t*>(a.order));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_pack_kernel, dim3(a.ntiles, p.B), dim3(256), 0, stream, a.plan,
                       a.order, p.ids, p.perm, p.offsets, p.n, p.K, p.w, a.TT,
                       attn_long_range_tile_keys(p.d), a.ntiles, a.pack_ints,
                       const_cast<int32_t*>(a.pack));
    return hipGetLastError();
}

hipError_t launch_attn_long_range_apply(const AttnProblem& p, hipStream_t stream) {
    if (!attn_has_long_range(p.n, p.w)) return hipSuccess;
    if (p.m != 1 && p.m != 2) return hipErrorInvalidValue;
    if (attn_uses_sets(p.n, p.d, p.m, p.K)) {
        // one pass over the set-sorted tokens, merged with the window partial
        AttnArgs a = set_pass_args(p);
        a.merge = 1;
        a.partial = 0;
        return launch<kLongSets>(a, p.d, stream);
    }
    AttnArgs a = long_range_args(p);
    a.merge = 1;     // start from the window partial
    if (p.m == 1) {
        a.partial = 0;   // write the final output
        return launch<kLongRange>(a, p.d, stream);
    }
    // Two groups per token: the first-group entries merge their keys into
    // the window partial and write the result as a second partial, then the
    // second-group entries merge theirs into that and write the final
    // output. A pair of tokens sharing both groups is kept only where the
    // query row's group is the lower of the two.
    const AttnWorkspace ws = attn_workspace_layout(p);
    char* base = static_cast<char*>(p.workspace);
    _Float16* og1 = reinterpret_cast<_Float16*>(base + ws.og1);
    f32x2* lseg1 = reinterpret_cast<f32x2*>(base + ws.lseg1);
    a.half = 0;
    a.partial = 1;
    a.og_dst = og1;
    a.lseg_dst = lseg1;
    hipError_t e = launch<kLongMulti>(a, p.d, stream);
    if (e != hipSuccess) return e;
    a.half = 1;
    a.partial = 0;
    a.og = og1;
    a.lseg = lseg1;
    return launch<kLongMulti>(a, p.d, stream);
}

hipError_t launch_attn_long_range(const AttnProblem& p, hipStream_t stream) {
    const hipError_t e = launch_attn_long_range_prepare(p, stream);
    if (e != hipSuccess) return e;
    return launch_attn_long_range_apply(p, stream);
}

hipError_t launch_attn_window(const AttnProblem& p, hipStream_t stream) {
    AttnArgs a = make_args(p);
    a.merge = 0;
    // with a long-range part to come, the window result is a partial
    a.partial = attn_has_long_range(p.n, p.w) ? 1 : 0;
    return launch<kWindow>(a, p.d, stream);
}

hipError_t launch_attn_soft_gate(const AttnProblem& p, const float* G, float lambda,
                                 hipStream_t stream) {
    const int KG = soft_gate_columns(p.K);
    uint16_t* gs = static_cast<uint16_t*>(p.workspace);
    const int64_t threads = (int64_t)p.B * p.n * KG;
    hipLaunchKernelGGL(gate_split_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, G, (int64_t)p.B * p.n, p.K, KG, gs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    AttnProblem q = p;
    q.workspace = nullptr;   // none of the two-pass buffers
    AttnArgs a = make_args(q);
    a.gs = gs;
    a.nl2 = -lambda * 1.44269504088896340736f;
    a.merge = 0;
    a.partial = 0;
    if (KG == 16) return launch<kSoftGate>(a, p.d, stream);
    if (KG == 32) return launch<kSoftGate + 1>(a, p.d, stream);
    return launch<kSoftGate + 2>(a, p.d, stream);
}

hipError_t launch_attn_dense(const AttnProblem& p, hipStream_t stream) {
    AttnArgs a = make_args(p);
    a.merge = 0;
    a.partial = 0;
    a.w = p.n;
    return launch<kDense>(a, p.d, stream);
}

}  // namespace focus
