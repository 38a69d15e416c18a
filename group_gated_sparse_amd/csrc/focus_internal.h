// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
// Every launcher assumes its arguments were validated by the ABI layer and
// returns the hipError_t of its launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace focus {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// ---- assignment -----------------------------------------------------------
// Padded row length of the split W^T = (P C^T)^T tables: a multiple of 64.
inline int assign_dpad(int d_model) { return (d_model + 63) / 64 * 64; }
inline int assign_kpad(int K) { return K <= 32 ? 32 : 64; }
inline size_t assign_workspace(int d_model, int K) {
    return 2 * align_up((size_t)assign_kpad(K) * assign_dpad(d_model) * 2);
}
// M = groups kept per token (1 or 2): ids [B][n][M], best first; margin =
// (M-th score) - ((M+1)-th score). M = 0: the raw scores [B][n][K] instead.
hipError_t launch_assign(const float* hidden, const float* P, const float* C, const float* bias,
                         int B, int n, int d_model, int d_proj, int K, int M, int32_t* ids,
                         float* margin, float* scores, void* workspace, hipStream_t stream);

// ---- Sinkhorn soft assignment -------------------------------------------------
// Workspace: column scales v [B][K] and per-workgroup column sums
// [B][nblk][K] (256-byte aligned).
struct SinkhornLayout {
    int rpb;      // rows per workgroup
    int nblk;     // workgroups per sequence
    size_t v, partial, total;
};
SinkhornLayout sinkhorn_layout(int B, int n, int K, int iters);
hipError_t launch_sinkhorn(const float* scores, int B, int n, int K, float tau, int iters,
                           float* G, void* workspace, hipStream_t stream);

// ---- grouping ---------------------------------------------------------------
constexpr int SORT_BLOCK_TOKENS = 2048;  // tokens per workgroup of the two sort passes
size_t group_sort_workspace(int B, int n, int K);
hipError_t launch_group_sort(const int32_t* ids, int B, int n, int K, int32_t* perm,
                             int32_t* offsets, void* workspace, hipStream_t stream);
// The library's own scratch for the sort (focus_group_sort_noalloc): a
// static device array of kSortScratchBytes; group_sort_scratch gives its
// address on the current device (looked up once per device).
constexpr size_t kSortScratchBytes = (size_t)1 << 20;
hipError_t group_sort_scratch(int32_t** ptr);

// ---- attention --------------------------------------------------------------
struct AttnProblem {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* ids;
    const int32_t* perm;
    const int32_t* offsets;
    int B, Hq, Hkv, n, d, K, w;
    float scale;
    void* out;
    int out_f32;
    float* lse;
    void* workspace;
    int m = 1;     // groups per token: ids [B][n][m]; perm holds entries t*m + c
    int force_copies = 0;   // long-range pass from group-sorted K/V copies at any size
};

// True when some pair further apart than the window can exist (n - 1 > w).
inline bool attn_has_long_range(int n, int w) { return (int64_t)n - 1 > (int64_t)w; }

constexpr int KPOS_PAD = 256;   // padding slots after the sorted positions (one 1 KB copy)
constexpr int SEGCAP = 7;       // group segments stored per planned query tile
constexpr int PLAN_INTS = 32;   // ints per plan record (4 + 4 * SEGCAP)

int attn_heads_per_wg(int hpk);
inline int attn_tokens_per_tile(int Hq, int Hkv) { return 128 / attn_heads_per_wg(Hq / Hkv); }
// Keys per tile of the long-range pass (32, or 64 at d = 32).
constexpr int attn_long_range_tile_keys(int d) { return d == 32 ? 64 : 32; }
// Ints per packed record of the single-group long-range pass: the plan
// record and tile index (64), then per row its entry and key-slot end (TT
// each), then the positions of the first key tile's rows (BN), rounded up to
// 256 bytes.
inline int attn_pack_ints(int TT, int BN) { return (64 + 2 * TT + BN + 63) / 64 * 64; }

// Two groups per token with few groups (K <= 4, so at most 6 membership
// sets): the long-range pass runs over tokens sorted by membership set.
inline int attn_membership_sets(int K) { return K * (K - 1) / 2; }
inline bool attn_uses_sets(int n, int d, int m, int K) {
    (void)n;
    (void)d;
    return m == 2 && K <= 4;
}
// Whether the long-range pass reads sorted copies of K and V (made by its
// prepare step) rather than key rows in place: always with two groups per
// token (copies in membership-entry or membership-set order); with one, when
// a kv head's K rows span 2^31 bytes or more (the reach of a buffer
// resource), or when the caller asks for them.
inline bool attn_sorted_copies(int n, int d, int m, int K, bool force) {
    (void)K;
    return force || m > 1 || (int64_t)n * d * 2 >= ((int64_t)1 << 31);
}

// Query tiles of the long-range pass. One group per token, and the set
// pass: ceil(n / TT) tiles over the sorted tokens. Two groups per token
// otherwise (the entry passes): ceil(n / TT) tiles over each half of the
// query order (first-group entries, then second-group entries).
inline int attn_long_range_tiles(int n, int TT, int m, bool sets) {
    const int t = (n + TT - 1) / TT;
    return (m == 2 && !sets) ? 2 * t : t;
}

// Attention workspace, byte offsets: the window partial output (fp16
// [B][Hq][n][d], scaled per row), its log2-sum-exp and scale exponent (fp32
// pairs [B][Hq][n]), the tile plan, the order in which the long-range pass
// takes the sorted query tiles (int32 [B][tiles], most work first) and, with
// one group per token, one packed record per ordered tile (int32
// [B][tiles][attn_pack_ints]: plan record, tile index, each row's entry and
// key-slot end, the first key tile's positions). With sorted copies
// (attn_sorted_copies) also the sorted K and V (bf16 [B][Hkv][slots][d])
// and the sorted slots' positions or (position, group) words (int32
// [B][slots + pad]). Two groups per token:
//  - the set pass (attn_uses_sets) sorts the n tokens by membership set:
//    the set id per token (okey), the set-sorted positions (operm), set
//    offsets (ooffs), the sort's per-block counts (ohist);
//  - the entry passes key on the caller's sort of the n*2 membership
//    entries by group and take their query rows in a second order, the
//    first-group entries then the second-group entries, each half in key
//    order: the stable sort by membership index of the key order (okey:
//    index per key slot, operm: the sorted key slots, ooffs, ohist), the
//    query order's entries (qent, int32 [B][2n]) and the first entry pass's
//    partial (og1, lseg1: laid out as og, lseg), from which the second pass
//    starts; the window partial is only read, so apply can be repeated on
//    it, and there is no partial per entry.
// The first two regions lead every layout, so the window pass, which uses
// only them, takes the same offsets for every m.
struct AttnWorkspace {
    size_t og, lseg, plan, order, pack, ks, vs, spos, okey, operm, ooffs, ohist, qent, og1, lseg1,
        total;
};
inline AttnWorkspace attn_workspace_layout(int B, int Hq, int Hkv, int n, int d, int m, int K,
                                           bool force_copies) {
    AttnWorkspace w{};
    const bool sets = attn_uses_sets(n, d, m, K);
    const bool copies = attn_sorted_copies(n, d, m, K, force_copies);
    const int S = attn_membership_sets(K);
    const int TT = attn_tokens_per_tile(Hq, Hkv);
    const bool entries = m == 2 && !sets;
    const size_t ne = sets ? (size_t)n : (size_t)n * m;
    const size_t ntiles = attn_long_range_tiles(n, TT, m, sets);
    size_t off = 0;
    w.og = off;   off += align_up((size_t)B * Hq * n * d * 2);
    w.lseg = off; off += align_up((size_t)B * Hq * n * 8);
    w.plan = off; off += align_up((size_t)B * ntiles * PLAN_INTS * 4);
    w.order = off; off += align_up((size_t)B * ntiles * 4);
    w.pack = off;
    off += m == 1 ? align_up((size_t)B * ntiles * attn_pack_ints(TT, attn_long_range_tile_keys(d)) * 4)
                  : 0;
    w.ks = off;   off += copies ? align_up((size_t)B * Hkv * ne * d * 2) : 0;
    w.vs = off;   off += copies ? align_up((size_t)B * Hkv * ne * d * 2) : 0;
    w.spos = off; off += (copies || sets) ? align_up((size_t)B * (ne + KPOS_PAD) * 4) : 0;
    // the order sort: S sets over n tokens, or 2 halves over 2n key slots
    const bool osort = sets || entries;
    const int okeys = sets ? S : 2;
    w.okey = off;  off += osort ? align_up((size_t)B * ne * 4) : 0;
    w.operm = off; off += osort ? align_up((size_t)B * ne * 4) : 0;
    w.ooffs = off; off += osort ? align_up((size_t)B * (okeys + 1) * 4) : 0;
    w.ohist = off; off += osort ? align_up(group_sort_workspace(B, (int)ne, okeys)) : 0;
    w.qent = off;  off += entries ? align_up((size_t)B * ne * 4) : 0;
    w.og1 = off;   off += entries ? align_up((size_t)B * Hq * n * d * 2) : 0;
    w.lseg1 = off; off += entries ? align_up((size_t)B * Hq * n * 8) : 0;
    w.total = off;
    return w;
}
inline AttnWorkspace attn_workspace_layout(const AttnProblem& p) {
    return attn_workspace_layout(p.B, p.Hq, p.Hkv, p.n, p.d, p.m, p.K, p.force_copies != 0);
}
// The window pass alone uses only the leading two regions (partial, L/e),
// which every layout above shares.
inline size_t attn_window_workspace(int B, int Hq, int Hkv, int n, int d, int w) {
    if (!attn_has_long_range(n, w)) return 0;
    const AttnWorkspace l = attn_workspace_layout(B, Hq, Hkv, n, d, 1, 1, false);
    return l.plan;
}
inline size_t attn_workspace(int B, int Hq, int Hkv, int n, int d, int w, int K, int m = 1,
                             bool force_copies = false) {
    if (!attn_has_long_range(n, w)) return 0;
    return attn_workspace_layout(B, Hq, Hkv, n, d, m, K, force_copies).total;
}

// The long-range pass: prepare (sorted K/V copies, tile plan and order, row
// ends; needs only k, v and the group data) then apply (the attention, merged
// with the window partial); launch_attn_long_range runs both.
hipError_t launch_attn_long_range_prepare(const AttnProblem& p, hipStream_t stream);
hipError_t launch_attn_long_range_apply(const AttnProblem& p, hipStream_t stream);
hipError_t launch_attn_long_range(const AttnProblem& p, hipStream_t stream);
hipError_t launch_attn_window(const AttnProblem& p, hipStream_t stream);
hipError_t launch_attn_dense(const AttnProblem& p, hipStream_t stream);

// Training-time soft-gated attention: every causal pair, far pairs weighted by
// sigmoid(lambda g_i . g_j). Workspace: the bf16 hi/lo split of the soft
// assignments G, [B][n][2][KG] with KG = K padded to 16, 32 or 64.
inline int soft_gate_columns(int K) { return K <= 16 ? 16 : (K <= 32 ? 32 : 64); }
inline size_t soft_gate_workspace(int B, int n, int K) {
    return align_up((size_t)B * n * 4 * soft_gate_columns(K));
}
hipError_t launch_attn_soft_gate(const AttnProblem& p, const float* G, float lambda,
                                 hipStream_t stream);

}  // namespace focus
