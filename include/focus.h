/*
 * focus.h -- C ABI of libfocus.so: the Focus group-gated attention forward
 * pass on AMD Instinct MI355X (gfx950).
 *
 * The method (Focus; pages "Why Attend to Everything? Focus is the Key",
 * Korean technical summary §2.1-§2.3, and "Focus: Learning Which Attention
 * Pairs Matter", Japanese technical summary §2.1-§2.2): every token is given
 * one of K groups by comparing its projected hidden state with K learned
 * centroids; attention then keeps the local window at full resolution and,
 * beyond it, only pairs whose tokens share a group, with the exact softmax
 * over the kept pairs. Inference uses a hard assignment, so dropped pairs
 * are skipped rather than zeroed.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors), contiguous, row-major in the layout stated, and 16-byte
 *     aligned unless stated otherwise. The caller owns every buffer; the
 *     library never allocates or frees device memory and keeps no pointer
 *     after the call returns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and runs asynchronously; buffers must stay valid until the
 *     stream has passed the call. No call synchronises the host.
 *   - Arguments are validated on the host before anything is enqueued: on a
 *     non-OK status nothing has been launched, and focus_last_error()
 *     returns a message (thread-local, valid until the next call on that
 *     thread). A failed launch returns FOCUS_ERR_DEVICE.
 *   - Device-side data (group ids, perm, offsets) cannot be checked on the
 *     host. Out-of-range values give undefined results but never an
 *     out-of-bounds access: kernels clamp every index they read.
 *   - Workspaces are caller-provided scratch of at least the size the
 *     matching *_workspace_bytes() function returns; contents are undefined
 *     between calls, and concurrent calls must not share one.
 *   - Results are bitwise deterministic for fixed inputs on one device.
 *   - Nothing is thrown across the ABI; the library never prints or exits.
 */
#ifndef FOCUS_H_
#define FOCUS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* focus_stream_t; /* hipStream_t */

typedef enum {
    FOCUS_OK = 0,
    FOCUS_ERR_INVALID_ARGUMENT = 1, /* null / misaligned pointer, bad size, overlap */
    FOCUS_ERR_UNSUPPORTED = 2,      /* valid request outside the supported range   */
    FOCUS_ERR_WORKSPACE = 3,        /* workspace missing or too small              */
    FOCUS_ERR_DEVICE = 4            /* a HIP launch or runtime call failed         */
} focus_status;

typedef enum { FOCUS_BF16 = 0, FOCUS_F32 = 1 } focus_dtype;

#define FOCUS_ABI_VERSION 4
#define FOCUS_MAX_GROUPS 64
#define FOCUS_MAX_MEMBERSHIPS 2 /* groups per token (m) of the top-k variant */
#define FOCUS_MAX_SINKHORN_ITERS 10000

int focus_abi_version(void);
const char* focus_last_error(void);

/* ------------------------------------------------------------------------
 * Step 1: hard group assignment (Japanese page §2.1: the hidden state h_t is
 * projected and compared with the centroids in centroid space; §2.2: a hard
 * top-k assignment at inference, here k = 1).
 *
 *   score[t][k] = (h_t · P) · C_k + bias[k]      computed as h_t · (P C^T)
 *   group_ids[t] = argmax_k score[t][k]          exact ties -> lowest k
 *   margin[t]    = top-1 score - top-2 score     (+inf when K == 1)
 *
 * hidden    [B][n][d_model] fp32     P [d_model][d_proj] fp32
 * C         [K][d_proj] fp32         bias [K] fp32 or NULL
 * group_ids [B][n] int32 (out)       margin [B][n] fp32 (out) or NULL
 * Limits: 1 <= K <= 64; d_model % 4 == 0; d_proj >= 1; B, n >= 1.
 * The scores are accumulated in fp32 from an exact bf16 hi/lo split of h
 * and of P C^T, so they agree with plain fp32 arithmetic to ~1e-6 relative;
 * tokens whose top-2 margin is below ~1e-3 may resolve either way.
 * ---------------------------------------------------------------------- */
size_t focus_assign_workspace_bytes(int d_model, int K);
focus_status focus_assign(const float* hidden, const float* P, const float* C, const float* bias,
                          int B, int n, int d_model, int d_proj, int K,
                          int32_t* group_ids, float* margin,
                          void* workspace, size_t workspace_bytes, focus_stream_t stream);

/* ------------------------------------------------------------------------
 * Top-k variant (Korean page §2.3 and §3.4, Japanese page §2.2 and §3.3: at
 * inference a token may join its top-k groups; the pages' runs use k = 2
 * with K = 4). Same scores; m = k groups per token:
 *   group_ids[t][0..m-1] = the m highest-scoring groups, best first (exact
 *                          ties -> lowest k)
 *   margin[t]            = m-th score - (m+1)-th score (+inf when K == m)
 * group_ids [B][n][m] int32 (out). Limits: 1 <= m <= FOCUS_MAX_MEMBERSHIPS,
 * m <= K; otherwise as focus_assign, with the same workspace size.
 * focus_assign_topk with m = 1 is focus_assign.
 * ---------------------------------------------------------------------- */
focus_status focus_assign_topk(const float* hidden, const float* P, const float* C,
                               const float* bias, int B, int n, int d_model, int d_proj, int K,
                               int m, int32_t* group_ids, float* margin,
                               void* workspace, size_t workspace_bytes, focus_stream_t stream);

/* ------------------------------------------------------------------------
 * Training-time soft assignment (Korean page §2.2; Japanese page §2.1 and
 * §2.3): tokens are assigned softly to the K groups, and the assignment
 * matrix of each sequence is made doubly stochastic by Sinkhorn
 * normalisation (every group receives the same number of tokens).
 *
 * focus_assign_scores writes the raw scores of focus_assign:
 *   scores[t][k] = (h_t · P) · C_k + bias[k]                 [B][n][K] fp32
 * (same arithmetic, limits and workspace as focus_assign).
 *
 * focus_sinkhorn: with A = exp(scores / tau) per sequence,
 *   G[t][k] = A[t][k] u[t] v[k], where the rows are normalised first
 *   (v = 1, u[t] = 1 / sum_k A[t][k]) and then `iters` rounds set
 *     v[k] = (n / K) / sum_t A[t][k] u[t]      (every group's total = n / K)
 *     u[t] = 1 / sum_k A[t][k] v[k]            (every token's row = 1)
 * so each row of G sums to 1 and, as iters grows, each column to n / K.
 * scores [B][n][K] fp32 (not modified), G [B][n][K] fp32 (out, must not
 * overlap scores). tau and iters are the caller's: the pages give neither.
 * Computed in fp32 (row max subtracted before the exponent, which cancels
 * exactly in u), one pass over the scores per round; sums in a fixed order,
 * so results are bitwise reproducible.
 * Limits: 1 <= K <= 64; 1 <= B <= 65535; n >= 1; 0 <= iters <= 10000;
 *   tau finite and > 0.
 * ---------------------------------------------------------------------- */
focus_status focus_assign_scores(const float* hidden, const float* P, const float* C,
                                 const float* bias, int B, int n, int d_model, int d_proj, int K,
                                 float* scores, void* workspace, size_t workspace_bytes,
                                 focus_stream_t stream);
size_t focus_sinkhorn_workspace_bytes(int B, int n, int K, int iters);
focus_status focus_sinkhorn(const float* scores, int B, int n, int K, float tau, int iters,
                            float* G, void* workspace, size_t workspace_bytes,
                            focus_stream_t stream);

/* ------------------------------------------------------------------------
 * Step 2: stable grouping of tokens (counting sort per batch element).
 *
 * The grouping the method rests on (Japanese page §2, opening: tokens are
 * gathered into groups by learnable centroids and far attention is limited
 * to pairs inside one group; §2.2: at inference, far pairs of different
 * groups are skipped, not zeroed; Korean page §2.3: the sparse pattern splits
 * into a local-window call and an intra-group long-range call). The
 * intra-group call attends each group's tokens among themselves, so the
 * tokens are laid out group by group, in sequence order inside each group;
 * this is that layout.
 *
 * group_offsets[b][k] = number of tokens of batch b whose id is < k (K+1
 *                       entries; empty groups repeat an offset)
 * perm[b][group_offsets[b][g] + r] = t, the r-th token (in increasing t)
 *                       with id g; so perm maps sorted slot -> position and
 *                       positions increase inside each group's segment.
 * group_ids [B][n] int32 in [0, K) (values outside are clamped)
 * perm [B][n] int32 (out), group_offsets [B][K+1] int32 (out)
 * workspace: per-block group counts, focus_group_sort_workspace_bytes() bytes
 * Limits: 1 <= K <= 64; 1 <= B <= 65535; n >= 1.
 * Top-k variant: pass the [B][n][m] ids of focus_assign_topk with n*m in
 * place of n. The sort then orders membership entries e = t*m + c (token t's
 * c-th group): perm [B][n*m] holds entries, each group's segment lists its
 * tokens once each in increasing position t = e / m.
 * ---------------------------------------------------------------------- */
size_t focus_group_sort_workspace_bytes(int B, int n, int K);
focus_status focus_group_sort(const int32_t* group_ids, int B, int n, int K,
                              int32_t* perm, int32_t* group_offsets,
                              void* workspace, size_t workspace_bytes, focus_stream_t stream);

/* focus_group_sort without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, results and limits, minus the
 * workspace: the per-block group counts go to a static device array of the
 * library, FOCUS_SORT_NOALLOC_SCRATCH_BYTES (1 MiB) on every GPU it runs on,
 * held until the process ends. The call allocates nothing; on its first use
 * on a device it looks up that device's copy of the array (the device current
 * at the call, which must be the stream's device).
 * Limit: focus_group_sort_workspace_bytes(B, n, K) <= 1 MiB, i.e.
 *   B * ceil(n / 2048) * K <= 262144 (e.g. B = 8 at n = 2^20, K = 64); larger
 *   requests return FOCUS_ERR_UNSUPPORTED and enqueue nothing.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (different streams or threads with no ordering between them) race and
 * give wrong results. Calls ordered on one stream are safe; no state carries
 * from one call to the next. */
#define FOCUS_SORT_NOALLOC_SCRATCH_BYTES (1u << 20)
focus_status focus_group_sort_noalloc(const int32_t* group_ids, int B, int n, int K,
                                      int32_t* perm, int32_t* group_offsets,
                                      focus_stream_t stream);

/* ------------------------------------------------------------------------
 * Step 3: exact-softmax attention over the Focus pattern (Korean page §2.1
 * and §2.3; Japanese page §2.1-§2.2). For query row (b, h, i), with kv head
 * h / (Hq / Hkv) and groups shared by all heads of a token:
 *
 *   A_i = { j : 0 <= i - j <= window }  U  { j : j < i - window,
 *                                             group_ids[b][j] == group_ids[b][i] }
 *   out[b][h][i] = sum_{j in A_i} softmax_j(scale * q_i . k_j) v_j
 *   lse[b][h][i] = log sum_{j in A_i} exp(scale * q_i . k_j)   (natural log)
 *
 * Each allowed pair is counted once (the two sets are disjoint). The work is
 * done in two passes, as the Korean page §2.3 splits the pattern: a
 * local-window pass in sequence order, which needs no group data, and an
 * intra-group long-range pass in group-sorted order (tiles of keys from
 * other groups are never visited) that merges both parts by log-sum-exp and
 * writes the result.
 *
 * q [B][Hq][n][d_head] bf16 bits; k, v [B][Hkv][n][d_head] bf16 bits
 * group_ids [B][n], perm [B][n], group_offsets [B][K+1]: as produced by
 *   focus_group_sort from the same ids
 * out [B][Hq][n][d_head], bf16 (round to nearest even) or fp32 per out_dtype;
 *   must not overlap q, k or v
 * lse [B][Hq][n] fp32 or NULL
 * Limits: d_head in {32, 64, 128}; 1 <= K <= 64; Hq % Hkv == 0; window >= 0;
 *   scale finite and > 0; B, n >= 1.
 * ---------------------------------------------------------------------- */
size_t focus_attn_workspace_bytes(int B, int Hq, int Hkv, int n, int d_head, int K, int window);
focus_status focus_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* group_ids, const int32_t* perm,
                            const int32_t* group_offsets,
                            int B, int Hq, int Hkv, int n, int d_head, int K, int window,
                            float scale, void* out, focus_dtype out_dtype, float* lse,
                            void* workspace, size_t workspace_bytes, focus_stream_t stream);

/* focus_attn_fwd with the long-range pass reading group-sorted copies of K
 * and V, which its preparation gathers into the workspace, instead of key
 * rows in place at the positions perm gives. focus_attn_fwd takes this path
 * by itself when one kv head's rows of K span 2^31 bytes or more (beyond a
 * buffer resource's reach), and the top-k calls always take it; this entry
 * point takes it at any size, so the path can be checked against the in-place
 * one (both load the same rows into every key tile, so the results agree bit
 * for bit). Same arguments and semantics as focus_attn_fwd; the workspace is
 * focus_attn_sorted_kv_workspace_bytes() bytes (the sorted K and V add
 * 2 * B * Hkv * n * d_head * 2 bytes to focus_attn_workspace_bytes()). */
size_t focus_attn_sorted_kv_workspace_bytes(int B, int Hq, int Hkv, int n, int d_head, int K,
                                            int window);
focus_status focus_attn_fwd_sorted_kv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                      const int32_t* group_ids, const int32_t* perm,
                                      const int32_t* group_offsets,
                                      int B, int Hq, int Hkv, int n, int d_head, int K,
                                      int window, float scale, void* out, focus_dtype out_dtype,
                                      float* lse, void* workspace, size_t workspace_bytes,
                                      focus_stream_t stream);

/* The two passes of focus_attn_fwd as separate calls, with the same
 * arguments and the same workspace, which carries the window partial result
 * from the first call to the second: focus_attn_fwd == focus_attn_window
 * then focus_attn_long_range_merge on one stream.
 *
 * focus_attn_window reads no group data (group_ids, perm and group_offsets
 * may be NULL), so a caller can run it on a second stream while the groups
 * are assigned and sorted, and start focus_attn_long_range_merge once both
 * are done. When no pair can lie beyond the window (n - 1 <= window) it
 * writes out and lse itself and focus_attn_long_range_merge does nothing;
 * otherwise it writes only the workspace. A workspace must not be used by a
 * second window pass before the merge of the first has run. */
focus_status focus_attn_window(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const int32_t* group_ids, const int32_t* perm,
                               const int32_t* group_offsets,
                               int B, int Hq, int Hkv, int n, int d_head, int K, int window,
                               float scale, void* out, focus_dtype out_dtype, float* lse,
                               void* workspace, size_t workspace_bytes, focus_stream_t stream);
focus_status focus_attn_long_range_merge(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                         const int32_t* group_ids, const int32_t* perm,
                                         const int32_t* group_offsets,
                                         int B, int Hq, int Hkv, int n, int d_head, int K,
                                         int window, float scale, void* out,
                                         focus_dtype out_dtype, float* lse, void* workspace,
                                         size_t workspace_bytes, focus_stream_t stream);

/* focus_attn_long_range_merge in two calls, with its arguments and workspace:
 * focus_attn_long_range_merge == focus_attn_long_range_prepare then
 * focus_attn_long_range_apply on one stream.
 *
 * focus_attn_long_range_prepare reads only k, v and the group data (q, out
 * and lse are checked, not read) and writes the query-tile plan and order
 * and each sorted row's key-slot end into the workspace; with two groups per
 * token, or when one kv head's rows of K span 2^31 bytes or more, also
 * group-sorted copies of K and V (otherwise the long-range pass reads key
 * rows in place, at the positions perm gives). Which of the two the calls
 * take depends only on the shape, so prepare and apply always agree. It
 * writes no part of the workspace that focus_attn_window writes, so it may
 * run on another stream while the window pass runs, once the sort is done. focus_attn_long_range_apply needs both (order them
 * before it with stream events): it runs the intra-group attention, merges
 * the window partial and writes out and lse. */
focus_status focus_attn_long_range_prepare(const uint16_t* q, const uint16_t* k,
                                           const uint16_t* v, const int32_t* group_ids,
                                           const int32_t* perm, const int32_t* group_offsets,
                                           int B, int Hq, int Hkv, int n, int d_head, int K,
                                           int window, float scale, void* out,
                                           focus_dtype out_dtype, float* lse, void* workspace,
                                           size_t workspace_bytes, focus_stream_t stream);
focus_status focus_attn_long_range_apply(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                         const int32_t* group_ids, const int32_t* perm,
                                         const int32_t* group_offsets,
                                         int B, int Hq, int Hkv, int n, int d_head, int K,
                                         int window, float scale, void* out,
                                         focus_dtype out_dtype, float* lse, void* workspace,
                                         size_t workspace_bytes, focus_stream_t stream);

/* ------------------------------------------------------------------------
 * Step 3, top-k variant (Korean page §2.3 and §3.4; Japanese page §2.2 and
 * §3.3): each token belongs to m groups (m = 2 in the pages' runs), and a far
 * pair is kept when the two tokens share at least one group:
 *
 *   A_i = { j : 0 <= i - j <= window }  U  { j : j < i - window,
 *           groups(i) and groups(j) intersect },  groups(t) = group_ids[b][t][*]
 *
 * with out and lse as for focus_attn_fwd. Each kept pair is counted once.
 * The long-range pass takes one of two forms, chosen by K:
 *   - m = 2 and K <= 4 (at most 6 membership sets; the pages' runs use
 *     K = 4, k = 2): the prepare call sorts the tokens by their set of two
 *     groups (a counting sort into the workspace; perm and group_offsets are
 *     checked but not read) and gathers set-sorted copies of K and V; a query
 *     tile of set S visits the key segments of every set sharing a group
 *     with S, so each kept pair meets exactly once, and the pass merges the
 *     window partial and writes out and lse itself.
 *   - otherwise (membership entries, m = 2): keys are the n*2 entries in
 *     the caller's group order; the query rows are taken in two passes, the
 *     tokens' first-group entries then their second-group entries (each in
 *     group order). The first pass merges its keys into the window partial
 *     in place, the second merges its keys into that and writes out and
 *     lse. A pair sharing two groups meets in both groups' segments and is
 *     kept only where the query row's group is the lower of the two.
 *
 * group_ids [B][n][m] (distinct groups per token, as from focus_assign_topk),
 * perm [B][n*m] and group_offsets [B][K+1] from focus_group_sort over the
 * n*m entries. Other arguments and layouts as focus_attn_fwd.
 * Limits: 1 <= m <= FOCUS_MAX_MEMBERSHIPS, m <= K, n*m <= 2^24; otherwise as
 *   focus_attn_fwd. With m = 1 the calls equal focus_attn_fwd and
 *   focus_attn_long_range_merge.
 *
 * focus_attn_topk_fwd == focus_attn_window then
 * focus_attn_topk_long_range_merge on one stream, with the workspace of
 * focus_attn_topk_workspace_bytes() passed to both (the window pass uses its
 * leading part, the window partial, laid out the same for every m).
 * ---------------------------------------------------------------------- */
size_t focus_attn_topk_workspace_bytes(int B, int Hq, int Hkv, int n, int d_head, int K, int m,
                                       int window);
focus_status focus_attn_topk_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const int32_t* group_ids, const int32_t* perm,
                                 const int32_t* group_offsets,
                                 int B, int Hq, int Hkv, int n, int d_head, int K, int m,
                                 int window, float scale, void* out, focus_dtype out_dtype,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 focus_stream_t stream);
focus_status focus_attn_topk_long_range_merge(const uint16_t* q, const uint16_t* k,
                                              const uint16_t* v, const int32_t* group_ids,
                                              const int32_t* perm, const int32_t* group_offsets,
                                              int B, int Hq, int Hkv, int n, int d_head, int K,
                                              int m, int window, float scale, void* out,
                                              focus_dtype out_dtype, float* lse,
                                              void* workspace, size_t workspace_bytes,
                                              focus_stream_t stream);
/* focus_attn_topk_long_range_merge in two calls, as for m = 1 above:
 * prepare (sorted K/V over the n*m entries and the query order of the two
 * entry passes, or over the tokens in membership-set order when K <= 4; plan
 * and order; may run beside the window pass) then apply (the two entry
 * passes, or the set pass; either merges the window partial itself). */
focus_status focus_attn_topk_long_range_prepare(const uint16_t* q, const uint16_t* k,
                                                const uint16_t* v, const int32_t* group_ids,
                                                const int32_t* perm,
                                                const int32_t* group_offsets, int B, int Hq,
                                                int Hkv, int n, int d_head, int K, int m,
                                                int window, float scale, void* out,
                                                focus_dtype out_dtype, float* lse,
                                                void* workspace, size_t workspace_bytes,
                                                focus_stream_t stream);
focus_status focus_attn_topk_long_range_apply(const uint16_t* q, const uint16_t* k,
                                              const uint16_t* v, const int32_t* group_ids,
                                              const int32_t* perm, const int32_t* group_offsets,
                                              int B, int Hq, int Hkv, int n, int d_head, int K,
                                              int m, int window, float scale, void* out,
                                              focus_dtype out_dtype, float* lse,
                                              void* workspace, size_t workspace_bytes,
                                              focus_stream_t stream);

/* ------------------------------------------------------------------------
 * Training-time soft-gated attention (Japanese page §2.1: group affinity
 * a_ij = g_i . g_j of the soft assignments and the gate sigmoid(lambda a_ij);
 * §2.2: while training the gate is soft and every pair is computed, O(n^2);
 * Korean page §2.1: the local window is attended at full resolution and the
 * softmax is kept exact). The pages' "product of the local mask and the
 * gate" is read as: pairs inside the causal window pass unchanged and pairs
 * beyond it are scaled by the gate, inside one renormalised softmax:
 *
 *   gate_ij = 1 for 0 <= i - j <= window, sigmoid(lambda * a_ij) for i - j > window
 *   out[b][h][i] = sum_{j <= i} gate_ij exp(scale q_i.k_j) v_j / sum_{j <= i} gate_ij exp(scale q_i.k_j)
 *   lse[b][h][i] = log sum_{j <= i} gate_ij exp(scale q_i.k_j)
 *
 * G [B][n][K] fp32 soft assignments (e.g. the rows of focus_sinkhorn's
 * output; any values are accepted), shared by all heads of a token. The
 * affinity is computed from a bf16 hi/lo split of G (about 2^-16 relative).
 * Other arguments and layouts as dense_causal_attn_fwd; lambda finite (any
 * sign). Workspace: focus_soft_gate_attn_workspace_bytes() bytes (the split
 * copy of G). Limits: 1 <= K <= 64, d_head in {32, 64, 128}.
 * ---------------------------------------------------------------------- */
size_t focus_soft_gate_attn_workspace_bytes(int B, int n, int K);
focus_status focus_soft_gate_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                      const float* G, int B, int Hq, int Hkv, int n, int d_head,
                                      int K, int window, float scale, float lambda, void* out,
                                      focus_dtype out_dtype, float* lse, void* workspace,
                                      size_t workspace_bytes, focus_stream_t stream);

/* ------------------------------------------------------------------------
 * Baseline: plain causal attention (every pair j <= i), the full attention
 * the Focus pages measure their speed-ups against (Korean page §2.3: 2x to
 * 8.6x over it with two FlashAttention calls; §3.4 and Japanese page §3.3:
 * 8.6x wall-clock at one million tokens, 2x with top-2 membership at K = 4).
 * It runs on the same kernel core as the Focus passes, so the speed-up of
 * focus_attn_fwd over it isolates the pairs skipped. Same layouts and limits
 * as above; needs no workspace.
 *
 *   out[b][h][i] = sum_{j <= i} softmax_j(scale * q_i . k_j) v_j
 *   lse[b][h][i] = log sum_{j <= i} exp(scale * q_i . k_j)   (natural log)
 * ---------------------------------------------------------------------- */
focus_status dense_causal_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   int B, int Hq, int Hkv, int n, int d_head, float scale,
                                   void* out, focus_dtype out_dtype, float* lse,
                                   focus_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FOCUS_H_ */
