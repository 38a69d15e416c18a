/*
 * Plain CPU oracle for the Focus group-gated attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library. The product path
 * never calls it and shares no code with it.
 *
 * Written from the method as the Focus pages describe it:
 *   - "Why Attend to Everything? Focus is the Key" (gist.science, Korean),
 *     technical summary §2.1 (K learnable centroids; local window pairs at full
 *     resolution; far pairs only inside one group; exact softmax kept) and
 *     §2.3 (inference switches to a hard discrete top-k group assignment;
 *     the pattern splits into a local-window part and an intra-group
 *     long-range part).
 *   - "Focus: Learning Which Attention Pairs Matter" (gist.science, Japanese),
 *     technical summary §2.1 (hidden state h_i is projected and compared with
 *     the centroids in centroid space) and §2.2 (at inference each token takes
 *     its top-k groups; far cross-group pairs are skipped, not zeroed; pair
 *     count O(n^2/K + n*w)).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   similarity = dot product of h·P with the rows of C, top-1 group, exact
 *   ties go to the lowest group index; the window is the causal band
 *   0 <= i-j <= w; long-range pairs are causal (j <= i); an allowed pair is
 *   counted once; the softmax is renormalised over the allowed set.
 *   Sinkhorn (training-time soft assignment): Sinkhorn-Knopp on exp(scores /
 *   tau), rows first, then a caller-given number of (column, row) rounds;
 *   every column's target is n / K (only its being equal matters: the final
 *   row step cancels a common factor); tau and the number of rounds are not
 *   given by the pages and are arguments.
 *   Soft gate (training): every causal pair is computed; pairs beyond the
 *   window are weighted by sigmoid(lambda * g_i . g_j) inside an exact,
 *   renormalised softmax (the pages' "product of the local mask and the
 *   gate" read as: the window passes unchanged, the gate scales the rest).
 *   Multi-membership (top-m groups per token, m = 2 in the pages' runs): a far
 *   pair is kept when the tokens share at least one group, and still counted
 *   once; the top-m groups are the m highest scores, ties to the lowest index.
 *
 * Precision: assignment in fp32 (build with -ffp-contract=off, sums in
 * ascending index order, as written); attention in fp64 on the exact values
 * of the bf16 inputs; exp/log from the C library.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_version(void) { return 1; }

/* bf16 is the upper half of an IEEE binary32: widen by a 16-bit shift. */
static double bf16_value(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Scores of one token: z = h P (fp32, summed in increasing index), then
 * s[k] = z . C_k + bias_k. */
static void token_scores(const float* h, const float* P, const float* C, const float* bias,
                         int64_t d_model, int64_t d_proj, int64_t K, float* z, float* s) {
    for (int64_t j = 0; j < d_proj; ++j) z[j] = 0.0f;
    for (int64_t m = 0; m < d_model; ++m) {
        const float hm = h[m];
        const float* Prow = P + m * d_proj;
        for (int64_t j = 0; j < d_proj; ++j) z[j] = z[j] + hm * Prow[j];
    }
    for (int64_t k = 0; k < K; ++k) {
        float acc = 0.0f;
        const float* Ck = C + k * d_proj;
        for (int64_t j = 0; j < d_proj; ++j) acc = acc + z[j] * Ck[j];
        s[k] = bias ? acc + bias[k] : acc;
    }
}

/*
 * Hard group assignment (Japanese page §2.1 and §2.2; Korean page §2.3):
 *   z = h_t · P            (d_proj values, each summed over m = 0..d_model-1)
 *   s_k = z · C_k + bias_k (summed over j = 0..d_proj-1, then the bias added)
 *   id = smallest k with s_k = max s
 *   margin = s_(1) - s_(2) (+inf when K == 1)
 * tokens: flattened indices b*n + t to evaluate, or NULL for all B*n tokens in
 * order; outputs are indexed by position in that list.
 */
int oracle_assign(const float* hidden, const float* P, const float* C, const float* bias,
                  int64_t B, int64_t n, int64_t d_model, int64_t d_proj, int64_t K,
                  const int64_t* tokens, int64_t ntokens,
                  int32_t* ids, float* margin, int nthreads) {
    if (!hidden || !P || !C || !ids || B < 1 || n < 1 || d_model < 1 || d_proj < 1 || K < 1)
        return -1;
    int64_t count = tokens ? ntokens : B * n;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel
    {
        float* z = (float*)malloc(sizeof(float) * (size_t)d_proj);
        float* s = (float*)malloc(sizeof(float) * (size_t)K);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < count; ++r) {
            int64_t tok = tokens ? tokens[r] : r;
            if (tok < 0 || tok >= B * n) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            token_scores(hidden + tok * d_model, P, C, bias, d_model, d_proj, K, z, s);
            int64_t best = 0;
            for (int64_t k = 1; k < K; ++k)
                if (s[k] > s[best]) best = k;
            float second = -INFINITY;
            for (int64_t k = 0; k < K; ++k)
                if (k != best && s[k] > second) second = s[k];
            ids[r] = (int32_t)best;
            if (margin) margin[r] = (K == 1) ? INFINITY : s[best] - second;
        }
        free(z);
        free(s);
    }
    return bad ? -1 : 0;
}

/*
 * Stable grouping of tokens (the grouping step; the pages only say tokens are
 * grouped): counting sort per batch element.
 *   offsets[b][k] = number of tokens of batch b with id < k  (K+1 entries)
 *   perm[b][offsets[b][g] + r] = t, where t is the r-th token (in increasing t)
 *   whose id is g.
 */
int oracle_group_sort(const int32_t* ids, int64_t B, int64_t n, int64_t K,
                      int32_t* perm, int32_t* offsets) {
    if (!ids || !perm || !offsets || B < 1 || n < 1 || K < 1) return -1;
    int64_t* seen = (int64_t*)malloc(sizeof(int64_t) * (size_t)K);
    for (int64_t b = 0; b < B; ++b) {
        const int32_t* g = ids + b * n;
        int32_t* off = offsets + b * (K + 1);
        for (int64_t k = 0; k <= K; ++k) off[k] = 0;
        for (int64_t t = 0; t < n; ++t) {
            if (g[t] < 0 || g[t] >= K) { free(seen); return -1; }
            off[g[t] + 1] += 1;
        }
        for (int64_t k = 0; k < K; ++k) off[k + 1] += off[k];
        for (int64_t k = 0; k < K; ++k) seen[k] = 0;
        for (int64_t t = 0; t < n; ++t) {
            int32_t k = g[t];
            perm[b * n + off[k] + seen[k]] = (int32_t)t;
            seen[k] += 1;
        }
    }
    free(seen);
    return 0;
}

/* Allowed-pair predicate: the causal window band or the same group, causal. */
static int pair_allowed(int64_t i, int64_t j, int64_t w, int32_t gi, int32_t gj) {
    if (j > i) return 0;
    if (i - j <= w) return 1;
    return gi == gj;
}

/* Softmax attention of one query row over an explicit key list (fp64). */
static void attend_list(const uint16_t* qrow, const uint16_t* kbase, const uint16_t* vbase,
                        int64_t d, double scale, const int64_t* keys, int64_t cnt,
                        double* s, double* out, double* lse) {
    for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
    if (cnt == 0) {
        *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (int64_t a = 0; a < cnt; ++a) {
        const uint16_t* krow = kbase + keys[a] * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += bf16_value(qrow[c]) * bf16_value(krow[c]);
        s[a] = scale * dot;
        if (s[a] > m) m = s[a];
    }
    double l = 0.0;
    for (int64_t a = 0; a < cnt; ++a) {
        double p = exp(s[a] - m);
        l += p;
        const uint16_t* vrow = vbase + keys[a] * d;
        for (int64_t c = 0; c < d; ++c) out[c] += p * bf16_value(vrow[c]);
    }
    for (int64_t c = 0; c < d; ++c) out[c] /= l;
    *lse = m + log(l);
}

static int check_attn_args(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const int32_t* ids, int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                           int64_t d, int64_t w) {
    if (!q || !k || !v || !ids) return -1;
    if (B < 1 || Hq < 1 || Hkv < 1 || n < 1 || d < 1 || w < 0 || Hq % Hkv) return -1;
    return 0;
}

/*
 * Exact masked softmax attention (Korean page §2.1 and §2.3, Japanese page
 * §2.1 and §2.2): for row (b, h, i) with kv head h / (Hq/Hkv),
 *   A_i = { j : j <= i and (i - j <= w or id[b][j] == id[b][i]) }
 *   out = sum_{j in A_i} softmax_j(scale * q_i·k_j) v_j,  lse = log sum exp.
 * rows: flattened (b*Hq + h)*n + i, or NULL for every row in order.
 * out [nrows][d], lse [nrows], visited [nrows] = |A_i| (each may be NULL
 * except out).
 */
int oracle_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* ids,
                int64_t B, int64_t Hq, int64_t Hkv, int64_t n, int64_t d, int64_t w,
                double scale, const int64_t* rows, int64_t nrows,
                double* out, double* lse, int64_t* visited, int nthreads) {
    if (check_attn_args(q, k, v, ids, B, Hq, Hkv, n, d, w) || !out) return -1;
    int64_t count = rows ? nrows : B * Hq * n;
    int64_t group = Hq / Hkv;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)n);
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < count; ++r) {
            int64_t row = rows ? rows[r] : r;
            if (row < 0 || row >= B * Hq * n) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            int64_t i = row % n, bh = row / n, h = bh % Hq, b = bh / Hq;
            int64_t kvh = h / group;
            const int32_t* g = ids + b * n;
            int64_t cnt = 0;
            for (int64_t j = 0; j <= i; ++j)
                if (pair_allowed(i, j, w, g[i], g[j])) keys[cnt++] = j;
            double l_se;
            attend_list(q + row * d, k + (b * Hkv + kvh) * n * d, v + (b * Hkv + kvh) * n * d,
                        d, scale, keys, cnt, s, out + r * d, &l_se);
            if (lse) lse[r] = l_se;
            if (visited) visited[r] = cnt;
        }
        free(s);
        free(keys);
    }
    return bad ? -1 : 0;
}

/*
 * The same result in two parts, as the Korean page §2.3 splits the pattern
 * (a local-window attention and an intra-group long-range attention), joined
 * by the log-sum-exp identity:
 *   W_i = { j : 0 <= i - j <= w },  L_i = { j : i - j > w, id_j == id_i }
 *   M = max(lse_W, lse_L), a = exp(lse_W - M), c = exp(lse_L - M)
 *   out = (a out_W + c out_L) / (a + c),  lse = M + log(a + c)
 * W_i and L_i are disjoint with union A_i, so each pair is counted once.
 */
int oracle_attn_two_phase(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const int32_t* ids, int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                          int64_t d, int64_t w, double scale, const int64_t* rows,
                          int64_t nrows, double* out, double* lse, int nthreads) {
    if (check_attn_args(q, k, v, ids, B, Hq, Hkv, n, d, w) || !out) return -1;
    int64_t count = rows ? nrows : B * Hq * n;
    int64_t group = Hq / Hkv;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)n);
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
        double* ow = (double*)malloc(sizeof(double) * (size_t)d);
        double* ol = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < count; ++r) {
            int64_t row = rows ? rows[r] : r;
            if (row < 0 || row >= B * Hq * n) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            int64_t i = row % n, bh = row / n, h = bh % Hq, b = bh / Hq;
            int64_t kvh = h / group;
            const int32_t* g = ids + b * n;
            const uint16_t* kb = k + (b * Hkv + kvh) * n * d;
            const uint16_t* vb = v + (b * Hkv + kvh) * n * d;
            int64_t cnt = 0;
            for (int64_t j = (i - w > 0 ? i - w : 0); j <= i; ++j) keys[cnt++] = j;
            double lw, ll;
            attend_list(q + row * d, kb, vb, d, scale, keys, cnt, s, ow, &lw);
            cnt = 0;
            for (int64_t j = 0; j < i - w; ++j)
                if (g[j] == g[i]) keys[cnt++] = j;
            attend_list(q + row * d, kb, vb, d, scale, keys, cnt, s, ol, &ll);
            double M = lw > ll ? lw : ll;
            double a = exp(lw - M);
            double c = (ll == -INFINITY) ? 0.0 : exp(ll - M);
            for (int64_t x = 0; x < d; ++x) out[r * d + x] = (a * ow[x] + c * ol[x]) / (a + c);
            if (lse) lse[r] = M + log(a + c);
        }
        free(s);
        free(keys);
        free(ow);
        free(ol);
    }
    return bad ? -1 : 0;
}

/*
 * Full softmax weight row of one query (for invariant checks on small cases):
 * weights[j] = softmax weight of pair (i, j), exactly 0 for j outside A_i.
 */
int oracle_attn_weights(const uint16_t* q, const uint16_t* k, const int32_t* ids,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t n, int64_t d, int64_t w,
                        double scale, int64_t b, int64_t h, int64_t i, double* weights) {
    if (!q || !k || !ids || !weights || B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || n < 1 ||
        d < 1 || w < 0 || b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= n)
        return -1;
    int64_t kvh = h / (Hq / Hkv);
    const uint16_t* qrow = q + ((b * Hq + h) * n + i) * d;
    const uint16_t* kb = k + (b * Hkv + kvh) * n * d;
    const int32_t* g = ids + b * n;
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        weights[j] = 0.0;
        if (!pair_allowed(i, j, w, g[i], g[j])) continue;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += bf16_value(qrow[c]) * bf16_value(kb[j * d + c]);
        weights[j] = scale * dot;
        if (weights[j] > m) m = weights[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j)
        if (pair_allowed(i, j, w, g[i], g[j])) {
            weights[j] = exp(weights[j] - m);
            l += weights[j];
        }
    for (int64_t j = 0; j < n; ++j)
        if (pair_allowed(i, j, w, g[i], g[j])) weights[j] /= l;
    return 0;
}

/* Number of allowed pairs sum_b sum_i |A_i| for one batch of ids (per head). */
int64_t oracle_pair_count(const int32_t* ids, int64_t B, int64_t n, int64_t w, int nthreads) {
    if (!ids || B < 1 || n < 1 || w < 0) return -1;
    set_threads(nthreads);
    int64_t total = 0;
    for (int64_t b = 0; b < B; ++b) {
        const int32_t* g = ids + b * n;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : total)
        for (int64_t i = 0; i < n; ++i) {
            int64_t cnt = 0;
            for (int64_t j = 0; j <= i; ++j) cnt += pair_allowed(i, j, w, g[i], g[j]);
            total += cnt;
        }
    }
    return total;
}

/* ------------------------------------------------------------------------
 * Multi-membership variant (Korean page §2.3 and Japanese page §2.2: at
 * inference each token takes its top-k groups; the Korean page §3.4 and
 * the Japanese page §3.3 report k = 2 at K = 4). A far pair is kept when the
 * two tokens share ANY group; the kept set is a set, so a pair sharing two
 * groups is still counted once.
 * ---------------------------------------------------------------------- */

/*
 * Top-m groups of each token, by the same fp32 scores as oracle_assign:
 * ids[r][0..m-1] = the m highest scores in decreasing order, exact ties to
 * the lowest index; margin[r] = s_(m) - s_(m+1) (+inf when K == m), the
 * score gap that decides membership of the m-th group.
 */
int oracle_assign_topk(const float* hidden, const float* P, const float* C, const float* bias,
                       int64_t B, int64_t n, int64_t d_model, int64_t d_proj, int64_t K,
                       int64_t m, const int64_t* tokens, int64_t ntokens,
                       int32_t* ids, float* margin, int nthreads) {
    if (!hidden || !P || !C || !ids || B < 1 || n < 1 || d_model < 1 || d_proj < 1 || K < 1 ||
        m < 1 || m > K)
        return -1;
    int64_t count = tokens ? ntokens : B * n;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel
    {
        float* z = (float*)malloc(sizeof(float) * (size_t)d_proj);
        float* s = (float*)malloc(sizeof(float) * (size_t)K);
        char* taken = (char*)malloc((size_t)K);
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < count; ++r) {
            int64_t tok = tokens ? tokens[r] : r;
            if (tok < 0 || tok >= B * n) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            token_scores(hidden + tok * d_model, P, C, bias, d_model, d_proj, K, z, s);
            for (int64_t k = 0; k < K; ++k) taken[k] = 0;
            float last = 0.0f;
            for (int64_t c = 0; c < m; ++c) {       /* repeated argmax over the rest */
                int64_t best = -1;
                for (int64_t k = 0; k < K; ++k)
                    if (!taken[k] && (best < 0 || s[k] > s[best])) best = k;
                taken[best] = 1;
                ids[r * m + c] = (int32_t)best;
                last = s[best];
            }
            float next = -INFINITY;
            for (int64_t k = 0; k < K; ++k)
                if (!taken[k] && s[k] > next) next = s[k];
            if (margin) margin[r] = (K == m) ? INFINITY : last - next;
        }
        free(z);
        free(s);
        free(taken);
    }
    return bad ? -1 : 0;
}

/* Does token j (groups gj[0..m-1]) share a group with token i (gi)? */
static int share_group(const int32_t* gi, const int32_t* gj, int64_t m) {
    for (int64_t a = 0; a < m; ++a)
        for (int64_t c = 0; c < m; ++c)
            if (gi[a] == gj[c]) return 1;
    return 0;
}

/*
 * Attention over the multi-membership pattern, fp64, same conventions as
 * oracle_attn: ids [B][n][m];
 *   A_i = { j : j <= i and (i - j <= w or groups(i) and groups(j) intersect) }.
 */
int oracle_attn_multi(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* ids, int64_t m, int64_t B, int64_t Hq, int64_t Hkv,
                      int64_t n, int64_t d, int64_t w, double scale, const int64_t* rows,
                      int64_t nrows, double* out, double* lse, int64_t* visited, int nthreads) {
    if (m < 1 || check_attn_args(q, k, v, ids, B, Hq, Hkv, n, d, w) || !out) return -1;
    int64_t count = rows ? nrows : B * Hq * n;
    int64_t group = Hq / Hkv;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)n);
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < count; ++r) {
            int64_t row = rows ? rows[r] : r;
            if (row < 0 || row >= B * Hq * n) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            int64_t i = row % n, bh = row / n, h = bh % Hq, b = bh / Hq;
            int64_t kvh = h / group;
            const int32_t* g = ids + b * n * m;
            int64_t cnt = 0;
            for (int64_t j = 0; j <= i; ++j)
                if (i - j <= w || share_group(g + i * m, g + j * m, m)) keys[cnt++] = j;
            double l_se;
            attend_list(q + row * d, k + (b * Hkv + kvh) * n * d, v + (b * Hkv + kvh) * n * d,
                        d, scale, keys, cnt, s, out + r * d, &l_se);
            if (lse) lse[r] = l_se;
            if (visited) visited[r] = cnt;
        }
        free(s);
        free(keys);
    }
    return bad ? -1 : 0;
}

/* Sum over b and i of |A_i| for the multi-membership pattern. */
int64_t oracle_pair_count_multi(const int32_t* ids, int64_t m, int64_t B, int64_t n, int64_t w,
                                int nthreads) {
    if (!ids || m < 1 || B < 1 || n < 1 || w < 0) return -1;
    set_threads(nthreads);
    int64_t total = 0;
    for (int64_t b = 0; b < B; ++b) {
        const int32_t* g = ids + b * n * m;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : total)
        for (int64_t i = 0; i < n; ++i) {
            int64_t cnt = 0;
            for (int64_t j = 0; j <= i; ++j)
                cnt += (i - j <= w) || share_group(g + i * m, g + j * m, m);
            total += cnt;
        }
    }
    return total;
}

/* ------------------------------------------------------------------------
 * Soft assignment with Sinkhorn normalisation (training-time step; Korean
 * page §2.2 and Japanese page §2.1 / §2.3): the n x K assignment matrix of
 * one sequence is made doubly stochastic, i.e. every token's row sums to 1
 * and every group's column sums to the same total n / K.
 * ---------------------------------------------------------------------- */

/* Raw scores s[t][k] = (h_t . P) . C_k + bias_k, fp32, as in oracle_assign. */
int oracle_assign_scores(const float* hidden, const float* P, const float* C, const float* bias,
                         int64_t B, int64_t n, int64_t d_model, int64_t d_proj, int64_t K,
                         float* scores, int nthreads) {
    if (!hidden || !P || !C || !scores || B < 1 || n < 1 || d_model < 1 || d_proj < 1 || K < 1)
        return -1;
    set_threads(nthreads);
#pragma omp parallel
    {
        float* z = (float*)malloc(sizeof(float) * (size_t)d_proj);
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < B * n; ++t)
            token_scores(hidden + t * d_model, P, C, bias, d_model, d_proj, K, z, scores + t * K);
        free(z);
    }
    return 0;
}

/*
 * Sinkhorn-Knopp on A = exp(scores / tau) for each batch element, fp64, in
 * the plain scaling-vector form G[t][k] = A[t][k] * u[t] * v[k]:
 *   u = 1 / (row sums of A)                                 (rows first)
 *   repeat iters times:
 *     v[k] = (n / K) / sum_t A[t][k] u[t]                     (columns)
 *     u[t] = 1 / sum_k A[t][k] v[k]                           (rows)
 * so every row of G sums to 1 and, as iters grows, every column to n / K.
 * v starts at 1. scores [B][n][K] fp32 -> G [B][n][K] fp64. The exponent is
 * taken as written, so |scores / tau| must stay below ~700.
 */
int oracle_sinkhorn(const float* scores, int64_t B, int64_t n, int64_t K, double tau,
                    int64_t iters, double* G) {
    if (!scores || !G || B < 1 || n < 1 || K < 1 || !(tau > 0.0) || iters < 0) return -1;
    double* A = (double*)malloc(sizeof(double) * (size_t)(n * K));
    double* u = (double*)malloc(sizeof(double) * (size_t)n);
    double* v = (double*)malloc(sizeof(double) * (size_t)K);
    double* col = (double*)malloc(sizeof(double) * (size_t)K);
    for (int64_t b = 0; b < B; ++b) {
        const float* S = scores + b * n * K;
        for (int64_t x = 0; x < n * K; ++x) A[x] = exp((double)S[x] / tau);
        for (int64_t k = 0; k < K; ++k) v[k] = 1.0;
        for (int64_t t = 0; t < n; ++t) {
            double r = 0.0;
            for (int64_t k = 0; k < K; ++k) r += A[t * K + k] * v[k];
            u[t] = 1.0 / r;
        }
        for (int64_t it = 0; it < iters; ++it) {
            for (int64_t k = 0; k < K; ++k) col[k] = 0.0;
            for (int64_t t = 0; t < n; ++t)
                for (int64_t k = 0; k < K; ++k) col[k] += A[t * K + k] * u[t];
            for (int64_t k = 0; k < K; ++k) v[k] = ((double)n / (double)K) / col[k];
            for (int64_t t = 0; t < n; ++t) {
                double r = 0.0;
                for (int64_t k = 0; k < K; ++k) r += A[t * K + k] * v[k];
                u[t] = 1.0 / r;
            }
        }
        double* Gb = G + b * n * K;
        for (int64_t t = 0; t < n; ++t)
            for (int64_t k = 0; k < K; ++k) Gb[t * K + k] = A[t * K + k] * u[t] * v[k];
    }
    free(A);
    free(u);
    free(v);
    free(col);
    return 0;
}

/* ------------------------------------------------------------------------
 * Training-time soft-gated attention (Japanese page §2.1: group affinity
 * a_ij = g_i . g_j of the soft assignments and a gate sigma(lambda a_ij);
 * §2.2: in training the gate is soft and every pair is computed, so the
 * cost stays O(n^2); Korean page §2.1: pairs inside the local window are
 * attended at full resolution, far pairs are controlled by the group gate,
 * and the softmax is kept exact). Reading: every causal pair enters the
 * softmax with weight gate_ij * exp(scale q_i . k_j), where gate_ij = 1 for
 * 0 <= i - j <= w and sigma(lambda a_ij) for i - j > w:
 *   out_i = sum_j gate_ij exp(s_ij) v_j / sum_j gate_ij exp(s_ij)
 *   lse_i = log sum_j gate_ij exp(s_ij)
 * G [B][n][K] fp32 soft assignments; everything else as oracle_attn.
 * ---------------------------------------------------------------------- */
int oracle_soft_gate_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const float* G, int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                          int64_t d, int64_t K, int64_t w, double scale, double lambda,
                          const int64_t* rows, int64_t nrows, double* out, double* lse,
                          int nthreads) {
    if (!q || !k || !v || !G || !out || B < 1 || Hq < 1 || Hkv < 1 || n < 1 || d < 1 || K < 1 ||
        w < 0 || Hq % Hkv)
        return -1;
    int64_t count = rows ? nrows : B * Hq * n;
    int64_t group = Hq / Hkv;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)n);
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < count; ++r) {
            int64_t row = rows ? rows[r] : r;
            if (row < 0 || row >= B * Hq * n) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            int64_t i = row % n, bh = row / n, h = bh % Hq, b = bh / Hq;
            int64_t kvh = h / group;
            const uint16_t* qrow = q + row * d;
            const uint16_t* kb = k + (b * Hkv + kvh) * n * d;
            const uint16_t* vb = v + (b * Hkv + kvh) * n * d;
            const float* gi = G + (b * n + i) * K;
            double m = -INFINITY;
            for (int64_t j = 0; j <= i; ++j) {
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c) dot += bf16_value(qrow[c]) * bf16_value(kb[j * d + c]);
                s[j] = scale * dot;
                if (s[j] > m) m = s[j];
            }
            double* o = out + r * d;
            for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
            double l = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                double gate = 1.0;
                if (i - j > w) {
                    const float* gj = G + (b * n + j) * K;
                    double a = 0.0;
                    for (int64_t x = 0; x < K; ++x) a += (double)gi[x] * (double)gj[x];
                    gate = 1.0 / (1.0 + exp(-lambda * a));
                }
                double p = gate * exp(s[j] - m);
                l += p;
                for (int64_t c = 0; c < d; ++c) o[c] += p * bf16_value(vb[j * d + c]);
            }
            for (int64_t c = 0; c < d; ++c) o[c] /= l;
            if (lse) lse[r] = m + log(l);
        }
        free(s);
    }
    return bad ? -1 : 0;
}
