// C ABI of libfocus.so (declared in include/focus.h): argument validation on
// the host, workspace sizing, and the kernel launches. Validation runs before
// any HIP call, so an invalid request enqueues nothing.
#include "focus.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "focus_internal.h"

namespace {

thread_local char g_err[512] = "";

focus_status fail(focus_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

focus_status ok() {
    g_err[0] = '\0';
    return FOCUS_OK;
}

focus_status device_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(FOCUS_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [p, p+bytes) and [q, q+qbytes) overlap?
bool overlaps(const void* p, size_t bytes, const void* q, size_t qbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + bytes;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(q), b1 = b0 + qbytes;
    return a0 < b1 && b0 < a1;
}

#define REQUIRE(cond, st, ...) \
    do {                        \
        if (!(cond)) return fail(st, __VA_ARGS__); \
    } while (0)

#define REQUIRE_PTR(p, align)                                                              \
    do {                                                                                   \
        if (!(p)) return fail(FOCUS_ERR_INVALID_ARGUMENT, "%s must not be NULL", #p);      \
        if (!aligned((p), (align)))                                                        \
            return fail(FOCUS_ERR_INVALID_ARGUMENT, "%s must be %d-byte aligned", #p,      \
                        (int)(align));                                                     \
    } while (0)

constexpr int64_t kMaxGrid = 2147483647;

struct AttnShape {
    int B, Hq, Hkv, n, d, K, w;
    int m = 1;   // groups per token
};

focus_status check_attn_shape(const AttnShape& s, bool needs_groups) {
    REQUIRE(s.B >= 1 && s.n >= 1, FOCUS_ERR_INVALID_ARGUMENT, "B and n must be >= 1 (got B=%d n=%d)",
            s.B, s.n);
    REQUIRE(s.Hq >= 1 && s.Hkv >= 1, FOCUS_ERR_INVALID_ARGUMENT, "Hq and Hkv must be >= 1");
    REQUIRE(s.Hq % s.Hkv == 0, FOCUS_ERR_INVALID_ARGUMENT,
            "Hq (%d) must be a multiple of Hkv (%d)", s.Hq, s.Hkv);
    REQUIRE(s.d == 32 || s.d == 64 || s.d == 128, FOCUS_ERR_UNSUPPORTED,
            "d_head must be 32, 64 or 128 (got %d)", s.d);
    if (needs_groups) {
        REQUIRE(s.K >= 1 && s.K <= FOCUS_MAX_GROUPS, FOCUS_ERR_UNSUPPORTED,
                "K must be in [1, %d] (got %d)", FOCUS_MAX_GROUPS, s.K);
        REQUIRE(s.w >= 0, FOCUS_ERR_INVALID_ARGUMENT, "window must be >= 0 (got %d)", s.w);
        REQUIRE(s.m >= 1 && s.m <= FOCUS_MAX_MEMBERSHIPS, FOCUS_ERR_UNSUPPORTED,
                "m must be in [1, %d] (got %d)", FOCUS_MAX_MEMBERSHIPS, s.m);
        REQUIRE(s.m <= s.K, FOCUS_ERR_INVALID_ARGUMENT, "m (%d) must be <= K (%d)", s.m, s.K);
        // entries of the sorted order: positions are packed with 6 bits of
        // group beside them when m = 2
        REQUIRE((int64_t)s.n * s.m <= (s.m == 1 ? (int64_t)INT32_MAX - 4096 : (int64_t)1 << 24),
                FOCUS_ERR_UNSUPPORTED, "n * m too large (n=%d, m=%d)", s.n, s.m);
    }
    const int64_t rows = (int64_t)s.B * s.Hq * s.n;
    REQUIRE(rows / s.Hq / s.B == s.n, FOCUS_ERR_INVALID_ARGUMENT, "B*Hq*n overflows");
    // Workgroup count of the attention grids: B * Hq * ceil(n * m / 16) / 8 at most.
    REQUIRE((int64_t)s.B * s.Hq * (((int64_t)s.n * s.m + 15) / 16) <= kMaxGrid,
            FOCUS_ERR_UNSUPPORTED,
            "problem too large for one launch grid");
    REQUIRE((int64_t)s.B * s.Hkv <= 65535, FOCUS_ERR_UNSUPPORTED, "B*Hkv must be <= 65535");
    return ok();
}

focus_status check_attn_buffers(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const AttnShape& s, void* out, focus_dtype out_dtype,
                                const float* lse, float scale) {
    REQUIRE_PTR(q, 16);
    REQUIRE_PTR(k, 16);
    REQUIRE_PTR(v, 16);
    REQUIRE_PTR(out, 16);
    if (lse) REQUIRE(aligned(lse, 4), FOCUS_ERR_INVALID_ARGUMENT, "lse must be 4-byte aligned");
    REQUIRE(out_dtype == FOCUS_BF16 || out_dtype == FOCUS_F32, FOCUS_ERR_INVALID_ARGUMENT,
            "out_dtype must be FOCUS_BF16 or FOCUS_F32");
    REQUIRE(std::isfinite(scale) && scale > 0.0f, FOCUS_ERR_INVALID_ARGUMENT,
            "scale must be finite and > 0");
    const size_t qbytes = (size_t)s.B * s.Hq * s.n * s.d * 2;
    const size_t kvbytes = (size_t)s.B * s.Hkv * s.n * s.d * 2;
    const size_t obytes = (size_t)s.B * s.Hq * s.n * s.d * (out_dtype == FOCUS_F32 ? 4 : 2);
    REQUIRE(!overlaps(out, obytes, q, qbytes) && !overlaps(out, obytes, k, kvbytes) &&
                !overlaps(out, obytes, v, kvbytes),
            FOCUS_ERR_INVALID_ARGUMENT, "out must not overlap q, k or v");
    if (lse) {
        const size_t lbytes = (size_t)s.B * s.Hq * s.n * 4;
        REQUIRE(!overlaps(lse, lbytes, out, obytes) && !overlaps(lse, lbytes, q, qbytes) &&
                    !overlaps(lse, lbytes, k, kvbytes) && !overlaps(lse, lbytes, v, kvbytes),
                FOCUS_ERR_INVALID_ARGUMENT, "lse must not overlap out, q, k or v");
    }
    return ok();
}

// kLongRangeMerge = kLongRangePrepare then kLongRangeApply
enum class AttnPart { kAll, kWindow, kLongRangeMerge, kLongRangePrepare, kLongRangeApply };

focus_status attn_entry(AttnPart part, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const int32_t* group_ids, const int32_t* perm,
                        const int32_t* group_offsets, int B, int Hq, int Hkv, int n, int d, int K,
                        int m, int w, float scale, void* out, focus_dtype out_dtype, float* lse,
                        void* workspace, size_t ws_bytes, focus_stream_t stream,
                        bool force_copies = false) {
    const AttnShape s{B, Hq, Hkv, n, d, K, w, m};
    focus_status st = check_attn_shape(s, true);
    if (st != FOCUS_OK) return st;
    st = check_attn_buffers(q, k, v, s, out, out_dtype, lse, scale);
    if (st != FOCUS_OK) return st;
    if (part != AttnPart::kWindow) {   // the window pass reads no group data
        REQUIRE_PTR(group_ids, 4);
        REQUIRE_PTR(perm, 4);
        REQUIRE_PTR(group_offsets, 4);
    }
    // the window pass only uses the leading part of the workspace, which
    // is laid out the same for every m
    const size_t need = part == AttnPart::kWindow
                            ? focus::attn_window_workspace(B, Hq, Hkv, n, d, w)
                            : focus::attn_workspace(B, Hq, Hkv, n, d, w, K, m, force_copies);
    if (need > 0) {
        REQUIRE(workspace != nullptr, FOCUS_ERR_WORKSPACE, "workspace of %zu bytes required", need);
        REQUIRE(aligned(workspace, 16), FOCUS_ERR_WORKSPACE, "workspace must be 16-byte aligned");
        REQUIRE(ws_bytes >= need, FOCUS_ERR_WORKSPACE,
                "workspace too small: %zu bytes given, %zu required", ws_bytes, need);
        const size_t qbytes = (size_t)B * Hq * n * d * 2, kvbytes = (size_t)B * Hkv * n * d * 2;
        const size_t obytes = (size_t)B * Hq * n * d * (out_dtype == FOCUS_F32 ? 4 : 2);
        REQUIRE(!overlaps(workspace, need, q, qbytes) && !overlaps(workspace, need, k, kvbytes) &&
                    !overlaps(workspace, need, v, kvbytes) &&
                    !overlaps(workspace, need, out, obytes),
                FOCUS_ERR_INVALID_ARGUMENT, "workspace must not overlap q, k, v or out");
    }
    focus::AttnProblem p{q, k, v, group_ids, perm, group_offsets, B, Hq, Hkv, n, d, K, w, scale,
                         out, out_dtype == FOCUS_F32 ? 1 : 0, lse, need > 0 ? workspace : nullptr,
                         m, force_copies ? 1 : 0};
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (part == AttnPart::kAll || part == AttnPart::kWindow) {
        hipError_t e = focus::launch_attn_window(p, hs);
        if (e != hipSuccess) return device_status(e, "window attention launch");
    }
    if (part == AttnPart::kAll || part == AttnPart::kLongRangeMerge ||
        part == AttnPart::kLongRangePrepare) {
        hipError_t e = focus::launch_attn_long_range_prepare(p, hs);
        if (e != hipSuccess) return device_status(e, "long-range preparation launch");
    }
    if (part == AttnPart::kAll || part == AttnPart::kLongRangeMerge ||
        part == AttnPart::kLongRangeApply) {
        hipError_t e = focus::launch_attn_long_range_apply(p, hs);
        if (e != hipSuccess) return device_status(e, "long-range attention launch");
    }
    return ok();
}

// m >= 1: top-m ids (and margin); m == 0: the raw scores [B][n][K].
focus_status assign_entry(const float* hidden, const float* P, const float* C, const float* bias,
                          int B, int n, int d_model, int d_proj, int K, int m,
                          int32_t* group_ids, float* margin, float* scores, void* workspace,
                          size_t workspace_bytes, focus_stream_t stream) {
    REQUIRE(B >= 1 && n >= 1, FOCUS_ERR_INVALID_ARGUMENT, "B and n must be >= 1 (got B=%d n=%d)",
            B, n);
    REQUIRE(d_model >= 1 && d_proj >= 1, FOCUS_ERR_INVALID_ARGUMENT,
            "d_model and d_proj must be >= 1");
    REQUIRE(d_model % 4 == 0, FOCUS_ERR_UNSUPPORTED, "d_model must be a multiple of 4 (got %d)",
            d_model);
    REQUIRE(K >= 1 && K <= FOCUS_MAX_GROUPS, FOCUS_ERR_UNSUPPORTED, "K must be in [1, %d] (got %d)",
            FOCUS_MAX_GROUPS, K);
    if (m != 0) {
        REQUIRE(m >= 1 && m <= FOCUS_MAX_MEMBERSHIPS, FOCUS_ERR_UNSUPPORTED,
                "m must be in [1, %d] (got %d)", FOCUS_MAX_MEMBERSHIPS, m);
        REQUIRE(m <= K, FOCUS_ERR_INVALID_ARGUMENT, "m (%d) must be <= K (%d)", m, K);
    }
    REQUIRE_PTR(hidden, 16);
    REQUIRE_PTR(P, 4);
    REQUIRE_PTR(C, 4);
    if (bias) REQUIRE(aligned(bias, 4), FOCUS_ERR_INVALID_ARGUMENT, "bias must be 4-byte aligned");
    if (m != 0) {
        REQUIRE_PTR(group_ids, 4);
        if (margin)
            REQUIRE(aligned(margin, 4), FOCUS_ERR_INVALID_ARGUMENT, "margin must be 4-byte aligned");
    } else {
        REQUIRE_PTR(scores, 4);
    }
    const int64_t ntok = (int64_t)B * n;
    REQUIRE((ntok + 31) / 32 <= kMaxGrid, FOCUS_ERR_UNSUPPORTED, "too many tokens for one launch");
    const size_t need = focus::assign_workspace(d_model, K);
    REQUIRE(workspace != nullptr, FOCUS_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    REQUIRE(aligned(workspace, 16), FOCUS_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    REQUIRE(workspace_bytes >= need, FOCUS_ERR_WORKSPACE,
            "workspace too small: %zu bytes given, %zu required", workspace_bytes, need);
    const size_t hbytes = (size_t)ntok * d_model * 4;
    if (m != 0)
        REQUIRE(!overlaps(group_ids, (size_t)ntok * m * 4, hidden, hbytes),
                FOCUS_ERR_INVALID_ARGUMENT, "group_ids must not overlap hidden");
    else
        REQUIRE(!overlaps(scores, (size_t)ntok * K * 4, hidden, hbytes),
                FOCUS_ERR_INVALID_ARGUMENT, "scores must not overlap hidden");
    return device_status(focus::launch_assign(hidden, P, C, bias, B, n, d_model, d_proj, K, m,
                                              group_ids, margin, scores, workspace,
                                              static_cast<hipStream_t>(stream)),
                         "assign launch");
}

}  // namespace

extern "C" {

int focus_abi_version(void) { return FOCUS_ABI_VERSION; }

const char* focus_last_error(void) { return g_err; }

size_t focus_assign_workspace_bytes(int d_model, int K) {
    if (d_model < 1 || K < 1 || K > FOCUS_MAX_GROUPS) return 0;
    return focus::assign_workspace(d_model, K);
}

focus_status focus_assign(const float* hidden, const float* P, const float* C, const float* bias,
                          int B, int n, int d_model, int d_proj, int K, int32_t* group_ids,
                          float* margin, void* workspace, size_t workspace_bytes,
                          focus_stream_t stream) {
    return assign_entry(hidden, P, C, bias, B, n, d_model, d_proj, K, 1, group_ids, margin,
                        nullptr, workspace, workspace_bytes, stream);
}

focus_status focus_assign_topk(const float* hidden, const float* P, const float* C,
                               const float* bias, int B, int n, int d_model, int d_proj, int K,
                               int m, int32_t* group_ids, float* margin, void* workspace,
                               size_t workspace_bytes, focus_stream_t stream) {
    if (m == 0) return fail(FOCUS_ERR_UNSUPPORTED, "m must be in [1, %d] (got 0)",
                            FOCUS_MAX_MEMBERSHIPS);
    return assign_entry(hidden, P, C, bias, B, n, d_model, d_proj, K, m, group_ids, margin,
                        nullptr, workspace, workspace_bytes, stream);
}

focus_status focus_assign_scores(const float* hidden, const float* P, const float* C,
                                 const float* bias, int B, int n, int d_model, int d_proj, int K,
                                 float* scores, void* workspace, size_t workspace_bytes,
                                 focus_stream_t stream) {
    return assign_entry(hidden, P, C, bias, B, n, d_model, d_proj, K, 0, nullptr, nullptr,
                        scores, workspace, workspace_bytes, stream);
}

size_t focus_sinkhorn_workspace_bytes(int B, int n, int K, int iters) {
    if (B < 1 || n < 1 || K < 1 || K > FOCUS_MAX_GROUPS || iters < 0) return 0;
    return focus::sinkhorn_layout(B, n, K, iters).total;
}

focus_status focus_sinkhorn(const float* scores, int B, int n, int K, float tau, int iters,
                            float* G, void* workspace, size_t workspace_bytes,
                            focus_stream_t stream) {
    REQUIRE(B >= 1 && n >= 1, FOCUS_ERR_INVALID_ARGUMENT, "B and n must be >= 1 (got B=%d n=%d)",
            B, n);
    REQUIRE(B <= 65535, FOCUS_ERR_UNSUPPORTED, "B must be <= 65535 (got %d)", B);
    REQUIRE(K >= 1 && K <= FOCUS_MAX_GROUPS, FOCUS_ERR_UNSUPPORTED, "K must be in [1, %d] (got %d)",
            FOCUS_MAX_GROUPS, K);
    REQUIRE(iters >= 0 && iters <= FOCUS_MAX_SINKHORN_ITERS, FOCUS_ERR_INVALID_ARGUMENT,
            "iters must be in [0, %d] (got %d)", FOCUS_MAX_SINKHORN_ITERS, iters);
    REQUIRE(std::isfinite(tau) && tau > 0.0f, FOCUS_ERR_INVALID_ARGUMENT,
            "tau must be finite and > 0");
    REQUIRE((int64_t)B * iters <= kMaxGrid && (int64_t)n * K <= ((int64_t)1 << 40),
            FOCUS_ERR_UNSUPPORTED, "problem too large");
    REQUIRE_PTR(scores, 4);
    REQUIRE_PTR(G, 4);
    const size_t bytes = (size_t)B * n * K * 4;
    REQUIRE(!overlaps(scores, bytes, G, bytes), FOCUS_ERR_INVALID_ARGUMENT,
            "G must not overlap scores");
    const size_t need = focus::sinkhorn_layout(B, n, K, iters).total;
    REQUIRE(workspace != nullptr, FOCUS_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    REQUIRE(aligned(workspace, 16), FOCUS_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    REQUIRE(workspace_bytes >= need, FOCUS_ERR_WORKSPACE,
            "workspace too small: %zu bytes given, %zu required", workspace_bytes, need);
    REQUIRE(!overlaps(workspace, need, scores, bytes) && !overlaps(workspace, need, G, bytes),
            FOCUS_ERR_INVALID_ARGUMENT, "workspace must not overlap scores or G");
    return device_status(focus::launch_sinkhorn(scores, B, n, K, tau, iters, G, workspace,
                                                static_cast<hipStream_t>(stream)),
                         "sinkhorn launch");
}

size_t focus_group_sort_workspace_bytes(int B, int n, int K) {
    if (B < 1 || n < 1 || K < 1 || K > FOCUS_MAX_GROUPS) return 0;
    return focus::group_sort_workspace(B, n, K);
}

focus_status focus_group_sort(const int32_t* group_ids, int B, int n, int K, int32_t* perm,
                              int32_t* group_offsets, void* workspace, size_t workspace_bytes,
                              focus_stream_t stream) {
    REQUIRE(B >= 1 && n >= 1, FOCUS_ERR_INVALID_ARGUMENT, "B and n must be >= 1 (got B=%d n=%d)",
            B, n);
    REQUIRE(K >= 1 && K <= FOCUS_MAX_GROUPS, FOCUS_ERR_UNSUPPORTED, "K must be in [1, %d] (got %d)",
            FOCUS_MAX_GROUPS, K);
    REQUIRE(B <= 65535, FOCUS_ERR_UNSUPPORTED, "B must be <= 65535 (got %d)", B);
    REQUIRE_PTR(group_ids, 4);
    REQUIRE_PTR(perm, 4);
    REQUIRE_PTR(group_offsets, 4);
    const size_t nb = (size_t)B * n * 4;
    REQUIRE(!overlaps(perm, nb, group_ids, nb) &&
                !overlaps(group_offsets, (size_t)B * (K + 1) * 4, group_ids, nb) &&
                !overlaps(group_offsets, (size_t)B * (K + 1) * 4, perm, nb),
            FOCUS_ERR_INVALID_ARGUMENT, "group_ids, perm and group_offsets must not overlap");
    const size_t need = focus::group_sort_workspace(B, n, K);
    REQUIRE(workspace != nullptr, FOCUS_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    REQUIRE(aligned(workspace, 4), FOCUS_ERR_WORKSPACE, "workspace must be 4-byte aligned");
    REQUIRE(workspace_bytes >= need, FOCUS_ERR_WORKSPACE,
            "workspace too small: %zu bytes given, %zu required", workspace_bytes, need);
    return device_status(focus::launch_group_sort(group_ids, B, n, K, perm, group_offsets,
                                                  workspace, static_cast<hipStream_t>(stream)),
                         "group sort launch");
}

static_assert(focus::kSortScratchBytes == FOCUS_SORT_NOALLOC_SCRATCH_BYTES,
              "the header states the size of the sort's static scratch");

focus_status focus_group_sort_noalloc(const int32_t* group_ids, int B, int n, int K,
                                      int32_t* perm, int32_t* group_offsets,
                                      focus_stream_t stream) {
    REQUIRE(B >= 1 && n >= 1, FOCUS_ERR_INVALID_ARGUMENT, "B and n must be >= 1 (got B=%d n=%d)",
            B, n);
    REQUIRE(K >= 1 && K <= FOCUS_MAX_GROUPS, FOCUS_ERR_UNSUPPORTED, "K must be in [1, %d] (got %d)",
            FOCUS_MAX_GROUPS, K);
    REQUIRE(B <= 65535, FOCUS_ERR_UNSUPPORTED, "B must be <= 65535 (got %d)", B);
    REQUIRE_PTR(group_ids, 4);
    REQUIRE_PTR(perm, 4);
    REQUIRE_PTR(group_offsets, 4);
    const size_t nb = (size_t)B * n * 4;
    REQUIRE(!overlaps(perm, nb, group_ids, nb) &&
                !overlaps(group_offsets, (size_t)B * (K + 1) * 4, group_ids, nb) &&
                !overlaps(group_offsets, (size_t)B * (K + 1) * 4, perm, nb),
            FOCUS_ERR_INVALID_ARGUMENT, "group_ids, perm and group_offsets must not overlap");
    const size_t need = focus::group_sort_workspace(B, n, K);
    REQUIRE(need <= focus::kSortScratchBytes, FOCUS_ERR_UNSUPPORTED,
            "the sort needs %zu bytes of scratch and the library's static scratch holds %zu "
            "(B * ceil(n / 2048) * K * 4 bytes); call focus_group_sort with a workspace",
            need, focus::kSortScratchBytes);
    int32_t* scratch = nullptr;
    const hipError_t e = focus::group_sort_scratch(&scratch);
    if (e != hipSuccess) return device_status(e, "sort scratch address");
    return device_status(focus::launch_group_sort(group_ids, B, n, K, perm, group_offsets,
                                                  scratch, static_cast<hipStream_t>(stream)),
                         "group sort launch");
}

size_t focus_attn_workspace_bytes(int B, int Hq, int Hkv, int n, int d_head, int K, int window) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || n < 1 || window < 0) return 0;
    if (d_head != 32 && d_head != 64 && d_head != 128) return 0;
    return focus::attn_workspace(B, Hq, Hkv, n, d_head, window, K);
}

focus_status focus_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* group_ids, const int32_t* perm,
                            const int32_t* group_offsets, int B, int Hq, int Hkv, int n,
                            int d_head, int K, int window, float scale, void* out,
                            focus_dtype out_dtype, float* lse, void* workspace,
                            size_t workspace_bytes, focus_stream_t stream) {
    return attn_entry(AttnPart::kAll, q, k, v, group_ids, perm, group_offsets, B, Hq, Hkv, n,
                      d_head, K, 1, window, scale, out, out_dtype, lse, workspace, workspace_bytes,
                      stream);
}

size_t focus_attn_sorted_kv_workspace_bytes(int B, int Hq, int Hkv, int n, int d_head, int K,
                                            int window) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || n < 1 || window < 0) return 0;
    if (d_head != 32 && d_head != 64 && d_head != 128) return 0;
    return focus::attn_workspace(B, Hq, Hkv, n, d_head, window, K, 1, true);
}

focus_status focus_attn_fwd_sorted_kv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                      const int32_t* group_ids, const int32_t* perm,
                                      const int32_t* group_offsets, int B, int Hq, int Hkv, int n,
                                      int d_head, int K, int window, float scale, void* out,
                                      focus_dtype out_dtype, float* lse, void* workspace,
                                      size_t workspace_bytes, focus_stream_t stream) {
    return attn_entry(AttnPart::kAll, q, k, v, group_ids, perm, group_offsets, B, Hq, Hkv, n,
                      d_head, K, 1, window, scale, out, out_dtype, lse, workspace, workspace_bytes,
                      stream, true);
}

focus_status focus_attn_window(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const int32_t* group_ids, const int32_t* perm,
                               const int32_t* group_offsets, int B, int Hq, int Hkv, int n,
                               int d_head, int K, int window, float scale, void* out,
                               focus_dtype out_dtype, float* lse, void* workspace,
                               size_t workspace_bytes, focus_stream_t stream) {
    return attn_entry(AttnPart::kWindow, q, k, v, group_ids, perm, group_offsets, B, Hq, Hkv, n,
                      d_head, K, 1, window, scale, out, out_dtype, lse, workspace, workspace_bytes,
                      stream);
}

focus_status focus_attn_long_range_merge(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                         const int32_t* group_ids, const int32_t* perm,
                                         const int32_t* group_offsets, int B, int Hq, int Hkv,
                                         int n, int d_head, int K, int window, float scale,
                                         void* out, focus_dtype out_dtype, float* lse,
                                         void* workspace, size_t workspace_bytes,
                                         focus_stream_t stream) {
    return attn_entry(AttnPart::kLongRangeMerge, q, k, v, group_ids, perm, group_offsets, B, Hq,
                      Hkv, n, d_head, K, 1, window, scale, out, out_dtype, lse, workspace,
                      workspace_bytes, stream);
}

focus_status focus_attn_long_range_prepare(const uint16_t* q, const uint16_t* k,
                                           const uint16_t* v, const int32_t* group_ids,
                                           const int32_t* perm, const int32_t* group_offsets,
                                           int B, int Hq, int Hkv, int n, int d_head, int K,
                                           int window, float scale, void* out,
                                           focus_dtype out_dtype, float* lse, void* workspace,
                                           size_t workspace_bytes, focus_stream_t stream) {
    return attn_entry(AttnPart::kLongRangePrepare, q, k, v, group_ids, perm, group_offsets, B,
                      Hq, Hkv, n, d_head, K, 1, window, scale, out, out_dtype, lse, workspace,
                      workspace_bytes, stream);
}

focus_status focus_attn_long_range_apply(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                         const int32_t* group_ids, const int32_t* perm,
                                         const int32_t* group_offsets, int B, int Hq, int Hkv,
                                         int n, int d_head, int K, int window, float scale,
                                         void* out, focus_dtype out_dtype, float* lse,
                                         void* workspace, size_t workspace_bytes,
                                         focus_stream_t stream) {
    return attn_entry(AttnPart::kLongRangeApply, q, k, v, group_ids, perm, group_offsets, B, Hq,
                      Hkv, n, d_head, K, 1, window, scale, out, out_dtype, lse, workspace,
                      workspace_bytes, stream);
}

size_t focus_soft_gate_attn_workspace_bytes(int B, int n, int K) {
    if (B < 1 || n < 1 || K < 1 || K > FOCUS_MAX_GROUPS) return 0;
    return focus::soft_gate_workspace(B, n, K);
}

focus_status focus_soft_gate_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                      const float* G, int B, int Hq, int Hkv, int n, int d_head,
                                      int K, int window, float scale, float lambda, void* out,
                                      focus_dtype out_dtype, float* lse, void* workspace,
                                      size_t workspace_bytes, focus_stream_t stream) {
    const AttnShape s{B, Hq, Hkv, n, d_head, K, window};
    focus_status st = check_attn_shape(s, true);
    if (st != FOCUS_OK) return st;
    st = check_attn_buffers(q, k, v, s, out, out_dtype, lse, scale);
    if (st != FOCUS_OK) return st;
    REQUIRE(std::isfinite(lambda), FOCUS_ERR_INVALID_ARGUMENT, "lambda must be finite");
    REQUIRE_PTR(G, 4);
    const size_t gbytes = (size_t)B * n * K * 4;
    const size_t obytes = (size_t)B * Hq * n * d_head * (out_dtype == FOCUS_F32 ? 4 : 2);
    REQUIRE(!overlaps(out, obytes, G, gbytes), FOCUS_ERR_INVALID_ARGUMENT,
            "out must not overlap G");
    const size_t need = focus::soft_gate_workspace(B, n, K);
    REQUIRE(workspace != nullptr, FOCUS_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    REQUIRE(aligned(workspace, 16), FOCUS_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    REQUIRE(workspace_bytes >= need, FOCUS_ERR_WORKSPACE,
            "workspace too small: %zu bytes given, %zu required", workspace_bytes, need);
    REQUIRE(!overlaps(workspace, need, G, gbytes) && !overlaps(workspace, need, out, obytes),
            FOCUS_ERR_INVALID_ARGUMENT, "workspace must not overlap G or out");
    focus::AttnProblem p{q, k, v, nullptr, nullptr, nullptr, B, Hq, Hkv, n, d_head, K, window,
                         scale, out, out_dtype == FOCUS_F32 ? 1 : 0, lse, workspace};
    return device_status(focus::launch_attn_soft_gate(p, G, lambda,
                                                      static_cast<hipStream_t>(stream)),
                         "soft-gated attention launch");
}

size_t focus_attn_topk_workspace_bytes(int B, int Hq, int Hkv, int n, int d_head, int K, int m,
                                       int window) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || n < 1 || window < 0) return 0;
    if (d_head != 32 && d_head != 64 && d_head != 128) return 0;
    if (K < 1 || K > FOCUS_MAX_GROUPS) return 0;
    if (m < 1 || m > FOCUS_MAX_MEMBERSHIPS || (int64_t)n * m > ((int64_t)1 << 24)) return 0;
    return focus::attn_workspace(B, Hq, Hkv, n, d_head, window, K, m);
}

focus_status focus_attn_topk_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const int32_t* group_ids, const int32_t* perm,
                                 const int32_t* group_offsets, int B, int Hq, int Hkv, int n,
                                 int d_head, int K, int m, int window, float scale, void* out,
                                 focus_dtype out_dtype, float* lse, void* workspace,
                                 size_t workspace_bytes, focus_stream_t stream) {
    return attn_entry(AttnPart::kAll, q, k, v, group_ids, perm, group_offsets, B, Hq, Hkv, n,
                      d_head, K, m, window, scale, out, out_dtype, lse, workspace,
                      workspace_bytes, stream);
}

focus_status focus_attn_topk_long_range_merge(const uint16_t* q, const uint16_t* k,
                                              const uint16_t* v, const int32_t* group_ids,
                                              const int32_t* perm, const int32_t* group_offsets,
                                              int B, int Hq, int Hkv, int n, int d_head, int K,
                                              int m, int window, float scale, void* out,
                                              focus_dtype out_dtype, float* lse,
                                              void* workspace, size_t workspace_bytes,
                                              focus_stream_t stream) {
    return attn_entry(AttnPart::kLongRangeMerge, q, k, v, group_ids, perm, group_offsets, B, Hq,
                      Hkv, n, d_head, K, m, window, scale, out, out_dtype, lse, workspace,
                      workspace_bytes, stream);
}

focus_status focus_attn_topk_long_range_prepare(const uint16_t* q, const uint16_t* k,
                                                const uint16_t* v, const int32_t* group_ids,
                                                const int32_t* perm,
                                                const int32_t* group_offsets, int B, int Hq,
                                                int Hkv, int n, int d_head, int K, int m,
                                                int window, float scale, void* out,
                                                focus_dtype out_dtype, float* lse,
                                                void* workspace, size_t workspace_bytes,
                                                focus_stream_t stream) {
    return attn_entry(AttnPart::kLongRangePrepare, q, k, v, group_ids, perm, group_offsets, B,
                      Hq, Hkv, n, d_head, K, m, window, scale, out, out_dtype, lse, workspace,
                      workspace_bytes, stream);
}

focus_status focus_attn_topk_long_range_apply(const uint16_t* q, const uint16_t* k,
                                              const uint16_t* v, const int32_t* group_ids,
                                              const int32_t* perm, const int32_t* group_offsets,
                                              int B, int Hq, int Hkv, int n, int d_head, int K,
                                              int m, int window, float scale, void* out,
                                              focus_dtype out_dtype, float* lse,
                                              void* workspace, size_t workspace_bytes,
                                              focus_stream_t stream) {
    return attn_entry(AttnPart::kLongRangeApply, q, k, v, group_ids, perm, group_offsets, B, Hq,
                      Hkv, n, d_head, K, m, window, scale, out, out_dtype, lse, workspace,
                      workspace_bytes, stream);
}

focus_status dense_causal_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   int B, int Hq, int Hkv, int n, int d_head, float scale,
                                   void* out, focus_dtype out_dtype, float* lse,
                                   focus_stream_t stream) {
    const AttnShape s{B, Hq, Hkv, n, d_head, 1, 0};
    focus_status st = check_attn_shape(s, false);
    if (st != FOCUS_OK) return st;
    st = check_attn_buffers(q, k, v, s, out, out_dtype, lse, scale);
    if (st != FOCUS_OK) return st;
    focus::AttnProblem p{q, k, v, nullptr, nullptr, nullptr, B, Hq, Hkv, n, d_head, 1, n,
                         scale, out, out_dtype == FOCUS_F32 ? 1 : 0, lse, nullptr};
    return device_status(focus::launch_attn_dense(p, static_cast<hipStream_t>(stream)),
                         "dense causal attention launch");
}

}  // extern "C"
