// extern "C" entry points of libfocus.so (declared in include/focus.h):
// argument validation, workspace checks and error reporting around the
// kernel launchers.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include <algorithm>

#include "common.hpp"

namespace focus {

namespace {
thread_local char g_last_error[512] = "";

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

focus_status invalid(const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return FOCUS_ERR_INVALID_ARGUMENT;
}

focus_status unsupported(const char *what)
{
    snprintf(g_last_error, sizeof g_last_error, "unsupported: %s", what);
    return FOCUS_ERR_UNSUPPORTED;
}

focus_status short_workspace(size_t have, size_t need)
{
    snprintf(g_last_error, sizeof g_last_error, "workspace of %zu bytes, %zu required", have,
             need);
    return FOCUS_ERR_WORKSPACE;
}

#define FOCUS_REQUIRE(cond, ...)                                                               \
    do {                                                                                       \
        if (!(cond))                                                                           \
            return invalid(__VA_ARGS__);                                                       \
    } while (0)

#define FOCUS_PTR(p)                                                                           \
    do {                                                                                       \
        if ((p) == nullptr || !aligned16(p))                                                   \
            return invalid("pointer %s is null or not 16-byte aligned", #p);                  \
    } while (0)

focus_status check_attn(const void *q, const void *k, const void *v, focus_dtype dt, int32_t Hq,
                        int32_t Hkv, int64_t n, int32_t d)
{
    FOCUS_PTR(q);
    FOCUS_PTR(k);
    FOCUS_PTR(v);
    FOCUS_REQUIRE(dt == FOCUS_F32 || dt == FOCUS_BF16, "dtype %d", (int)dt);
    FOCUS_REQUIRE(Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, "heads Hq=%d Hkv=%d", Hq, Hkv);
    FOCUS_REQUIRE(n >= 1 && n <= INT32_MAX / 2, "n=%lld", (long long)n);
    if (d != 64 && d != 128)
        return unsupported("head dim must be 64 or 128");
    return FOCUS_OK;
}

// With 2 top-k > K any two tokens' group sets intersect (pigeonhole), so
// A(i) is every j <= i and the layer is causal attention.  The window pass
// then takes every pair (window = n) and the group pass finds none: the same
// set, evaluated once, without the group pass visiting pairs in several
// buckets to mask all but the lowest.
int64_t all_pairs_window(int32_t K, int32_t topk, int64_t n, int64_t window)
{
    return 2 * (int64_t)topk > K ? std::max(window, n) : window;
}

// FOCUS_DEBUG=1 in the environment (read at every call, so a process can
// switch it on and off) makes the entry points that index rows through a
// bucketing check it first.
bool debug_checks()
{
    const char *v = std::getenv("FOCUS_DEBUG");
    return v != nullptr && v[0] == '1' && v[1] == '\0';
}

// Runs the bucketing check on the stream (synchronously) with the first bytes
// of `ws` as its flag word; INVALID_ARGUMENT names the failed checks.
focus_status check_buckets(const uint32_t *gmask, const int32_t *offsets, const int32_t *tokens,
                           const int32_t *slot_entry, int32_t H, int64_t n, int32_t K,
                           int32_t topk, void *ws, hipStream_t stream)
{
    uint32_t found = 0u;
    hipError_t e = launch_check_buckets(gmask, offsets, tokens, slot_entry, H, n, K, topk, ws,
                                        stream, &found);
    if (e != hipSuccess)
        return hip_failure(e, "bucket check");
    if (found == 0u)
        return FOCUS_OK;
    return invalid("buckets inconsistent with the routing:%s%s%s%s",
                   (found & 1u) ? " offsets" : "", (found & 2u) ? " tokens" : "",
                   (found & 4u) ? " groups/lower-set codes/gmask" : "",
                   (found & 8u) ? " slot_entry" : "");
}

}  // namespace

void set_error(const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
}

focus_status hip_failure(hipError_t e, const char *what)
{
    set_error("%s: %s", what, hipGetErrorString(e));
    return FOCUS_ERR_HIP;
}

}  // namespace focus

using namespace focus;

extern "C" {

const char *focus_status_string(focus_status s)
{
    switch (s) {
    case FOCUS_OK:
        return "FOCUS_OK";
    case FOCUS_ERR_INVALID_ARGUMENT:
        return "FOCUS_ERR_INVALID_ARGUMENT";
    case FOCUS_ERR_UNSUPPORTED:
        return "FOCUS_ERR_UNSUPPORTED";
    case FOCUS_ERR_WORKSPACE:
        return "FOCUS_ERR_WORKSPACE";
    case FOCUS_ERR_HIP:
        return "FOCUS_ERR_HIP";
    }
    return "FOCUS_ERR_UNKNOWN";
}

const char *focus_last_error(void) { return g_last_error; }

int32_t focus_abi_version(void) { return 1; }

focus_status focus_route(const float *r, const float *centroids, int32_t H, int64_t n,
                         int32_t d_g, int32_t K, int32_t topk, int32_t *groups,
                         uint32_t *gmask, focus_stream stream)
{
    g_last_error[0] = 0;
    FOCUS_PTR(r);
    FOCUS_PTR(centroids);
    FOCUS_PTR(groups);
    FOCUS_PTR(gmask);
    FOCUS_REQUIRE(H >= 1 && n >= 1 && K >= 1, "H=%d n=%lld K=%d", H, (long long)n, K);
    FOCUS_REQUIRE(n <= INT32_MAX, "n=%lld", (long long)n);
    if (d_g != kRouteDim)
        return unsupported("routing dimension must be 16");
    if (K > kMaxGroups)
        return unsupported("at most 32 centroids");
    FOCUS_REQUIRE(topk >= 1 && topk <= K, "topk=%d K=%d", topk, K);
    hipError_t e = launch_route(r, centroids, H, n, K, topk, groups, gmask,
                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FOCUS_OK : hip_failure(e, "focus_route launch");
}

focus_status focus_route_project(const void *x, focus_dtype xdt, int64_t n, int32_t d_model,
                                 const float *Wt, const float *centroids, int32_t H,
                                 int32_t d_g, int32_t K, int32_t topk, int32_t *groups,
                                 uint32_t *gmask, float *r, focus_stream stream)
{
    g_last_error[0] = 0;
    FOCUS_PTR(x);
    FOCUS_PTR(Wt);
    FOCUS_PTR(centroids);
    FOCUS_PTR(groups);
    FOCUS_PTR(gmask);
    if (r != nullptr && !aligned16(r))
        return invalid("pointer r is not 16-byte aligned");
    FOCUS_REQUIRE(xdt == FOCUS_F32 || xdt == FOCUS_BF16, "dtype %d", (int)xdt);
    FOCUS_REQUIRE(H >= 1 && n >= 1 && K >= 1, "H=%d n=%lld K=%d", H, (long long)n, K);
    FOCUS_REQUIRE(n <= INT32_MAX, "n=%lld", (long long)n);
    FOCUS_REQUIRE(d_model >= 1, "d_model=%d", d_model);
    if (d_g != kRouteDim)
        return unsupported("routing dimension must be 16");
    if (K > kMaxGroups)
        return unsupported("at most 32 centroids");
    FOCUS_REQUIRE(topk >= 1 && topk <= K, "topk=%d K=%d", topk, K);
    hipError_t e = launch_route_project(x, xdt == FOCUS_BF16, n, d_model, Wt, centroids, H, K,
                                        topk, groups, gmask, r,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FOCUS_OK : hip_failure(e, "focus_route_project launch");
}

int32_t focus_num_subbuckets(int32_t K, int32_t topk)
{
    if (K < 1 || K > kMaxGroups || topk < 1 || topk > K)
        return 0;
    return num_subbuckets(K, topk);
}

size_t focus_bucket_workspace_bytes(int32_t H, int64_t n, int32_t K, int32_t topk)
{
    if (H < 1 || n < 1 || K < 1 || K > kMaxGroups || topk < 1 || topk > K)
        return 0;
    return bucket_workspace_bytes(H, n, K, topk);
}

focus_status focus_bucket(const int32_t *groups, int32_t H, int64_t n, int32_t K, int32_t topk,
                          int32_t *offsets, int32_t *tokens, int32_t *slot_entry,
                          void *workspace, size_t workspace_bytes, focus_stream stream)
{
    g_last_error[0] = 0;
    FOCUS_PTR(groups);
    FOCUS_PTR(offsets);
    FOCUS_PTR(tokens);
    FOCUS_PTR(slot_entry);
    FOCUS_REQUIRE(H >= 1 && n >= 1 && K >= 1, "H=%d n=%lld K=%d", H, (long long)n, K);
    if (K > kMaxGroups)
        return unsupported("at most 32 centroids");
    FOCUS_REQUIRE(topk >= 1 && topk <= K, "topk=%d K=%d", topk, K);
    FOCUS_REQUIRE(n * (int64_t)topk <= INT32_MAX, "n*topk exceeds int32");
    const size_t need = bucket_workspace_bytes(H, n, K, topk);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
        return short_workspace(workspace_bytes, need);
    hipError_t e = launch_bucket(groups, H, n, K, topk, offsets, tokens, slot_entry, workspace,
                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FOCUS_OK : hip_failure(e, "focus_bucket launch");
}

size_t focus_attn_workspace_bytes(focus_dtype dt, int32_t Hq, int32_t Hkv, int64_t n, int32_t d,
                                  int32_t K, int32_t topk)
{
    if (Hq < 1 || Hkv < 1 || Hq % Hkv || n < 1 || (d != 64 && d != 128) || K < 1 ||
        K > kMaxGroups || topk < 1 || topk > K || n * (int64_t)topk > INT32_MAX)
        return 0;
    AttnShape sh{dt, Hq, Hkv, d, K, topk, n, 0, 1.f};
    return attn_workspace_bytes(sh);
}

focus_status focus_bucket_noalloc(const int32_t *groups, int32_t H, int64_t n, int32_t K,
                                  int32_t topk, int32_t *offsets, int32_t *tokens,
                                  int32_t *slot_entry, focus_stream stream)
{
    g_last_error[0] = 0;
    FOCUS_PTR(groups);
    FOCUS_PTR(offsets);
    FOCUS_PTR(tokens);
    FOCUS_PTR(slot_entry);
    FOCUS_REQUIRE(H >= 1 && n >= 1 && K >= 1, "H=%d n=%lld K=%d", H, (long long)n, K);
    if (K > kMaxGroups)
        return unsupported("at most 32 centroids");
    FOCUS_REQUIRE(topk >= 1 && topk <= K, "topk=%d K=%d", topk, K);
    FOCUS_REQUIRE(n * (int64_t)topk <= INT32_MAX, "n*topk exceeds int32");
    const size_t need = bucket_workspace_bytes(H, n, K, topk);
    if (need > FOCUS_BUCKET_NOALLOC_SCRATCH_BYTES) {
        set_error("focus_bucket_noalloc: this shape needs %zu bytes of count scratch, more "
                  "than the library's fixed %zu (use focus_bucket with a workspace)",
                  need, (size_t)FOCUS_BUCKET_NOALLOC_SCRATCH_BYTES);
        return FOCUS_ERR_WORKSPACE;
    }
    void *ws = nullptr;
    size_t have = 0;
    hipError_t e = bucket_noalloc_scratch(&ws, &have);
    if (e != hipSuccess)
        return hip_failure(e, "focus_bucket_noalloc scratch address");
    if (have < need)
        return short_workspace(have, need);
    e = launch_bucket(groups, H, n, K, topk, offsets, tokens, slot_entry, ws,
                      static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FOCUS_OK : hip_failure(e, "focus_bucket_noalloc launch");
}

size_t focus_attn_fwd_workspace_bytes(focus_dtype dt, int32_t Hq, int32_t Hkv, int64_t n,
                                      int32_t d, int32_t K, int32_t topk)
{
    return focus_attn_workspace_bytes(dt, Hq, Hkv, n, d, K, topk);
}

focus_status focus_check_buckets(const uint32_t *gmask, const int32_t *offsets,
                                 const int32_t *tokens, const int32_t *slot_entry, int32_t H,
                                 int64_t n, int32_t K, int32_t topk, void *workspace,
                                 size_t workspace_bytes, focus_stream stream)
{
    g_last_error[0] = 0;
    FOCUS_PTR(gmask);
    FOCUS_PTR(offsets);
    FOCUS_PTR(tokens);
    FOCUS_PTR(slot_entry);
    FOCUS_REQUIRE(H >= 1 && n >= 1 && K >= 1, "H=%d n=%lld K=%d", H, (long long)n, K);
    if (K > kMaxGroups)
        return unsupported("at most 32 centroids");
    FOCUS_REQUIRE(topk >= 1 && topk <= K, "topk=%d K=%d", topk, K);
    FOCUS_REQUIRE(n * (int64_t)topk <= INT32_MAX, "n*topk exceeds int32");
    if (workspace == nullptr || workspace_bytes < FOCUS_CHECK_WORKSPACE_BYTES ||
        !aligned16(workspace))
        return short_workspace(workspace_bytes, FOCUS_CHECK_WORKSPACE_BYTES);
    return check_buckets(gmask, offsets, tokens, slot_entry, H, n, K, topk, workspace,
                         static_cast<hipStream_t>(stream));
}

focus_status focus_attn_fwd_part(const void *q, const void *k, const void *v, focus_dtype dt,
                                 int32_t Hq, int32_t Hkv, int64_t n, int32_t d,
                                 const uint32_t *gmask, const int32_t *offsets,
                                 const int32_t *tokens, const int32_t *slot_entry, int32_t K,
                                 int32_t topk, int64_t window, float scale, void *out, float *lse,
                                 void *workspace, size_t workspace_bytes, int32_t parts,
                                 focus_stream stream)
{
    g_last_error[0] = 0;
    focus_status st = check_attn(q, k, v, dt, Hq, Hkv, n, d);
    if (st != FOCUS_OK)
        return st;
    FOCUS_PTR(gmask);
    FOCUS_PTR(offsets);
    FOCUS_PTR(tokens);
    FOCUS_PTR(slot_entry);
    FOCUS_PTR(out);
    FOCUS_PTR(lse);
    FOCUS_REQUIRE(K >= 1, "K=%d", K);
    if (K > kMaxGroups)
        return unsupported("at most 32 centroids");
    FOCUS_REQUIRE(topk >= 1 && topk <= K, "topk=%d K=%d", topk, K);
    FOCUS_REQUIRE(window >= 0, "window=%lld", (long long)window);
    FOCUS_REQUIRE(n * (int64_t)topk <= INT32_MAX, "n*topk exceeds int32");
    FOCUS_REQUIRE(scale > 0.f && scale < 1e30f, "scale must be positive and finite");
    FOCUS_REQUIRE(parts >= 1 && parts <= FOCUS_PART_ALL, "parts=%d", parts);
    AttnShape sh{dt, Hq, Hkv, d, K, topk, n, all_pairs_window(K, topk, n, window), scale};
    const size_t need = attn_workspace_bytes(sh);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
        return short_workspace(workspace_bytes, need);
    // (the check's flag word sits in workspace bytes that PREPARE rewrites)
    if ((parts & FOCUS_PART_PREPARE) && debug_checks()) {
        st = check_buckets(gmask, offsets, tokens, slot_entry, Hkv, n, K, topk, workspace,
                           static_cast<hipStream_t>(stream));
        if (st != FOCUS_OK)
            return st;
    }
    hipError_t e = launch_attn(sh, q, k, v, gmask, offsets, tokens, slot_entry, out, lse,
                               workspace, parts, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FOCUS_OK : hip_failure(e, "focus_attn_fwd launch");
}

focus_status focus_attn_fwd(const void *q, const void *k, const void *v, focus_dtype dt,
                            int32_t Hq, int32_t Hkv, int64_t n, int32_t d, const uint32_t *gmask,
                            const int32_t *offsets, const int32_t *tokens,
                            const int32_t *slot_entry, int32_t K, int32_t topk, int64_t window,
                            float scale, void *out, float *lse, void *workspace,
                            size_t workspace_bytes, focus_stream stream)
{
    return focus_attn_fwd_part(q, k, v, dt, Hq, Hkv, n, d, gmask, offsets, tokens, slot_entry, K,
                               topk, window, scale, out, lse, workspace, workspace_bytes,
                               FOCUS_PART_ALL, stream);
}

size_t focus_attn_bwd_workspace_bytes(focus_dtype dt, int32_t Hq, int32_t Hkv, int64_t n,
                                      int32_t d, int32_t K, int32_t topk)
{
    if (dt != FOCUS_BF16 || Hq < 1 || Hkv < 1 || Hq % Hkv || n < 1 || n > INT32_MAX / 2 ||
        (d != 64 && d != 128) || K < 1 || K > kMaxGroups || topk < 1 || topk > K ||
        n * (int64_t)topk > INT32_MAX)
        return 0;
    AttnShape sh{dt, Hq, Hkv, d, K, topk, n, 0, 1.f};
    return attn_bwd_workspace_bytes(sh);
}

focus_status focus_attn_bwd(const void *q, const void *k, const void *v, const void *out,
                            const float *lse, const void *dout, focus_dtype dt, int32_t Hq,
                            int32_t Hkv, int64_t n, int32_t d, const uint32_t *gmask,
                            const int32_t *offsets, const int32_t *tokens,
                            const int32_t *slot_entry, int32_t K, int32_t topk, int64_t window,
                            float scale, void *dq, void *dk, void *dv, void *workspace,
                            size_t workspace_bytes, focus_stream stream)
{
    g_last_error[0] = 0;
    focus_status st = check_attn(q, k, v, dt, Hq, Hkv, n, d);
    if (st != FOCUS_OK)
        return st;
    if (dt != FOCUS_BF16)
        return unsupported("the backward takes bf16 inputs");
    FOCUS_PTR(out);
    FOCUS_PTR(lse);
    FOCUS_PTR(dout);
    FOCUS_PTR(gmask);
    FOCUS_PTR(offsets);
    FOCUS_PTR(tokens);
    FOCUS_PTR(slot_entry);
    FOCUS_PTR(dq);
    FOCUS_PTR(dk);
    FOCUS_PTR(dv);
    FOCUS_REQUIRE(K >= 1, "K=%d", K);
    if (K > kMaxGroups)
        return unsupported("at most 32 centroids");
    FOCUS_REQUIRE(topk >= 1 && topk <= K, "topk=%d K=%d", topk, K);
    FOCUS_REQUIRE(window >= 0, "window=%lld", (long long)window);
    FOCUS_REQUIRE(n * (int64_t)topk <= INT32_MAX, "n*topk exceeds int32");
    FOCUS_REQUIRE(scale > 0.f && scale < 1e30f, "scale must be positive and finite");
    AttnShape sh{dt, Hq, Hkv, d, K, topk, n, all_pairs_window(K, topk, n, window), scale};
    const size_t need = attn_bwd_workspace_bytes(sh);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
        return short_workspace(workspace_bytes, need);
    if (debug_checks()) {
        st = check_buckets(gmask, offsets, tokens, slot_entry, Hkv, n, K, topk, workspace,
                           static_cast<hipStream_t>(stream));
        if (st != FOCUS_OK)
            return st;
    }
    hipError_t e = launch_attn_bwd(sh, q, k, v, out, lse, dout, gmask, offsets, tokens,
                                   slot_entry, dq, dk, dv, workspace,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FOCUS_OK : hip_failure(e, "focus_attn_bwd launch");
}

size_t focus_sinkhorn_workspace_bytes(int32_t H, int64_t n)
{
    if (H < 1 || n < 1 || n > INT32_MAX)
        return 0;
    return sinkhorn_workspace_bytes(H, n);
}

focus_status focus_sinkhorn(const float *r, const float *centroids, int32_t H, int64_t n,
                            int32_t d_g, int32_t K, int32_t iters, float *assign,
                            void *workspace, size_t workspace_bytes, focus_stream stream)
{
    g_last_error[0] = 0;
    FOCUS_PTR(r);
    FOCUS_PTR(centroids);
    FOCUS_PTR(assign);
    FOCUS_REQUIRE(H >= 1 && n >= 1 && K >= 1, "H=%d n=%lld K=%d", H, (long long)n, K);
    FOCUS_REQUIRE(n <= INT32_MAX, "n=%lld", (long long)n);
    if (d_g != kRouteDim)
        return unsupported("routing dimension must be 16");
    if (K > kMaxGroups)
        return unsupported("at most 32 centroids");
    FOCUS_REQUIRE(iters >= 1 && iters <= 1000, "iters=%d", iters);
    const size_t need = sinkhorn_workspace_bytes(H, n);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
        return short_workspace(workspace_bytes, need);
    hipError_t e = launch_sinkhorn(r, centroids, H, n, K, iters, assign, workspace,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FOCUS_OK : hip_failure(e, "focus_sinkhorn launch");
}

size_t focus_gated_attn_workspace_bytes(int32_t Hkv, int64_t n, int32_t d, int32_t K)
{
    if (Hkv < 1 || n < 1 || n > INT32_MAX / 2 || (d != 64 && d != 128) || K < 1 ||
        K > kMaxGroups)
        return 0;
    AttnShape sh{FOCUS_BF16, Hkv, Hkv, d, K, 1, n, n, 1.f};
    return gated_dense_workspace_bytes(sh);
}

focus_status focus_gated_attn_fwd(const void *q, const void *k, const void *v, focus_dtype dt,
                                  int32_t Hq, int32_t Hkv, int64_t n, int32_t d,
                                  const float *assign, int32_t K, int64_t window, float lambda,
                                  float scale, void *out, float *lse, void *workspace,
                                  size_t workspace_bytes, focus_stream stream)
{
    g_last_error[0] = 0;
    focus_status st = check_attn(q, k, v, dt, Hq, Hkv, n, d);
    if (st != FOCUS_OK)
        return st;
    if (dt != FOCUS_BF16)
        return unsupported("the gated forward takes bf16 inputs");
    FOCUS_PTR(assign);
    FOCUS_PTR(out);
    FOCUS_PTR(lse);
    FOCUS_REQUIRE(K >= 1, "K=%d", K);
    if (K > kMaxGroups)
        return unsupported("at most 32 centroids");
    FOCUS_REQUIRE(window >= 0, "window=%lld", (long long)window);
    FOCUS_REQUIRE(scale > 0.f && scale < 1e30f, "scale must be positive and finite");
    FOCUS_REQUIRE(lambda == lambda && lambda > -1e30f && lambda < 1e30f,
                  "lambda must be finite");
    AttnShape sh{dt, Hq, Hkv, d, K, 1, n, window, scale};
    const size_t need = gated_dense_workspace_bytes(sh);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
        return short_workspace(workspace_bytes, need);
    hipError_t e = launch_gated_dense(sh, q, k, v, assign, lambda, out, lse, workspace,
                                      static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FOCUS_OK : hip_failure(e, "focus_gated_attn_fwd launch");
}

size_t focus_dense_workspace_bytes(focus_dtype dt, int32_t Hkv, int64_t n, int32_t d)
{
    if (Hkv < 1 || n < 1 || (d != 64 && d != 128))
        return 0;
    AttnShape sh{dt, Hkv, Hkv, d, 1, 1, n, n, 1.f};
    return dense_workspace_bytes(sh);
}

focus_status focus_dense_causal_fwd(const void *q, const void *k, const void *v, focus_dtype dt,
                                    int32_t Hq, int32_t Hkv, int64_t n, int32_t d, float scale,
                                    void *out, float *lse, void *workspace,
                                    size_t workspace_bytes, focus_stream stream)
{
    g_last_error[0] = 0;
    focus_status st = check_attn(q, k, v, dt, Hq, Hkv, n, d);
    if (st != FOCUS_OK)
        return st;
    FOCUS_PTR(out);
    FOCUS_PTR(lse);
    FOCUS_REQUIRE(scale > 0.f && scale < 1e30f, "scale must be positive and finite");
    AttnShape sh{dt, Hq, Hkv, d, 1, 1, n, n, scale};
    const size_t need = dense_workspace_bytes(sh);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
        return short_workspace(workspace_bytes, need);
    hipError_t e =
        launch_dense(sh, q, k, v, out, lse, workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FOCUS_OK : hip_failure(e, "focus_dense_causal_fwd launch");
}

}  // extern "C"
