// Internal definitions shared by the HIP sources of libfocus.so.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/focus.h"

namespace focus {

constexpr int kWave = 64;
constexpr int kRouteDim = 16;
constexpr int kMaxGroups = 32;

// One 16-byte vector of eight bf16 values: the A/B operand of
// v_mfma_f32_32x32x16_bf16.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

// Sub-buckets: every group g is split by the token's lower set inside it,
// its groups below g.  The sub-bucket's key keeps the m lowest of them as a
// code, m = code_members(K, topk) (the whole lower set when top-k <= m + 1):
//     no group below g          -> 0
//     only a                    -> 1 + a
//     a < b                     -> 1 + g + C(b, 2) + a
//     a < b < c (m = 3)         -> 1 + g + C(g, 2) + C(c, 3) + C(b, 2) + a
// (with m = 2, a lower set of three or more keeps a < b; with m = 3, one of
// four or more keeps a < b < c).  Two tokens of g share a group below g
// exactly when their lower sets meet; when the kept members already meet,
// the pair belongs to a lower group.
//
// Three members cost C(g, 3) more codes per group; they are kept up to
// K = 16 (576 codes in the last group), so that the per-block code lists
// stay small in LDS.
constexpr int kThreeMemberMaxK = 16;
inline __host__ __device__ int code_members(int K, int topk)
{
    return topk <= 1 ? 0 : topk == 2 ? 1 : (topk >= 4 && K <= kThreeMemberMaxK) ? 3 : 2;
}
inline __host__ __device__ int choose2(int x) { return x * (x - 1) / 2; }
inline __host__ __device__ int choose3(int x) { return x * (x - 1) * (x - 2) / 6; }
inline __host__ __device__ int choose4(int x) { return x * (x - 1) * (x - 2) * (x - 3) / 24; }
// Codes a token of group g can take with m members kept: sum_{j <= m} C(g, j).
inline __host__ __device__ int codes_of_group(int g, int m)
{
    return 1 + (m >= 1 ? g : 0) + (m >= 2 ? choose2(g) : 0) + (m >= 3 ? choose3(g) : 0);
}
// First sub-bucket of group g: the codes of all groups below it,
// sum_{j <= m} C(g, j + 1).
inline __host__ __device__ int group_base(int g, int m)
{
    return g + (m >= 1 ? choose2(g) : 0) + (m >= 2 ? choose3(g) : 0) + (m >= 3 ? choose4(g) : 0);
}
// Sub-buckets per head.
inline __host__ __device__ int num_subbuckets(int K, int topk)
{
    return group_base(K, code_members(K, topk));
}
// Code of a lower set given by its kept members a < b < c (-1 when absent).
inline __host__ __device__ int lower_code(int g, int a, int b, int c)
{
    return a < 0 ? 0 : b < 0 ? 1 + a : c < 0 ? 1 + g + choose2(b) + a
                                              : 1 + g + choose2(g) + choose3(c) + choose2(b) + a;
}
// The kept members of the lower set with code `code` (-1 when absent).
struct LowerSet {
    int a, b, c;
};
inline __host__ __device__ LowerSet decode_lower(int g, int code)
{
    LowerSet r{-1, -1, -1};
    if (code == 0)
        return r;
    if (code <= g) {
        r.a = code - 1;
        return r;
    }
    int p = code - 1 - g;  // pairs (a, b), a < b, ordered by b then a
    if (p >= choose2(g)) {
        p -= choose2(g);  // triples, ordered by c, then b, then a
        int c = 2;
        while (choose3(c + 1) <= p)
            ++c;
        r.c = c;
        p -= choose3(c);
    }
    int b = 1;
    while (choose2(b + 1) <= p)
        ++b;
    r.b = b;
    r.a = p - choose2(b);
    return r;
}
// Whether two lower sets' kept members share a group.
// (Arguments by value, scalar tests: a reference or an array here may be
// turned into a per-thread LDS slot by the compiler.)
inline __host__ __device__ bool lower_set_has(int v, LowerSet s)
{
    return v >= 0 && (v == s.a || v == s.b || v == s.c);
}
inline __host__ __device__ bool lower_sets_meet(LowerSet x, LowerSet y)
{
    return lower_set_has(x.a, y) || lower_set_has(x.b, y) || lower_set_has(x.c, y);
}
// Whether a pair of sub-buckets whose kept members miss each other may still
// share a lower group: only when a side kept all m members and the top-k
// leaves room for more (a lower set holds up to top-k - 1 groups).
inline __host__ __device__ bool owner_test_needed(int topk, int m, LowerSet x, LowerSet y)
{
    if (topk < m + 2)
        return false;
    const bool xf = m == 3 ? x.c >= 0 : m == 2 ? x.b >= 0 : x.a >= 0;
    const bool yf = m == 3 ? y.c >= 0 : m == 2 ? y.b >= 0 : y.a >= 0;
    return xf || yf;
}
// Largest number of codes of one group, and of sub-buckets of a head, over
// every K <= 32 and top-k.
constexpr int kMaxCodes = 1 + 15 + 15 * 14 / 2 + 15 * 14 * 13 / 6;  // K = 16, m = 3
constexpr int kMaxSubbuckets = 32 + 32 * 31 / 2 + 32 * 31 * 30 / 6;  // K = 32, m = 2
static_assert(kMaxCodes >= 1 + 31 + 31 * 30 / 2, "m = 2 lists fit too");

// Host-side record of the last error on this thread (read by
// focus_last_error).
void set_error(const char *fmt, ...);

// Status for a failed HIP call, recording its text.
focus_status hip_failure(hipError_t e, const char *what);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- route.hip
hipError_t launch_route(const float *r, const float *centroids, int H, int64_t n, int K,
                        int topk, int32_t *groups, uint32_t *gmask, hipStream_t s);
hipError_t launch_route_project(const void *x, bool bf16, int64_t n, int dm, const float *Wt,
                                const float *centroids, int H, int K, int topk,
                                int32_t *groups, uint32_t *gmask, float *r_out, hipStream_t s);

// ---- bucket.hip
size_t bucket_workspace_bytes(int H, int64_t n, int K, int topk);
hipError_t launch_bucket(const int32_t *groups, int H, int64_t n, int K, int topk,
                         int32_t *offsets, int32_t *tokens, int32_t *slot_entry,
                         void *ws, hipStream_t s);
// device address and size of the current device's focus_bucket_noalloc scratch
hipError_t bucket_noalloc_scratch(void **ptr, size_t *bytes);

// ---- check.hip: consistency of a bucketing with its routing (synchronous:
// waits for the stream, then stores the failed-check bits in *found)
hipError_t launch_check_buckets(const uint32_t *gmask, const int32_t *offsets,
                                const int32_t *tokens, const int32_t *slot_entry, int H,
                                int64_t n, int K, int topk, void *ws, hipStream_t s,
                                uint32_t *found);

// ---- attn.hip
struct AttnShape {
    focus_dtype dt;
    int hq, hkv, d, K, topk;
    int64_t n, window;
    float scale;
};
size_t attn_workspace_bytes(const AttnShape &sh);
size_t dense_workspace_bytes(const AttnShape &sh);
hipError_t launch_attn(const AttnShape &sh, const void *q, const void *k, const void *v,
                       const uint32_t *gmask, const int32_t *offsets, const int32_t *tokens,
                       const int32_t *slot_entry, void *out, float *lse, void *ws,
                       int parts, hipStream_t s);
hipError_t launch_dense(const AttnShape &sh, const void *q, const void *k, const void *v,
                        void *out, float *lse, void *ws, hipStream_t s);
size_t gated_dense_workspace_bytes(const AttnShape &sh);
hipError_t launch_gated_dense(const AttnShape &sh, const void *q, const void *k, const void *v,
                              const float *assign, float lambda, void *out, float *lse, void *ws,
                              hipStream_t s);

// ---- attn_train.hip
size_t sinkhorn_workspace_bytes(int H, int64_t n);
hipError_t launch_sinkhorn(const float *r, const float *centroids, int H, int64_t n, int K,
                           int iters, float *A, void *ws, hipStream_t s);

// ---- attn_bwd.hip
size_t attn_bwd_workspace_bytes(const AttnShape &sh);
hipError_t launch_attn_bwd(const AttnShape &sh, const void *q, const void *k, const void *v,
                           const void *out, const float *lse, const void *dout,
                           const uint32_t *gmask, const int32_t *offsets, const int32_t *tokens,
                           const int32_t *slot_entry, void *dq, void *dk, void *dv, void *ws,
                           hipStream_t s);

}  // namespace focus
