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
// its groups below g.  The sub-bucket's key keeps the two lowest of them
// (the whole lower set at top-k <= 3) as a code:
//     no group below g  -> 0
//     only a            -> 1 + a
//     a < b (and more)  -> 1 + g + b (b - 1) / 2 + a
// Two tokens of g share a group below g exactly when their lower sets meet;
// when the two-lowest keys already meet, the pair belongs to a lower group.
// Codes a token of group g can take at this top-k.
inline __host__ __device__ int codes_of_group(int g, int topk)
{
    return topk == 1 ? 1 : topk == 2 ? 1 + g : 1 + g + g * (g - 1) / 2;
}
// First sub-bucket of group g: the codes of all groups below it.
inline __host__ __device__ int group_base(int g, int topk)
{
    const int pairs = g * (g - 1) / 2;  // sum of g' over g' < g
    if (topk == 1)
        return g;
    if (topk == 2)
        return g + pairs;
    return g + pairs + g * (g - 1) * (g - 2) / 6;
}
// Sub-buckets per head.
inline __host__ __device__ int num_subbuckets(int K, int topk) { return group_base(K, topk); }
// Most codes of one group (the last one).
inline __host__ __device__ int max_codes(int K, int topk) { return codes_of_group(K - 1, topk); }
// Code of a lower set given by its lowest member a and second-lowest b
// (-1 when absent).
inline __host__ __device__ int lower_code(int g, int a, int b)
{
    return a < 0 ? 0 : b < 0 ? 1 + a : 1 + g + b * (b - 1) / 2 + a;
}
// The two lowest members (a, b; -1 when absent) of the lower set with code c.
inline __host__ __device__ void decode_lower(int g, int c, int &a, int &b)
{
    a = -1;
    b = -1;
    if (c == 0)
        return;
    if (c <= g) {
        a = c - 1;
        return;
    }
    int p = c - 1 - g;  // index of the pair (a, b), a < b, ordered by b then a
    int bb = 1;
    while ((bb + 1) * bb / 2 <= p)
        ++bb;
    b = bb;
    a = p - bb * (bb - 1) / 2;
}
// Largest number of codes of one group, and of sub-buckets of a head, over
// every K <= 32 and top-k.
constexpr int kMaxCodes = 1 + 31 + 31 * 30 / 2;
constexpr int kMaxSubbuckets = 32 + 32 * 31 / 2 + 32 * 31 * 30 / 6;

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
