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

// Sub-buckets per head: (group, partner) with partner in [0, K].
inline __host__ __device__ int num_subbuckets(int K) { return K * (K + 1); }

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
