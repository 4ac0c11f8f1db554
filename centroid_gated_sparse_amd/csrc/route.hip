// Routing: centroid scores and top-k group membership.
//
// Technical Summary (gist.science), section 2: Token Grouping (the projected
// state is compared with each centroid) and Inference Efficiency (Top-k)
// (each token joins its k highest-scoring groups); jindou-blog method
// bullets: K centroids per layer, 16-dimensional routing, dot products.
//
// Layout: a token is served by Kp = next power of two >= K consecutive lanes
// of a wavefront, lane g scoring centroid g; 64 / Kp tokens per wavefront
// step.  The top-k is k rounds of a butterfly arg-max across the Kp lanes
// (order: larger score first, lower group index on equal scores; -0.0 and
// +0.0 are equal).  The routing vectors are read once per lane group and the
// work is bound by HBM: 64 B in and 4*(k+1) B out per token.
#include "common.hpp"

namespace focus {
namespace {

// Fixed-order fp32 score: products accumulated left to right, no fused
// multiply-add, so that any IEEE implementation reproduces it bit for bit.
__device__ __forceinline__ float score16(const float4 (&r)[4], const float (&c)[16])
{
#pragma clang fp contract(off)
    const float *rv = reinterpret_cast<const float *>(r);
    float s = rv[0] * c[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) {
        float p = rv[e] * c[e];
        s = s + p;
    }
    return s;
}

// True if candidate (sa, ga) ranks before (sb, gb).
__device__ __forceinline__ bool ranks_before(bool va, float sa, int ga, bool vb, float sb,
                                             int gb)
{
    if (va != vb)
        return va;
    if (sa > sb)
        return true;
    if (sa < sb)
        return false;
    return ga < gb;
}

__global__ __launch_bounds__(256) void route_kernel(const float *__restrict__ r,
                                                    const float *__restrict__ centroids,
                                                    int64_t n, int K, int kp_log2, int topk,
                                                    int32_t *__restrict__ groups,
                                                    uint32_t *__restrict__ gmask)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int Kp = 1 << kp_log2;
    const int g = lane & (Kp - 1);
    const int slot = lane >> kp_log2;
    const int tokens_per_step = kWave >> kp_log2;
    const int h = blockIdx.y;
    const bool g_valid = g < K;

    float c[16];
    {
        const float *cg = centroids + ((int64_t)h * K + (g_valid ? g : 0)) * kRouteDim;
#pragma unroll
        for (int e = 0; e < 16; ++e)
            c[e] = cg[e];
    }
    const float *rh = r + (int64_t)h * n * kRouteDim;
    int32_t *gh = groups + (int64_t)h * n * topk;
    uint32_t *mh = gmask + (int64_t)h * n;

    const int64_t waves_per_grid = (int64_t)gridDim.x * (blockDim.x / kWave);
    const int64_t wave_id = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    for (int64_t base = wave_id * tokens_per_step; base < n;
         base += waves_per_grid * tokens_per_step) {
        const int64_t t = base + slot;
        const bool t_valid = t < n;
        float s = 0.f;
        if (t_valid) {
            const float4 *rt = reinterpret_cast<const float4 *>(rh + t * kRouteDim);
            float4 rv[4] = {rt[0], rt[1], rt[2], rt[3]};
            s = score16(rv, c);
        }
        bool avail = g_valid;
        uint32_t bits = 0;
        for (int round = 0; round < topk; ++round) {
            bool bv = avail;
            float bs = s;
            int bg = g;
            for (int off = 1; off < Kp; off <<= 1) {
                const bool ov = __shfl_xor((int)bv, off) != 0;
                const float os = __shfl_xor(bs, off);
                const int og = __shfl_xor(bg, off);
                if (ranks_before(ov, os, og, bv, bs, bg)) {
                    bv = ov;
                    bs = os;
                    bg = og;
                }
            }
            if (g == bg)
                avail = false;
            bits |= 1u << bg;
            if (t_valid && g == 0)
                gh[t * topk + round] = bg;
        }
        if (t_valid && g == 0)
            mh[t] = bits;
    }
}

}  // namespace

hipError_t launch_route(const float *r, const float *centroids, int H, int64_t n, int K,
                        int topk, int32_t *groups, uint32_t *gmask, hipStream_t s)
{
    int kp_log2 = 0;
    while ((1 << kp_log2) < K)
        ++kp_log2;
    const int64_t tokens_per_block = (int64_t)(256 / kWave) * (kWave >> kp_log2);
    int64_t blocks = (n + tokens_per_block - 1) / tokens_per_block;
    if (blocks > 4096)
        blocks = 4096;
    dim3 grid((unsigned)blocks, (unsigned)H);
    hipLaunchKernelGGL(route_kernel, grid, dim3(256), 0, s, r, centroids, n, K, kp_log2,
                       topk, groups, gmask);
    return hipGetLastError();
}

}  // namespace focus
