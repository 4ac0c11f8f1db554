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

// One token per lane (K <= 8): each lane reads its token's 64-byte routing
// vector, consecutive lanes consecutive tokens, so every byte of r is loaded
// once and the loads coalesce; the centroids are wave-uniform scalar loads.
// Same fixed-order scores and the same ranking as route_kernel (a scan that
// takes a group only on a strictly larger score keeps the lower index on
// equal scores, as the butterfly's order does).
template <int KMAX>
__global__ __launch_bounds__(256) void route_lane_kernel(const float *__restrict__ r,
                                                         const float *__restrict__ centroids,
                                                         int64_t n, int K, int topk,
                                                         int32_t *__restrict__ groups,
                                                         uint32_t *__restrict__ gmask);

// ---------------------------------------------------------------------------
// Fused projection + routing: r_t = W x_t, then every routing head's top-k
// from r_t (Technical Summary, Core Architecture / Token Grouping: each
// hidden state is projected to the 16-dimensional centroid space; the
// projection is one d_model x 16 matrix per layer, the parameter counts of
// the thelatestinai.com Tables 2 and 3).
//
// The work is plain fp32 vector arithmetic: r_t[j] starts at +0 and adds
// Wt[e][j] * x_t[e] for e = 0, 1, ... with a separate multiply and add (no
// fused multiply-add), so it is reproducible bit for bit.  One lane owns one
// token and its 16 sums (more tokens per lane measured slower: fewer waves
// hide less latency).  Wt (d_model rows of 16 weights) is the same for every
// lane: a row is one 64-byte scalar load whose values enter the vector
// instructions as scalar operands.  The rows come through a ring of
// kProjAhead + 1 SGPR rows, fetched kProjAhead rows ahead of their use, with
// scheduling fences so the compiler keeps the loads early.  Hidden states
// stream through 16-byte loads, one 8-element chunk ahead.  At 2 * 16
// vector operations per element the kernel is bound by the fp32 vector rate,
// not by HBM.

constexpr int kProjBlock = 256;  // threads per block
constexpr int kProjChunk = 8;    // hidden-state elements per load
constexpr int kProjAhead = 3;    // weight rows in flight ahead of the arithmetic

template <bool BF16>
struct XChunk;

// Eight bf16 hidden-state values (one 16-byte load), widened exactly.
template <>
struct XChunk<true> {
    uint4 raw;
    __device__ __forceinline__ void load(const char *row, int e0)
    {
        raw = *reinterpret_cast<const uint4 *>(row + (size_t)e0 * 2);
    }
    __device__ __forceinline__ float at(int u) const
    {
        const uint32_t w = u < 2 ? raw.x : u < 4 ? raw.y : u < 6 ? raw.z : raw.w;
        return __uint_as_float((u & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};

// Eight fp32 hidden-state values (two 16-byte loads).
template <>
struct XChunk<false> {
    float4 a, b;
    __device__ __forceinline__ void load(const char *row, int e0)
    {
        const float4 *p = reinterpret_cast<const float4 *>(row + (size_t)e0 * 4);
        a = p[0];
        b = p[1];
    }
    __device__ __forceinline__ float at(int u) const
    {
        const float4 &h = u < 4 ? a : b;
        const int k = u & 3;
        return k == 0 ? h.x : k == 1 ? h.y : k == 2 ? h.z : h.w;
    }
};

__device__ __forceinline__ float load_one(const char *row, bool bf16, int e)
{
    if (bf16)
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(row)[e] << 16);
    return reinterpret_cast<const float *>(row)[e];
}

// Score of a routing vector against one centroid: the same order as score16.
__device__ __forceinline__ float score_r(const float (&r)[16], const float *__restrict__ c)
{
#pragma clang fp contract(off)
    float s = r[0] * c[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) {
        float p = r[e] * c[e];
        s = s + p;
    }
    return s;
}

// Routing of one token for every head: selection of the k best groups,
// scanning upward and taking a group only on a strictly larger score, so
// equal scores go to the lower index.
template <int KMAX = kMaxGroups>
__device__ __forceinline__ void route_token(const float (&r)[16], int64_t t, int64_t n,
                                            const float *__restrict__ centroids, int H, int K,
                                            int topk, int32_t *__restrict__ groups,
                                            uint32_t *__restrict__ gmask)
{
    for (int h = 0; h < H; ++h) {
        const float *ch = centroids + (int64_t)h * K * kRouteDim;
        float s[KMAX];
#pragma unroll
        for (int g = 0; g < KMAX; ++g)
            s[g] = g < K ? score_r(r, ch + g * kRouteDim) : 0.f;
        uint32_t taken = 0;
        int32_t *gt = groups + ((int64_t)h * n + t) * topk;
        for (int sel = 0; sel < topk; ++sel) {
            int best = -1;
            float bs = 0.f;
#pragma unroll
            for (int g = 0; g < KMAX; ++g) {
                if (g < K && !((taken >> g) & 1u) && (best < 0 || s[g] > bs)) {
                    best = g;
                    bs = s[g];
                }
            }
            taken |= 1u << best;
            gt[sel] = best;
        }
        gmask[(int64_t)h * n + t] = taken;
    }
}

template <int KMAX>
__global__ __launch_bounds__(256) void route_lane_kernel(const float *__restrict__ r,
                                                         const float *__restrict__ centroids,
                                                         int64_t n, int K, int topk,
                                                         int32_t *__restrict__ groups,
                                                         uint32_t *__restrict__ gmask)
{
    const int h = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n)
        return;
    const float4 *rt = reinterpret_cast<const float4 *>(r + ((int64_t)h * n + t) * kRouteDim);
    float rv[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 v = rt[q];
        rv[4 * q] = v.x;
        rv[4 * q + 1] = v.y;
        rv[4 * q + 2] = v.z;
        rv[4 * q + 3] = v.w;
    }
    route_token<KMAX>(rv, t, n, centroids + (int64_t)h * K * kRouteDim, 1, K, topk,
                      groups + (int64_t)h * n * topk, gmask + (int64_t)h * n);
}

// Adds one chunk of 8 elements to the sums, element by element in order.
// On entry ring[16 * a + j] holds weight row e0 + a (a < kProjAhead); `next`
// points at the chunk after this one (rows e0 + 8, ...), or at any valid
// chunk when this is the last.
template <bool BF16>
__device__ __forceinline__ void project_chunk(float (&acc)[16], const XChunk<BF16> &xc,
                                              float (&ring)[16 * kProjAhead],
                                              const float *__restrict__ wt,
                                              const float *__restrict__ next)
{
#pragma clang fp contract(off)
#pragma unroll
    for (int u = 0; u < kProjChunk; ++u) {
        const float xv = xc.at(u);
        const float *src = u + kProjAhead < kProjChunk
                               ? wt + (u + kProjAhead) * kRouteDim
                               : next + (u + kProjAhead - kProjChunk) * kRouteDim;
        float fetched[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            fetched[j] = src[j];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float p = ring[j] * xv;
            acc[j] = acc[j] + p;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int a = 0; a + 1 < kProjAhead; ++a)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                ring[16 * a + j] = ring[16 * (a + 1) + j];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            ring[16 * (kProjAhead - 1) + j] = fetched[j];
    }
}

// VEC: d_model is a multiple of 8, so rows are 16-byte aligned and the
// hidden states move in 8-element chunks; otherwise one element at a time.
// Thread g of the grid owns token g.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kProjBlock) void route_project_kernel(
    const void *__restrict__ x, int64_t n, int dm, const float *__restrict__ Wt,
    const float *__restrict__ centroids, int H, int K, int topk,
    int32_t *__restrict__ groups, uint32_t *__restrict__ gmask, float *__restrict__ r_out)
{
#pragma clang fp contract(off)
    constexpr size_t esize = BF16 ? 2 : 4;
    const int64_t t = (int64_t)blockIdx.x * kProjBlock + threadIdx.x;
    const int64_t tl = t < n ? t : n - 1;  // tail lanes repeat the last row
    const char *row = static_cast<const char *>(x) + (size_t)tl * dm * esize;

    float acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        acc[j] = 0.f;

    if constexpr (VEC) {
        const int chunks = dm / kProjChunk;
        const float *last = Wt + (size_t)(chunks - 1) * kProjChunk * kRouteDim;
        auto chunk_w = [&](int c) {
            return c < chunks ? Wt + (size_t)c * kProjChunk * kRouteDim : last;
        };
        float ring[16 * kProjAhead];
#pragma unroll
        for (int a = 0; a < 16 * kProjAhead; ++a)
            ring[a] = Wt[a];  // rows 0 .. kProjAhead-1 (d_model >= 8)
        // two chunk buffers: the loads of one chunk are in flight while the
        // other is summed
        XChunk<BF16> xa, xb;
        xa.load(row, 0);
        int c = 0;
        for (; c + 2 <= chunks; c += 2) {
            xb.load(row, (c + 1) * kProjChunk);
            project_chunk<BF16>(acc, xa, ring, chunk_w(c), chunk_w(c + 1));
            xa.load(row, (c + 2 < chunks ? c + 2 : c + 1) * kProjChunk);
            project_chunk<BF16>(acc, xb, ring, chunk_w(c + 1), chunk_w(c + 2));
        }
        if (c < chunks)  // odd chunk count: xa holds the last chunk
            project_chunk<BF16>(acc, xa, ring, chunk_w(c), chunk_w(c + 1));
    } else {
        for (int e = 0; e < dm; ++e) {
            const float xv = load_one(row, BF16, e);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float p = Wt[(size_t)e * kRouteDim + j] * xv;
                acc[j] = acc[j] + p;
            }
        }
    }

    if (t >= n)
        return;
    if (r_out != nullptr) {
        float4 *ro = reinterpret_cast<float4 *>(r_out + t * kRouteDim);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            ro[q4] = make_float4(acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]);
    }
    route_token(acc, t, n, centroids, H, K, topk, groups, gmask);
}

}  // namespace

hipError_t launch_route(const float *r, const float *centroids, int H, int64_t n, int K,
                        int topk, int32_t *groups, uint32_t *gmask, hipStream_t s)
{
    if (K <= 8) {
        const dim3 grid((unsigned)((n + 255) / 256), (unsigned)H);
        if (K <= 4)
            hipLaunchKernelGGL(route_lane_kernel<4>, grid, dim3(256), 0, s, r, centroids, n, K,
                               topk, groups, gmask);
        else
            hipLaunchKernelGGL(route_lane_kernel<8>, grid, dim3(256), 0, s, r, centroids, n, K,
                               topk, groups, gmask);
        return hipGetLastError();
    }
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

hipError_t launch_route_project(const void *x, bool bf16, int64_t n, int dm, const float *Wt,
                                const float *centroids, int H, int K, int topk,
                                int32_t *groups, uint32_t *gmask, float *r_out, hipStream_t s)
{
    const int64_t blocks = (n + kProjBlock - 1) / kProjBlock;
    const bool vec = dm % kProjChunk == 0;
    auto kern = bf16 ? (vec ? route_project_kernel<true, true> : route_project_kernel<true, false>)
                     : (vec ? route_project_kernel<false, true>
                            : route_project_kernel<false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kProjBlock), 0, s, x, n, dm, Wt,
                       centroids, H, K, topk, groups, gmask, r_out);
    return hipGetLastError();
}

}  // namespace focus
