// Training-mode Focus forward: the Sinkhorn soft assignment (the gated dense
// causal attention is the GATED form of the kernel in attn.hip).
//
// gist.science Technical Summary, Core Architecture (tokens are softly
// assigned to groups; distant pairs pass a learned gate
// s_ij = q_i.k_j * sigmoid(lambda a_ij), a_ij the group affinity), Key
// Technical Innovation (Sinkhorn normalisation in place of softmax keeps the
// group sizes balanced: a doubly-stochastic assignment) and Significance
// (training still evaluates all O(n^2) pairs because of the soft gate).
// Readings where the pages are silent: the assignment starts from
// exp(score - the token's max score); one Sinkhorn iteration scales every
// group column to total n/K and then every token row to total 1; a_ij =
// A_i . A_j; the gate multiplies the scores of far pairs (i - j >= w) only,
// window pairs keep the plain score, and every j <= i is attended.
//
// Sinkhorn: per routing head an n x K fp32 matrix; each pass is one kernel
// over the tokens that also leaves per-block column sums (fp64, summed in a
// fixed order by a one-block kernel), so the result is deterministic.
//
// The gated attention itself runs in the inference forward's dense window
// kernel (attn.hip, its GATED form).
#include <algorithm>

#include "attn_common.hpp"

namespace focus {
namespace {
using namespace attn;

// ---------------------------------------------------------------------------
// Sinkhorn

constexpr int kSkBlock = 256;

__device__ __forceinline__ float score_fixed(const float *__restrict__ r,
                                             const float *__restrict__ c)
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

// Block-level column sums of a [tokens][K] tile (fp64, fixed tree order).
__device__ void block_column_sums(const float (&a)[kMaxGroups], int K, double *out)
{
    __shared__ double red[kSkBlock / kWave][kMaxGroups];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    for (int g = 0; g < K; ++g) {
        double x = a[g];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1)
            x += __shfl_xor(x, off);
        if (lane == 0)
            red[wave][g] = x;
    }
    __syncthreads();
    if (threadIdx.x < K) {
        double x = 0.0;
        for (int w = 0; w < kSkBlock / kWave; ++w)
            x += red[w][threadIdx.x];
        out[threadIdx.x] = x;
    }
}

// exp(score - row max) of every token; block column sums into part.
__global__ __launch_bounds__(kSkBlock) void sinkhorn_init_kernel(
    const float *__restrict__ r, const float *__restrict__ centroids, int64_t n, int K,
    float *__restrict__ A, double *__restrict__ part)
{
    const int h = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * kSkBlock + threadIdx.x;
    float a[kMaxGroups];
#pragma unroll
    for (int g = 0; g < kMaxGroups; ++g)
        a[g] = 0.f;
    if (t < n) {
        const float *rt = r + ((int64_t)h * n + t) * kRouteDim;
        float rv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e)
            rv[e] = rt[e];
        float mx = -INFINITY;
#pragma unroll
        for (int g = 0; g < kMaxGroups; ++g)
            if (g < K) {
                a[g] = score_fixed(rv, centroids + ((int64_t)h * K + g) * kRouteDim);
                mx = fmaxf(mx, a[g]);
            }
        float *At = A + ((int64_t)h * n + t) * K;
#pragma unroll
        for (int g = 0; g < kMaxGroups; ++g)
            if (g < K) {
                a[g] = expf(a[g] - mx);
                At[g] = a[g];
            }
    }
    block_column_sums(a, K, part + ((int64_t)h * gridDim.x + blockIdx.x) * kMaxGroups);
}

// col[h][g] = sum over blocks of part (fixed order), one block per head.
__global__ __launch_bounds__(kSkBlock) void sinkhorn_colsum_kernel(
    const double *__restrict__ part, int nblocks, int K, double *__restrict__ col)
{
    const int h = blockIdx.x;
    __shared__ double red[kSkBlock];
    for (int g = 0; g < K; ++g) {
        double x = 0.0;
        for (int b = threadIdx.x; b < nblocks; b += kSkBlock)
            x += part[((int64_t)h * nblocks + b) * kMaxGroups + g];
        red[threadIdx.x] = x;
        __syncthreads();
        for (int s = kSkBlock / 2; s >= 1; s >>= 1) {
            if (threadIdx.x < s)
                red[threadIdx.x] += red[threadIdx.x + s];
            __syncthreads();
        }
        if (threadIdx.x == 0)
            col[(int64_t)h * kMaxGroups + g] = red[0];
        __syncthreads();
    }
}

// One iteration: columns to n/K, then rows to 1; block column sums of the
// result for the next iteration.
__global__ __launch_bounds__(kSkBlock) void sinkhorn_step_kernel(
    int64_t n, int K, const double *__restrict__ col, float *__restrict__ A,
    double *__restrict__ part)
{
    const int h = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * kSkBlock + threadIdx.x;
    float a[kMaxGroups];
#pragma unroll
    for (int g = 0; g < kMaxGroups; ++g)
        a[g] = 0.f;
    if (t < n) {
        float *At = A + ((int64_t)h * n + t) * K;
        const double target = (double)n / K;
        double rs = 0.0;
        double x[kMaxGroups];
#pragma unroll
        for (int g = 0; g < kMaxGroups; ++g)
            if (g < K) {
                x[g] = (double)At[g] * (target / col[(int64_t)h * kMaxGroups + g]);
                rs += x[g];
            }
#pragma unroll
        for (int g = 0; g < kMaxGroups; ++g)
            if (g < K) {
                a[g] = (float)(x[g] / rs);
                At[g] = a[g];
            }
    }
    block_column_sums(a, K, part + ((int64_t)h * gridDim.x + blockIdx.x) * kMaxGroups);
}

}  // namespace

size_t sinkhorn_workspace_bytes(int H, int64_t n)
{
    const int64_t nblocks = (n + kSkBlock - 1) / kSkBlock;
    return align_up(sizeof(double) * H * nblocks * kMaxGroups, 256) +
           sizeof(double) * H * kMaxGroups;
}

hipError_t launch_sinkhorn(const float *r, const float *centroids, int H, int64_t n, int K,
                           int iters, float *A, void *ws, hipStream_t s)
{
    const int nblocks = (int)((n + kSkBlock - 1) / kSkBlock);
    double *part = static_cast<double *>(ws);
    double *col = reinterpret_cast<double *>(
        static_cast<char *>(ws) + align_up(sizeof(double) * H * nblocks * kMaxGroups, 256));
    const dim3 grid((unsigned)nblocks, (unsigned)H);
    hipLaunchKernelGGL(sinkhorn_init_kernel, grid, dim3(kSkBlock), 0, s, r, centroids, n, K, A,
                       part);
    for (int it = 0; it < iters; ++it) {
        hipLaunchKernelGGL(sinkhorn_colsum_kernel, dim3(H), dim3(kSkBlock), 0, s, part, nblocks,
                           K, col);
        hipLaunchKernelGGL(sinkhorn_step_kernel, grid, dim3(kSkBlock), 0, s, n, K, col, A, part);
    }
    return hipGetLastError();
}

}  // namespace focus
