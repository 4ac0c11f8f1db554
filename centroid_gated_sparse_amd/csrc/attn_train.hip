// Training-mode Focus forward: Sinkhorn soft assignment and gated dense
// causal attention.
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
// Gated attention: query-major like the forward (128 query rows per block,
// 32 per wavefront, 64-key tiles staged through LDS).  S^T = K Q^T on bf16
// MFMA; the affinity tile a^T = A_k A_q^T is one more MFMA per 32 keys and
// 16 groups (the assignment rounded to bf16, zero-padded to 16 or 32
// groups); online softmax in the exp2 domain with lazy rescaling; O^T +=
// V^T P^T with V^T written transposed into LDS at staging time.
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

// ---------------------------------------------------------------------------
// gated dense causal attention

constexpr int kGThreads = 256;  // 4 wavefronts
constexpr int kGRows = 128;     // query rows per block
constexpr int kGKeys = 64;      // keys per staged tile

struct GatedParams {
    int hq, hkv, ratio, K, window, row_tiles;
    int64_t n;
    float c;        // scale * log2(e)
    float lam2;     // lambda * log2(e): sigmoid(lambda a) = 1 / (1 + 2^(-lam2 a))
    const __bf16 *q, *k, *v;
    const bf16x8 *apack;  // [hkv][n][KA / 8]: the assignment in bf16, zero-padded
    __bf16 *out;
    float *lse;
};

template <int D>
__device__ __forceinline__ int grswz(int row)
{
    if (D == 128)
        return (row & 3) | (((row >> 4) & 1) << 2) | (((row >> 2) & 1) << 3);
    return ((row & 3) | (((row >> 4) & 1) << 2)) ^ ((row >> 2) & 1);
}
template <int D>
__device__ __forceinline__ int grslot(int row, int c)
{
    return row * (D / 8) + (c ^ grswz<D>(row));
}
__device__ __forceinline__ int gtslot(int d, int c)  // [D][64 keys], 8 chunks a row
{
    return d * 8 + (c ^ ((d & 7) ^ ((d >> 3) & 1)));
}
__device__ __forceinline__ bf16x8 glds16(const char *base, int slot)
{
    return *reinterpret_cast<const bf16x8 *>(base + slot * 16);
}

// The assignment rounded to bf16 and zero-padded to KA groups, one row of
// KA / 8 16-byte chunks per token, so the attention kernel reads it with
// unconditional vector loads.
__global__ __launch_bounds__(256) void gated_pack_kernel(const float *__restrict__ assign,
                                                         int64_t rows, int K, int KA,
                                                         __bf16 *__restrict__ apack)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * KA)
        return;
    const int64_t t = idx / KA;
    const int g = (int)(idx % KA);
    apack[idx] = (__bf16)(g < K ? assign[t * K + g] : 0.f);
}

template <int D, int KA>  // KA: groups padded to 16 or 32
__global__ __launch_bounds__(kGThreads, 1) void gated_fwd_kernel(GatedParams p)
{
    constexpr int KS = D / 16, DB = D / 32, KCH = D / 8;
    constexpr int CHUNKS = kGKeys * KCH / kGThreads;
    constexpr int ACH = KA / 8;  // 16-byte chunks of a padded assignment row
    __shared__ __attribute__((aligned(16))) char k_lds[kGKeys * D * 2];
    __shared__ __attribute__((aligned(16))) char vt_lds[D * kGKeys * 2];
    __shared__ __attribute__((aligned(16))) char a_lds[kGKeys * KA * 2];

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int m = lane % 32;
    const int h = lane / 32;

    const int slot = blockIdx.x % p.row_tiles;
    const int hq = blockIdx.x / p.row_tiles;
    const int kvh = hq / p.ratio;
    const int64_t p_start = (int64_t)slot * kGRows;
    const int tile_rows = (int)std::min<int64_t>(kGRows, p.n - p_start);

    const int qr = wave * 32 + m;
    const bool qvalid = qr < tile_rows;
    const int qpos = (int)(p_start + (qvalid ? qr : 0));
    bf16x8 qf[KS], aq[KA / 16];
    {
        const bf16x8 *qs = reinterpret_cast<const bf16x8 *>(p.q + ((int64_t)hq * p.n + qpos) * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = qs[ks * 2 + h];
        const bf16x8 *arow = p.apack + ((int64_t)kvh * p.n + qpos) * ACH;
#pragma unroll
        for (int j = 0; j < KA / 16; ++j)
            aq[j] = arow[2 * j + h];
    }
    const int w = p.window;

    // keys 0 .. last row of the block, in tiles of 64
    const int n_tiles = (int)((p_start + tile_rows - 1) / kGKeys + 1);

    // staging: thread t stages key row t % 64, chunks 4 i + t / 64
    const int srow = threadIdx.x % kGKeys;
    const int sc0 = threadIdx.x / kGKeys;
    uint4 kr[CHUNKS], vr[CHUNKS];
    bf16x8 ar;
    auto fetch = [&](int tile) {
        const int64_t j = std::min<int64_t>((int64_t)tile * kGKeys + srow, p.n - 1);
        const int64_t base = ((int64_t)kvh * p.n + j) * D;
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int c = 4 * i + sc0;
            kr[i] = *reinterpret_cast<const uint4 *>(p.k + base + c * 8);
            vr[i] = *reinterpret_cast<const uint4 *>(p.v + base + c * 8);
        }
        if (sc0 < ACH)
            ar = p.apack[((int64_t)kvh * p.n + j) * ACH + sc0];
    };
    auto land = [&]() {
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int c = 4 * i + sc0;
            *reinterpret_cast<uint4 *>(k_lds + grslot<D>(srow, c) * 16) = kr[i];
            const uint32_t wv[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint16_t bits =
                    (uint16_t)((u & 1) ? (wv[u >> 1] >> 16) : (wv[u >> 1] & 0xffffu));
                *reinterpret_cast<uint16_t *>(vt_lds + gtslot(8 * c + u, srow >> 3) * 16 +
                                              (srow & 7) * 2) = bits;
            }
        }
        if (sc0 < ACH)
            *reinterpret_cast<bf16x8 *>(a_lds + (srow * ACH + sc0) * 16) = ar;
    };

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            o[db][r] = 0.f;
    float mrun = -INFINITY, lrun = 0.f;  // log2-domain running max and sum

    int koff[KS], vtoff[4];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        koff[ks] = grslot<D>(sigma(m), 2 * ks + h);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        vtoff[j] = gtslot(m, 4 * (j >> 1) + 2 * h + (j & 1));

    fetch(0);
    for (int it = 0; it < n_tiles; ++it) {
        __syncthreads();
        land();
        __syncthreads();
        if (it + 1 < n_tiles)
            fetch(it + 1);
        const int origin = it * kGKeys;
        // per lane: keys kk <= chi are causal, kk <= fhi are far (gated)
        const int chi = qvalid ? qpos - origin : -1;
        const int fhi = qpos - w - origin;
        const bool all_in = __builtin_amdgcn_ballot_w64(!(chi >= kGKeys - 1)) == 0;
        const bool all_far = __builtin_amdgcn_ballot_w64(!(fhi >= kGKeys - 1)) == 0;
        const bool none_far = __builtin_amdgcn_ballot_w64(fhi >= 0) == 0;

        // S^T for the two 32-key blocks: block 1's K fragments are read
        // between block 0's MFMAs, the assignment and V^T fragments between
        // block 1's (fenced order, so LDS latency is not paid per MFMA).
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[kb][r] = 0.f;
        bf16x8 kfr[KS], vf[DB][4], af[2][KA / 16];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kfr[ks] = glds16(k_lds, koff[ks]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[ks], qf[ks], s[0], 0, 0, 0);
            kfr[ks] = glds16(k_lds, koff[ks] + 32 * KCH);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < KA / 16; ++j)
                af[kb][j] = glds16(a_lds, (kb * 32 + sigma(m)) * ACH + 2 * j + h);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[ks], qf[ks], s[1], 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4 * DB / KS; ++q) {
                const int f = ks * (4 * DB / KS) + q;
                vf[f / 4][f % 4] = glds16(vt_lds, vtoff[f % 4] + (f / 4) * 32 * 8);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (!none_far) {
                // affinity a^T = A_k A_q^T for these 32 keys
                f32x16 a;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    a[r] = 0.f;
#pragma unroll
                for (int j = 0; j < KA / 16; ++j)
                    a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kb][j], aq[j], a, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float gate =
                        __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-p.lam2 * a[r]));
                    const int kk = kb * 32 + 16 * h + r;
                    s[kb][r] *= (all_far || kk <= fhi) ? gate : 1.f;
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float t = s[kb][r] * p.c;
                if (!all_in)
                    t = (kb * 32 + 16 * h + r <= chi) ? t : -INFINITY;
                s[kb][r] = t;
            }
        }
        // online softmax: tile max over both halves of the wavefront
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mx = fmaxf(mx, s[kb][r]);
        mx = swap_halves_max(mx);
        if (__builtin_amdgcn_ballot_w64(mx > mrun + kLazyRescale) != 0) {
            const float mnew = fmaxf(mrun, mx);
            const float alpha = (mrun == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mrun - mnew);
            lrun *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    o[db][r] *= alpha;
            mrun = mnew;
        }
        float ls = 0.f;
        bf16x8 pf[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = __builtin_amdgcn_exp2f(s[kb][r] - mrun);
                s[kb][r] = pr;
                ls += pr;
            }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    pf[kb][t][u] = (__bf16)s[kb][8 * t + u];
        }
        lrun += swap_halves_sum(ls);
        // O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][j], pf[j >> 1][j & 1],
                                                               o[db], 0, 0, 0);
    }

    if (qvalid) {
        const float inv = 1.f / lrun;
        __bf16 *dst = p.out + ((int64_t)hq * p.n + qpos) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    dst[db * 32 + 8 * j + 4 * h + u] = (__bf16)(o[db][4 * j + u] * inv);
        if (h == 0)
            p.lse[(int64_t)hq * p.n + qpos] = (mrun + __builtin_amdgcn_logf(lrun)) * kLn2;
    }
}

template <int D, int KA>
void launch_gated_d(const GatedParams &p, hipStream_t s)
{
    hipLaunchKernelGGL((gated_fwd_kernel<D, KA>), dim3((unsigned)(p.hq * p.row_tiles)),
                       dim3(kGThreads), 0, s, p);
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

size_t gated_workspace_bytes(int hkv, int64_t n, int K)
{
    return sizeof(__bf16) * (size_t)hkv * n * (K > 16 ? 32 : 16);
}

hipError_t launch_gated_attn(const AttnShape &sh, const void *q, const void *k, const void *v,
                             const float *assign, float lambda, void *out, float *lse, void *ws,
                             hipStream_t s)
{
    GatedParams p{};
    p.hq = sh.hq;
    p.hkv = sh.hkv;
    p.ratio = sh.hq / sh.hkv;
    p.K = sh.K;
    p.n = sh.n;
    p.window = (int)std::min<int64_t>(sh.window, sh.n);
    p.row_tiles = (int)((sh.n + kGRows - 1) / kGRows);
    p.c = sh.scale * kLog2e;
    p.lam2 = lambda * kLog2e;
    p.q = static_cast<const __bf16 *>(q);
    p.k = static_cast<const __bf16 *>(k);
    p.v = static_cast<const __bf16 *>(v);
    const bool wide = sh.K > 16;
    const int KA = wide ? 32 : 16;
    const int64_t rows = (int64_t)sh.hkv * sh.n;
    hipLaunchKernelGGL(gated_pack_kernel, dim3((unsigned)((rows * KA + 255) / 256)), dim3(256),
                       0, s, assign, rows, sh.K, KA, static_cast<__bf16 *>(ws));
    p.apack = static_cast<const bf16x8 *>(ws);
    p.out = static_cast<__bf16 *>(out);
    p.lse = lse;
    if (sh.d == 128)
        wide ? launch_gated_d<128, 32>(p, s) : launch_gated_d<128, 16>(p, s);
    else
        wide ? launch_gated_d<64, 32>(p, s) : launch_gated_d<64, 16>(p, s);
    return hipGetLastError();
}

}  // namespace focus
