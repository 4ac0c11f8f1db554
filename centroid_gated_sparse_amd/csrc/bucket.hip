// Bucketing: the per-group token lists for within-group causal attention.
//
// The pages split the sparse pattern into a local-window call and a
// within-group causal call (Technical Summary, Key Contributions 5) without
// saying how tokens are gathered.  Here the n*topk (token, group) entries of
// each routing head are counting-sorted, stably, by the sub-bucket
// group_base(g) + lower_code(g, a, b, c), where a < b (< c) are the token's
// two (three) lowest groups below g (see common.hpp).  Inside a sub-bucket
// positions ascend, so "causal" in bucket order is causal in positions, and a
// tile of one sub-bucket meets a tile of another with a single owner
// decision: their pairs belong to a lower group exactly when the two lower
// sets meet (whenever the codes keep the whole lower set: top-k <= 3, and
// top-k = 4 at K <= 16).
//
// Three kernels, all bound by HBM and integer only:
//   count   one wavefront per chunk of tokens; LDS histogram per wave
//   scan    one block per head: exclusive scan over (sub-bucket, chunk)
//   scatter one wavefront per chunk; stable ranks from wavefront ballots
// A scatter wavefront settles one sub-bucket key per pass, so its time grows
// with the chunk, not with n: short sequences take short chunks (down to one
// wavefront width) so that there are enough wavefronts to spread them.
#include <mutex>

#include "common.hpp"

namespace focus {
namespace {

constexpr int kChunkMax = 512;           // tokens per wavefront chunk, long sequences
constexpr int kChunkMin = 64;            // ... and the shortest chunk
constexpr int64_t kChunkWaves = 8192;    // wavefronts wanted before chunks shrink
constexpr int kWavesPerBlock = 4;       // ... while their histograms fit in 64 KB of LDS
constexpr size_t kHistLdsBytes = 64 * 1024;
constexpr int kCachedTopk = 4;           // scatter keeps keys in registers up to here
constexpr int kScanThreads = 1024;

// Lowest three groups of token t (K where absent).
struct Lowest3 {
    int lo1, lo2, lo3;
};
__device__ __forceinline__ void take_lowest(Lowest3 &l, int g)
{
    const int hi1 = max(g, l.lo1);
    l.lo1 = min(g, l.lo1);
    const int hi2 = max(hi1, l.lo2);
    l.lo2 = min(hi1, l.lo2);
    l.lo3 = min(hi2, l.lo3);
}
__device__ __forceinline__ Lowest3 three_lowest(const int32_t *gt, int topk, int K)
{
    Lowest3 l{K, K, K};
    for (int s = 0; s < topk; ++s)
        take_lowest(l, gt[s]);
    return l;
}

// Sub-bucket of the token's entry in its group g, from its lowest groups
// lo1 < lo2 < lo3: below lo1 it has no lower group, below lo2 only lo1,
// below lo3 lo1 and lo2, and below any higher one lo1, lo2 and (with three
// members kept, m = 3) lo3 are the kept members.
__device__ __forceinline__ int subbucket(int g, const Lowest3 &l, int m)
{
    const int code = g == l.lo1   ? 0
                     : g == l.lo2 ? 1 + l.lo1
                     : (g == l.lo3 || m < 3)
                         ? 1 + g + choose2(l.lo2) + l.lo1
                         : 1 + g + choose2(g) + choose3(l.lo3) + choose2(l.lo2) + l.lo1;
    return group_base(g, m) + code;
}

// Sub-bucket keys of a token's entries, in registers (topk <= TK).  An
// absent token (valid false) or slot s >= topk gets no key that is used.
template <int TK>
__device__ __forceinline__ void entry_keys(const int32_t *gt, int topk, int K, int m, bool valid,
                                           int (&key)[TK])
{
    int g[TK];
    Lowest3 l{K, K, K};
#pragma unroll
    for (int s = 0; s < TK; ++s) {
        g[s] = (valid && s < topk) ? gt[s] : K;  // K: no entry
        take_lowest(l, g[s]);
    }
#pragma unroll
    for (int s = 0; s < TK; ++s)
        key[s] = subbucket(g[s], l, m);
}

// counts[h][sb][chunk]; WPB wavefronts (chunks) per block
template <int TK, int WPB>
__global__ __launch_bounds__(256) void bucket_count_kernel(const int32_t *__restrict__ groups,
                                                           int64_t n, int K, int topk,
                                                           int chunk_len, int nchunks,
                                                           int32_t *__restrict__ counts)
{
    extern __shared__ int32_t hist[];  // [WPB][nsb]
    const int nsb = num_subbuckets(K, topk);
    const int m = code_members(K, topk);
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int h = blockIdx.y;
    const int chunk = blockIdx.x * WPB + wave;
    int32_t *my = hist + wave * nsb;
    for (int i = lane; i < nsb; i += kWave)
        my[i] = 0;
    __syncthreads();
    if (chunk < nchunks) {
        const int32_t *gh = groups + (int64_t)h * n * topk;
        const int64_t t0 = (int64_t)chunk * chunk_len;
        for (int64_t t = t0 + lane; t < t0 + chunk_len && t < n; t += kWave) {
            const int32_t *gt = gh + t * topk;
            if constexpr (TK > 0) {
                int key[TK];
                entry_keys<TK>(gt, topk, K, m, true, key);
#pragma unroll
                for (int s = 0; s < TK; ++s)
                    if (s < topk)
                        atomicAdd(&my[key[s]], 1);
            } else {
                const Lowest3 lo = three_lowest(gt, topk, K);
                for (int s = 0; s < topk; ++s)
                    atomicAdd(&my[subbucket(gt[s], lo, m)], 1);
            }
        }
    }
    __syncthreads();
    if (chunk < nchunks) {
        int32_t *ch = counts + (int64_t)h * nsb * nchunks;
        for (int i = lane; i < nsb; i += kWave)
            ch[(int64_t)i * nchunks + chunk] = my[i];
    }
}

// In place: counts[h][sb][chunk] -> exclusive prefix in (sb, chunk) order;
// offsets[h][sb] = start of sub-bucket sb, offsets[h][nsb] = total.
__global__ __launch_bounds__(kScanThreads) void bucket_scan_kernel(int32_t *__restrict__ counts,
                                                                   int nsb, int nchunks,
                                                                   int32_t *__restrict__ offsets)
{
    __shared__ int32_t partial[kScanThreads / kWave];
    __shared__ int32_t carry_s;
    const int h = blockIdx.x;
    int32_t *c = counts + (int64_t)h * nsb * nchunks;
    int32_t *off = offsets + (int64_t)h * (nsb + 1);
    const int64_t total = (int64_t)nsb * nchunks;
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    if (threadIdx.x == 0)
        carry_s = 0;
    __syncthreads();
    for (int64_t base = 0; base < total; base += kScanThreads) {
        const int64_t i = base + threadIdx.x;
        const int32_t x = i < total ? c[i] : 0;
        // inclusive scan inside the wavefront
        int32_t inc = x;
#pragma unroll
        for (int off_l = 1; off_l < kWave; off_l <<= 1) {
            const int32_t y = __shfl_up(inc, off_l);
            if (lane >= off_l)
                inc += y;
        }
        if (lane == kWave - 1)
            partial[wave] = inc;
        __syncthreads();
        int32_t wave_base = 0;
        for (int w = 0; w < wave; ++w)
            wave_base += partial[w];
        const int32_t carry = carry_s;
        const int32_t excl = carry + wave_base + inc - x;
        if (i < total) {
            c[i] = excl;
            if (i % nchunks == 0)
                off[i / nchunks] = excl;
        }
        __syncthreads();
        if (threadIdx.x == kScanThreads - 1)
            carry_s = excl + x;
        __syncthreads();
    }
    if (threadIdx.x == 0)
        off[nsb] = carry_s;
}

// TK > 0: topk <= TK and each lane keeps its entries' sub-bucket keys in
// registers, so a pass touches memory only for the LDS cursor and the stores.
// TK == 0 serves any topk and re-reads the group ids each pass.  The count
// kernel takes the same two forms.
template <int TK, int WPB>
__global__ __launch_bounds__(256) void bucket_scatter_kernel(
    const int32_t *__restrict__ groups, int64_t n, int K, int topk, int chunk_len, int nchunks,
    const int32_t *__restrict__ bases, int32_t *__restrict__ tokens,
    int32_t *__restrict__ slot_entry)
{
    extern __shared__ int32_t run[];  // [WPB][nsb] running cursor
    const int nsb = num_subbuckets(K, topk);
    const int m = code_members(K, topk);
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int h = blockIdx.y;
    const int chunk = blockIdx.x * WPB + wave;
    if (chunk >= nchunks)
        return;  // whole wavefront leaves together; no block barrier below
    int32_t *my = run + wave * nsb;
    const int32_t *bh = bases + (int64_t)h * nsb * nchunks;
    for (int i = lane; i < nsb; i += kWave)
        my[i] = bh[(int64_t)i * nchunks + chunk];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");

    const int32_t *gh = groups + (int64_t)h * n * topk;
    int32_t *th = tokens + (int64_t)h * n * topk;
    int32_t *sh = slot_entry + (int64_t)h * n * topk;
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int64_t t0 = (int64_t)chunk * chunk_len;
    for (int64_t tb = t0; tb < t0 + chunk_len && tb < n; tb += kWave) {
        const int64_t t = tb + lane;
        const bool valid = t < n;
        const int32_t *gt = gh + (valid ? t : tb) * topk;
        int key[TK > 0 ? TK : 1];
        Lowest3 lo{K, K, K};
        if constexpr (TK > 0)
            entry_keys<TK>(gt, topk, K, m, valid, key);
        else if (valid)
            lo = three_lowest(gt, topk, K);
        uint32_t pending = valid ? (topk >= 32 ? ~0u : ((1u << topk) - 1u)) : 0u;
        // Each pass settles one sub-bucket key X: every lane holding an entry
        // with key X takes rank (cursor[X] + number of lower lanes holding X).
        // A token has at most one entry per key, so lane order is token order.
        while (true) {
            const uint64_t any = __ballot(pending != 0);
            if (any == 0)
                break;
            const int leader = __ffsll((unsigned long long)any) - 1;
            int my_key = -1;
            if constexpr (TK > 0) {
#pragma unroll
                for (int s = TK - 1; s >= 0; --s)
                    if ((pending >> s) & 1u)
                        my_key = key[s];
            } else if (pending != 0) {
                my_key = subbucket(gt[__ffs(pending) - 1], lo, m);
            }
            const int X = __builtin_amdgcn_readlane(my_key, leader);
            int sx = -1;
            if constexpr (TK > 0) {
#pragma unroll
                for (int s = 0; s < TK; ++s)
                    if (((pending >> s) & 1u) && key[s] == X)
                        sx = s;
            } else {
                for (uint32_t p = pending; p != 0; p &= p - 1) {
                    const int s = __ffs(p) - 1;
                    if (subbucket(gt[s], lo, m) == X)
                        sx = s;
                }
            }
            const uint64_t members = __ballot(sx >= 0);
            const int32_t cursor = my[X];
            if (sx >= 0) {
                const int32_t e = cursor + __popcll(members & lanes_below);
                th[e] = (int32_t)t;
                sh[t * topk + sx] = e;
                pending &= ~(1u << sx);
            }
            __builtin_amdgcn_wave_barrier();
            if (lane == leader)
                my[X] = cursor + __popcll(members);
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        }
    }
}

// Scratch of focus_bucket_noalloc: the per-chunk sub-bucket counts, one int
// per (head, sub-bucket, chunk), as the workspace of focus_bucket holds them.
// Each device the library runs on keeps its own copy until the process ends.
// In host code `scratch` names a host-side stand-in, not the device array:
// the device address comes from hipGetSymbolAddress (bucket_noalloc_scratch).
static __device__ __align__(256) int32_t scratch[FOCUS_BUCKET_NOALLOC_SCRATCH_BYTES / 4];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

// Device address of this device's scratch array, looked up once per device
// (with that device current) and kept.
hipError_t bucket_noalloc_scratch(void **ptr, size_t *bytes)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = sizeof(scratch);
    return hipSuccess;
}

// Tokens per chunk: kChunkMax, halved (down to kChunkMin) while the heads
// have fewer than kChunkWaves chunks between them.
int bucket_chunk(int H, int64_t n)
{
    int c = kChunkMax;
    while (c > kChunkMin && (int64_t)H * ((n + c - 1) / c) < kChunkWaves)
        c /= 2;
    return c;
}

size_t bucket_workspace_bytes(int H, int64_t n, int K, int topk)
{
    const int chunk = bucket_chunk(H, n);
    const int64_t nchunks = (n + chunk - 1) / chunk;
    return align_up((size_t)H * num_subbuckets(K, topk) * nchunks * sizeof(int32_t), 256);
}

namespace {
template <int WPB>
hipError_t launch_bucket_wpb(const int32_t *groups, int H, int64_t n, int K, int topk,
                             int32_t *offsets, int32_t *tokens, int32_t *slot_entry, void *ws,
                             hipStream_t s)
{
    const int nsb = num_subbuckets(K, topk);
    const int chunk = bucket_chunk(H, n);
    const int nchunks = (int)((n + chunk - 1) / chunk);
    int32_t *counts = static_cast<int32_t *>(ws);
    const dim3 grid((nchunks + WPB - 1) / WPB, H);
    const size_t lds = sizeof(int32_t) * nsb * WPB;
    if (topk <= kCachedTopk)
        hipLaunchKernelGGL((bucket_count_kernel<kCachedTopk, WPB>), grid, dim3(kWave * WPB), lds, s,
                           groups, n, K, topk, chunk, nchunks, counts);
    else
        hipLaunchKernelGGL((bucket_count_kernel<0, WPB>), grid, dim3(kWave * WPB), lds, s, groups,
                           n, K, topk, chunk, nchunks, counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(bucket_scan_kernel, dim3(H), dim3(kScanThreads), 0, s, counts, nsb,
                       nchunks, offsets);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (topk <= kCachedTopk)
        hipLaunchKernelGGL((bucket_scatter_kernel<kCachedTopk, WPB>), grid, dim3(kWave * WPB), lds,
                           s, groups, n, K, topk, chunk, nchunks, counts, tokens, slot_entry);
    else
        hipLaunchKernelGGL((bucket_scatter_kernel<0, WPB>), grid, dim3(kWave * WPB), lds, s,
                           groups, n, K, topk, chunk, nchunks, counts, tokens, slot_entry);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_bucket(const int32_t *groups, int H, int64_t n, int K, int topk,
                         int32_t *offsets, int32_t *tokens, int32_t *slot_entry, void *ws,
                         hipStream_t s)
{
    // four chunks per block while their LDS histograms fit in 64 KB (up to
    // 4,096 sub-buckets), one otherwise (K above 28 at top-3 or more)
    if (sizeof(int32_t) * num_subbuckets(K, topk) * kWavesPerBlock <= kHistLdsBytes)
        return launch_bucket_wpb<kWavesPerBlock>(groups, H, n, K, topk, offsets, tokens,
                                                 slot_entry, ws, s);
    return launch_bucket_wpb<1>(groups, H, n, K, topk, offsets, tokens, slot_entry, ws, s);
}

}  // namespace focus
