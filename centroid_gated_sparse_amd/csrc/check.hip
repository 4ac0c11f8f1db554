// Consistency check of a bucketing against the routing it claims to come
// from, run before anything indexes key/value rows through it.
//
// focus_attn_fwd and focus_attn_bwd read K, V and Q rows at positions taken
// from `tokens` and find each row's partial results through `slot_entry`; a
// bucketing that was not built from the same routing would send those reads
// anywhere.  The check reads every array only inside its own extent (every
// value is range-tested before it serves as an index), so inconsistent input
// turns into an error bit, never into a stray access.  What it establishes,
// per head (the bucketing of focus_bucket: a stable sort of the n*topk
// (token, group) entries by sub-bucket group_base(g) + lower-set code):
//   offsets  start at 0, never decrease, end at n*topk              (bit 1)
//   tokens   in [0, n), strictly ascending inside each sub-bucket   (bit 2)
//   groups   the entry's group is one of its token's gmask bits and the
//            sub-bucket's lower-set code is the token's (its lowest two or
//            three groups below the entry's group); every gmask holds exactly topk
//            bits                                                  (bit 4)
//   slots    slot_entry[t][s] is an entry of token t, and the groups of a
//            token's topk entries are exactly its gmask bits          (bit 8)
// Together these make slot_entry a bijection onto the entries.
#include <algorithm>

#include "common.hpp"

namespace focus {
namespace {

constexpr uint32_t kBadOffsets = 1u, kBadTokens = 2u, kBadGroups = 4u, kBadSlots = 8u;

__global__ void check_clear_kernel(uint32_t *flag) { *flag = 0u; }

// Sub-bucket holding entry e: the last sb in [0, nsb) with off[sb] <= e.  Any
// offsets (even invalid ones) give an index in range.
__device__ __forceinline__ int find_subbucket(const int32_t *off, int nsb, int64_t e)
{
    int lo = 0, hi = nsb;  // answer in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)off[mid] <= e)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

// Group of sub-bucket sb (0 <= sb < num_subbuckets(K, topk)).
__device__ __forceinline__ int group_of(int sb, int K, int topk)
{
    int g = 0;
    while (g + 1 < K && group_base(g + 1, code_members(K, topk)) <= sb)
        ++g;
    return g;
}

// one block per head
__global__ __launch_bounds__(256) void check_offsets_kernel(const int32_t *__restrict__ offsets,
                                                            int nsb, int64_t E,
                                                            uint32_t *__restrict__ flag)
{
    const int32_t *off = offsets + (int64_t)blockIdx.x * (nsb + 1);
    bool bad = false;
    for (int i = threadIdx.x; i <= nsb; i += blockDim.x) {
        const int64_t v = off[i];
        bad |= v < 0 || v > E;
        bad |= (i == 0 && v != 0) || (i == nsb && v != E);
        bad |= i < nsb && (int64_t)off[i + 1] < v;
    }
    if (bad)
        atomicOr(flag, kBadOffsets);
}

// one thread per (head, entry)
__global__ __launch_bounds__(256) void check_entries_kernel(
    const uint32_t *__restrict__ gmask, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ tokens, int H, int64_t n, int K, int topk, int64_t E,
    uint32_t *__restrict__ flag)
{
    const int nsb = num_subbuckets(K, topk);
    const int64_t total = (int64_t)H * E;
    uint32_t bits = 0u;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t h = i / E, e = i % E;
        const int32_t *off = offsets + h * (nsb + 1);
        const int sb = find_subbucket(off, nsb, e);
        const int32_t t = tokens[i];
        if (t < 0 || (int64_t)t >= n) {
            bits |= kBadTokens;
            continue;
        }
        // the next entry of the same sub-bucket lies later in position
        const int64_t end = off[sb + 1];
        if (e + 1 < E && e + 1 < end && !(t < tokens[i + 1]))
            bits |= kBadTokens;
        const int g = group_of(sb, K, topk);
        const int cm = code_members(K, topk);
        const int code = sb - group_base(g, cm);
        const uint32_t m = gmask[h * n + t];
        const uint32_t lower = m & ((1u << g) - 1u);     // the token's groups below g
        const uint32_t rest = lower & (lower - 1u);       // ... without the lowest
        const uint32_t rest2 = rest & (rest - 1u);        // ... without the two lowest
        const int want = lower_code(g, lower ? __builtin_ctz(lower) : -1,
                                    rest ? __builtin_ctz(rest) : -1,
                                    (cm >= 3 && rest2) ? __builtin_ctz(rest2) : -1);
        if (!((m >> g) & 1u) || code != want)
            bits |= kBadGroups;
    }
    if (bits)
        atomicOr(flag, bits);
}

// one thread per (head, token)
__global__ __launch_bounds__(256) void check_slots_kernel(
    const uint32_t *__restrict__ gmask, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ tokens, const int32_t *__restrict__ slot_entry, int H,
    int64_t n, int K, int topk, uint32_t *__restrict__ flag)
{
    const int nsb = num_subbuckets(K, topk);
    const int64_t E = n * topk;
    const int64_t total = (int64_t)H * n;
    uint32_t bits = 0u;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t h = i / n, t = i % n;
        const uint32_t m = gmask[i];
        if (__builtin_popcount(m) != topk || (K < 32 && (m >> K) != 0u))
            bits |= kBadGroups;
        const int32_t *off = offsets + h * (nsb + 1);
        uint32_t seen = 0u;
        for (int s = 0; s < topk; ++s) {
            const int32_t e = slot_entry[i * topk + s];
            if (e < 0 || (int64_t)e >= E) {
                bits |= kBadSlots;
                continue;
            }
            if ((int64_t)tokens[h * E + e] != t)
                bits |= kBadSlots;
            seen |= 1u << group_of(find_subbucket(off, nsb, e), K, topk);
        }
        if (seen != m)
            bits |= kBadSlots;
    }
    if (bits)
        atomicOr(flag, bits);
}

int grid_for(int64_t items)
{
    return (int)std::min<int64_t>((items + 255) / 256, 16384);
}

}  // namespace

hipError_t launch_check_buckets(const uint32_t *gmask, const int32_t *offsets,
                                const int32_t *tokens, const int32_t *slot_entry, int H,
                                int64_t n, int K, int topk, void *ws, hipStream_t s,
                                uint32_t *found)
{
    uint32_t *flag = static_cast<uint32_t *>(ws);
    const int64_t E = n * topk;
    hipLaunchKernelGGL(check_clear_kernel, dim3(1), dim3(1), 0, s, flag);
    hipLaunchKernelGGL(check_offsets_kernel, dim3(H), dim3(256), 0, s, offsets,
                       num_subbuckets(K, topk), E, flag);
    hipLaunchKernelGGL(check_entries_kernel, dim3(grid_for((int64_t)H * E)), dim3(256), 0, s,
                       gmask, offsets, tokens, H, n, K, topk, E, flag);
    hipLaunchKernelGGL(check_slots_kernel, dim3(grid_for((int64_t)H * n)), dim3(256), 0, s,
                       gmask, offsets, tokens, slot_entry, H, n, K, topk, flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    e = hipMemcpyAsync(found, flag, sizeof(uint32_t), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess)
        return e;
    return hipStreamSynchronize(s);
}

}  // namespace focus
