// Focus attention forward: gathered within-group attention, sliding-window
// attention and the log-sum-exp merge.
//
// What is computed (gist.science Technical Summary, section 2, Gated
// Attention and Inference Efficiency (Top-k); jindou-blog: exact softmax in
// the local window and inside groups): for query i,
//     A(i) = { j <= i : i - j < w  or  G(i) and G(j) share a group }
// and O_i = softmax over A(i).  The pages run this as a local-window call plus
// a within-group causal call (Key Contributions 5).  Here every surviving pair
// is evaluated exactly once:
//   * window kernel: pairs with i - j < w, over original positions;
//   * group kernel : pairs with i - j >= w, inside the bucket of the lowest
//     group the two tokens share (the "owner"), one (O, LSE) partial per
//     (query, group) entry;
//   * the window kernel's epilogue merges its own part with the k partials of
//     the row by log-sum-exp.
//
// Kernel design (gfx950, CDNA4):
//   * 256 threads = 4 wavefronts; each wavefront owns 64 query rows as two
//     32-row blocks and holds Q in registers for the whole key loop.
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16 (fp32 inputs:
//     v_mfma_f32_32x32x2f32).  Computing the transposes puts one query per
//     lane column, so row max / row sum need one cross-half exchange per tile
//     and the P tile feeds the second product straight from registers.
//   * Key rows inside a 32-key block are permuted (sigma) so that lane half h,
//     register r of the S^T accumulator is key h*16 + r: the P fragment for
//     one 32x32x16 step is then 8 consecutive keys, matching one 16-byte read
//     of the V^T tile.
//   * K and V^T tiles of 64 keys are staged through LDS (XOR-swizzled, double
//     buffered, one barrier per tile).  Keys and values are first gathered
//     into bucket order (and V transposed) by a prepare pass, so every tile
//     load in the hot loop is contiguous.
//   * Grouped-query heads sharing a key/value head are packed into one block
//     (up to 4 heads x 64 rows), sharing every K/V tile and mask.
//   * Online softmax in the exp2 domain with lazy rescaling: the running max
//     is only moved when a tile raises it by more than 2^8.
#include <algorithm>
#include <cstring>

#include "common.hpp"

namespace focus {
namespace {

constexpr int kThreads = 512;  // 8 wavefronts, 2 per SIMD
constexpr int kRowsPerBlock = 256;  // 8 wavefronts x 32 query rows
constexpr int kKeyTile = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyRescale = 8.0f;
constexpr int kXcds = 8;

struct Params {
    int hq, hkv, ratio, hpb, nhg;  // ratio = hq/hkv; hpb heads per block; nhg = ratio/hpb
    int64_t n;
    int K, topk;
    int window;  // min(w, n)
    float c;     // scale * log2(e)
    const void *q;
    const void *kmat;  // row-major [hkv][krows][D]
    const void *vmat;  // bf16: [hkv][D][vcols] (transposed); fp32: [hkv][krows][D]
    int64_t krows, vcols;
    // group pass
    const int32_t *tokens;
    const int32_t *offsets;
    const uint32_t *gmask;
    const uint32_t *egm;  // gmask of each bucket entry's token, [hkv][E]
    const int4 *tiles;
    const int32_t *ntiles;
    int max_tiles;
    int64_t E;
    float *part_o;
    float *part_lse;
    // window pass
    const int32_t *slot_entry;
    int merge;
    void *out;
    float *lse;
    int row_tiles;
    int total_blocks;
};

// ---------------------------------------------------------------------------
// small helpers

__device__ __forceinline__ float swap_halves_max(float x)
{
    auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                               false);
    return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}

__device__ __forceinline__ float swap_halves_sum(float x)
{
    auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                               false);
    return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// Row of the 32x32 accumulator held by lane half h in register r (the MFMA
// output layout), and the key that row carries after the sigma permutation.
__device__ __forceinline__ int sigma(int m)
{
    return ((m >> 2) & 1) * 16 + (m & 3) + 4 * (m >> 3);
}

// Remap of a linear block index so that each XCD (blocks are dealt to the 8
// XCDs round-robin) walks one contiguous range of the work list: tiles of one
// head and group then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int total_padded)
{
    const int per = total_padded / kXcds;
    return (b % kXcds) * per + b / kXcds;
}

// ---------------------------------------------------------------------------
// per-dtype tile machinery: one 32-row query block per wavefront

template <int D, bool BF16>
struct Tile;

// bf16: K tile [64][D] and V^T tile [D][64] in LDS, both XOR-swizzled in
// 16-byte units so that the MFMA operand reads are free of bank conflicts.
template <int D>
struct Tile<D, true> {
    using T = __bf16;
    static constexpr int KS = D / 16;  // 32x32x16 steps over d
    static constexpr int DB = D / 32;  // 32-row blocks of d in O^T
    static constexpr int KCH = D / 8;  // 16-byte chunks per K row
    static constexpr int K_BYTES = kKeyTile * D * 2;
    static constexpr int V_BYTES = D * kKeyTile * 2;
    static constexpr int LOADS = (K_BYTES / 16) / kThreads;  // per thread, K and V each

    struct QFrag {
        bf16x8 v[KS];
    };
    struct Staged {};
    struct PFrag {  // probabilities as the B operand of O^T += V^T P^T
        bf16x8 v[2][2];
    };

    __device__ static int kswz(int row)
    {
        if (D == 128)
            return (row & 3) | (((row >> 4) & 1) << 2) | (((row >> 2) & 1) << 3);
        return ((row & 3) | (((row >> 4) & 1) << 2)) ^ ((row >> 2) & 1);
    }
    __device__ static int vswz(int d) { return (d & 7) ^ ((d >> 3) & 1); }
    __device__ static int kslot(int row, int c) { return row * KCH + (c ^ kswz(row)); }
    __device__ static int vslot(int d, int c) { return d * 8 + (c ^ vswz(d)); }

    __device__ static void load_q(QFrag &qf, const T *q, int64_t row_off, int h)
    {
        const bf16x8 *src = reinterpret_cast<const bf16x8 *>(q + row_off);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf.v[ks] = src[ks * 2 + h];
    }

    // Start the loads of one key tile straight into LDS: K rows row0.. of
    // kmat (clamped to its last row) and V^T columns row0.. of vmat.  Each
    // global_load_lds writes 64 consecutive 16-byte LDS slots (one per lane),
    // so every lane fetches the chunk that the swizzled layout keeps in its
    // slot.  Completion is awaited by the caller (vmcnt) before the barrier.
    __device__ static void prefetch(Staged &, const Params &p, int kvh, int64_t row0, char *kl,
                                    char *vl)
    {
        const T *km = static_cast<const T *>(p.kmat) + (int64_t)kvh * p.krows * D;
        const T *vm = static_cast<const T *>(p.vmat) + (int64_t)kvh * D * p.vcols;
        const int lane = threadIdx.x % kWave;
        const int wave = threadIdx.x / kWave;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int inst = wave * LOADS + i;
            const int P = inst * kWave + lane;
            const int row = P / KCH;
            const int c = (P % KCH) ^ kswz(row);
            int64_t gr = row0 + row;
            if (gr > p.krows - 1)
                gr = p.krows - 1;
            __builtin_amdgcn_global_load_lds(
                km + gr * D + c * 8, (__attribute__((address_space(3))) void *)(kl + inst * 1024),
                16, 0, 0);
            const int d = P / 8;
            const int vc = (P % 8) ^ vswz(d);
            __builtin_amdgcn_global_load_lds(
                vm + (int64_t)d * p.vcols + row0 + vc * 8,
                (__attribute__((address_space(3))) void *)(vl + inst * 1024), 16, 0, 0);
        }
    }
    __device__ static void land(const Staged &, char *, char *) {}

    // S^T[key][query] for the two 32-key blocks of the tile.
    __device__ static void qk(f32x16 (&s)[2], const QFrag &qf, const char *kl, int m, int h)
    {
        s[0] = f32x16{};
        s[1] = f32x16{};
        const int row0 = sigma(m), row1 = 32 + sigma(m);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a0 = reinterpret_cast<const bf16x8 *>(kl)[kslot(row0, ks * 2 + h)];
            const bf16x8 a1 = reinterpret_cast<const bf16x8 *>(kl)[kslot(row1, ks * 2 + h)];
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf.v[ks], s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf.v[ks], s[1], 0, 0, 0);
        }
    }

    // O^T[d][query] += V^T P^T.
    __device__ static void pv(f32x16 (&o)[DB], const PFrag &pf, const char *vl, int m, int h)
    {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bf16x8 a = reinterpret_cast<const bf16x8 *>(
                        vl)[vslot(db * 32 + m, kb * 4 + h * 2 + kk)];
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf.v[kb][kk], o[db], 0, 0, 0);
                }
    }

    // Exponentials of one tile -> bf16 P fragments; returns their fp32 sum.
    // (The sum is taken before rounding: near-uniform rows round their
    // probabilities the same way, and a sum of the rounded values would bias
    // the log-sum-exp by up to ~1e-3.)
    __device__ static float exp_tile(const f32x16 (&s)[2], float c, float mc, PFrag &pf)
    {
        float l0 = 0.f, l1 = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float p0 =
                        __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][kk * 8 + e], c, -mc));
                    const float p1 =
                        __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][kk * 8 + e + 1], c, -mc));
                    l0 += p0;
                    l1 += p1;
                    pf.v[kb][kk][e] = (__bf16)p0;
                    pf.v[kb][kk][e + 1] = (__bf16)p1;
                }
        return l0 + l1;
    }
};

// fp32: K tile [64][D+1] (padded rows), V tile [64][D] row-major; operands
// come one float per lane (32x32x2 steps).
template <int D>
struct Tile<D, false> {
    using T = float;
    static constexpr int KS = D / 2;
    static constexpr int DB = D / 32;
    static constexpr int KROW = D + 1;
    static constexpr int K_BYTES = kKeyTile * KROW * 4;
    static constexpr int V_BYTES = kKeyTile * D * 4;
    static constexpr int LOADS = (kKeyTile * D / 4) / kThreads;  // float4 per thread

    struct QFrag {
        float v[KS];
    };
    struct Staged {
        float4 k[LOADS];
        float4 v[LOADS];
    };
    struct PFrag {
        f32x16 s[2];
    };

    __device__ static void load_q(QFrag &qf, const T *q, int64_t row_off, int h)
    {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf.v[ks] = q[row_off + ks * 2 + h];
    }

    __device__ static void prefetch(Staged &st, const Params &p, int kvh, int64_t row0, char *,
                                    char *)
    {
        const T *km = static_cast<const T *>(p.kmat) + (int64_t)kvh * p.krows * D;
        const T *vm = static_cast<const T *>(p.vmat) + (int64_t)kvh * p.krows * D;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int ci = threadIdx.x + i * kThreads;
            const int row = ci / (D / 4), c = ci % (D / 4);
            int64_t gr = row0 + row;
            if (gr > p.krows - 1)
                gr = p.krows - 1;
            st.k[i] = *reinterpret_cast<const float4 *>(km + gr * D + c * 4);
            st.v[i] = *reinterpret_cast<const float4 *>(vm + gr * D + c * 4);
        }
    }

    __device__ static void land(const Staged &st, char *kl, char *vl)
    {
        float *kf = reinterpret_cast<float *>(kl);
        float *vf = reinterpret_cast<float *>(vl);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int ci = threadIdx.x + i * kThreads;
            const int row = ci / (D / 4), c = ci % (D / 4);
            kf[row * KROW + c * 4 + 0] = st.k[i].x;
            kf[row * KROW + c * 4 + 1] = st.k[i].y;
            kf[row * KROW + c * 4 + 2] = st.k[i].z;
            kf[row * KROW + c * 4 + 3] = st.k[i].w;
            reinterpret_cast<float4 *>(vf)[ci] = st.v[i];
        }
    }

    __device__ static void qk(f32x16 (&s)[2], const QFrag &qf, const char *kl, int m, int h)
    {
        const float *kf = reinterpret_cast<const float *>(kl);
        s[0] = f32x16{};
        s[1] = f32x16{};
        const float *k0 = kf + sigma(m) * KROW + h;
        const float *k1 = kf + (32 + sigma(m)) * KROW + h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(k0[ks * 2], qf.v[ks], s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(k1[ks * 2], qf.v[ks], s[1], 0, 0, 0);
        }
    }

    __device__ static void pv(f32x16 (&o)[DB], const PFrag &pf, const char *vl, int m, int h)
    {
        const float *vf = reinterpret_cast<const float *>(vl);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float *vrow = vf + (kb * 32 + h * 16 + r) * D + m;
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[db * 32], pf.s[kb][r], o[db],
                                                                 0, 0, 0);
            }
    }

    __device__ static float exp_tile(const f32x16 (&s)[2], float c, float mc, PFrag &pf)
    {
        float l = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));
                pf.s[kb][r] = pr;
                l += pr;
            }
        return l;
    }
};

// ---------------------------------------------------------------------------
// online softmax state of one wavefront: one query per lane column, both lane
// halves carry the same row statistics and half of each row's keys

template <class TL>
struct Acc {
    f32x16 o[TL::DB];
    float m;  // running max in the scaled log2 domain (may be -inf)
    float l;  // this lane half's partial row sum

    __device__ void init()
    {
#pragma unroll
        for (int db = 0; db < TL::DB; ++db)
            o[db] = f32x16{};
        m = -INFINITY;
        l = 0.f;
    }

    // Fold one tile of raw logits into the state; P receives the
    // probabilities for the PV product.
    __device__ void softmax(const f32x16 (&s)[2], float c, typename TL::PFrag &pf)
    {
        float t = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                t = fmaxf(t, s[kb][r]);
        const float mx = swap_halves_max(t) * c;
        // Lazy rescale: the running max only moves when a row's max grew by
        // more than 2^8, so P stays below 2^8 and O is rarely rescaled.
        if (__builtin_amdgcn_ballot_w64(mx > m + kLazyRescale) != 0) {
            const float m_new = fmaxf(m, mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m - m_use);
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < TL::DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    o[db][r] *= alpha;
        }
        const float mc = (m == -INFINITY) ? 0.f : m;
        l += TL::exp_tile(s, c, mc, pf);
    }
};

// ---------------------------------------------------------------------------
// the attention kernel: GROUP selects the gathered within-group pass

template <int D, bool BF16, bool GROUP>
__global__ __launch_bounds__(kThreads) void attn_kernel(Params p)
{
    using TL = Tile<D, BF16>;
    using T = typename TL::T;
    constexpr int DB = TL::DB;
    constexpr int STAGE = TL::K_BYTES + TL::V_BYTES + 2 * kKeyTile * 4;
    __shared__ __attribute__((aligned(16))) char smem0[STAGE];
    __shared__ __attribute__((aligned(16))) char smem1[STAGE];
    __shared__ int sub_start[kMaxGroups + 1];
    __shared__ int sub_count[kMaxGroups + 1];
    __shared__ int sub_owner[kMaxGroups + 1];

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int m = lane % 32;
    const int h = lane / 32;

    // ---- which work item this block owns
    const int b_lin = xcd_remap(blockIdx.x, gridDim.x);
    if (b_lin >= p.total_blocks)
        return;
    int kvh, hg, slot;
    if (GROUP) {
        slot = b_lin % p.max_tiles;
        const int rest = b_lin / p.max_tiles;
        hg = rest % p.nhg;
        kvh = rest / p.nhg;
        if (slot >= p.ntiles[kvh])
            return;
    } else {
        slot = b_lin % p.row_tiles;
        const int rest = b_lin / p.row_tiles;
        hg = rest % p.nhg;
        kvh = rest / p.nhg;
        slot = p.row_tiles - 1 - slot;  // late rows (most keys when w is large) first
    }
    const int rows_per_head = kRowsPerBlock / p.hpb;
    const int hsub = wave % p.hpb;
    const int wrow0 = (wave / p.hpb) * 32;  // first row of this wavefront in the tile
    const int hq = kvh * p.ratio + hg * p.hpb + hsub;

    // ---- rows of this block
    int g = 0, mq = 0, e_start = 0;
    int64_t p_start = 0;
    int tile_rows;
    if (GROUP) {
        const int4 t = p.tiles[(int64_t)kvh * p.max_tiles + slot];
        g = t.x / (p.K + 1);
        mq = t.x % (p.K + 1);
        e_start = t.y;
        tile_rows = t.z;
    } else {
        p_start = (int64_t)slot * rows_per_head;
        tile_rows = (int)min<int64_t>(rows_per_head, p.n - p_start);
    }
    const int32_t *tok = GROUP ? p.tokens + (int64_t)kvh * p.E : nullptr;
    const uint32_t *gmh = GROUP ? p.gmask + (int64_t)kvh * p.n : nullptr;

    // query row of this lane (column m of the wavefront's 32-row block)
    const int qr = wrow0 + m;
    const bool qvalid = qr < tile_rows;
    const int qpos = GROUP ? tok[e_start + (qvalid ? qr : 0)] : (int)(p_start + (qvalid ? qr : 0));
    const bool wave_active = wrow0 < tile_rows;
    const int wave_last_row = min(wrow0 + 31, tile_rows - 1);
    const int wq_min = GROUP ? tok[e_start + (wave_active ? wrow0 : 0)] : (int)(p_start + wrow0);
    const int wq_max = GROUP ? tok[e_start + (wave_active ? wave_last_row : 0)]
                             : (int)(p_start + wave_last_row);
    const int bq_max = GROUP ? tok[e_start + tile_rows - 1] : (int)(p_start + tile_rows - 1);

    typename TL::QFrag qf;
    TL::load_q(qf, static_cast<const T *>(p.q), ((int64_t)hq * p.n + qpos) * D, h);

    Acc<TL> acc;
    acc.init();

    // ---- key tile schedule
    const int w = p.window;
    uint32_t qlow = 0u;
    int64_t j_first = 0;
    int n_tiles_total = 0;
    if (GROUP) {
        qlow = gmh[qpos] & ((1u << g) - 1u);
        // wave 0 lanes find, per key sub-bucket, how many keys lie at or
        // before (last query position - w)
        if (wave == 0 && lane <= p.K) {
            const int mk = lane;
            const int sbk = g * (p.K + 1) + mk;
            const int32_t *offh = p.offsets + (int64_t)kvh * (num_subbuckets(p.K) + 1);
            const int lo0 = offh[sbk], hi0 = offh[sbk + 1];
            const bool skip = (p.topk >= 2) && (mk == mq) && (mq < g);
            int cnt = 0;
            if (!skip && hi0 > lo0) {
                const int64_t lim = (int64_t)bq_max - w;
                int lo = lo0, hi = hi0;  // first entry with position > lim
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if ((int64_t)tok[mid] <= lim)
                        lo = mid + 1;
                    else
                        hi = mid;
                }
                cnt = lo - lo0;
            }
            sub_start[mk] = lo0;
            sub_count[mk] = cnt;
            sub_owner[mk] = (p.topk >= 3) && (mq < g) && (mk < g) && (mk != mq);
        }
        __syncthreads();
        for (int i = 0; i <= p.K; ++i)
            n_tiles_total += (sub_count[i] + kKeyTile - 1) / kKeyTile;
        n_tiles_total = __builtin_amdgcn_readfirstlane(n_tiles_total);
    } else {
        const int64_t lo = max<int64_t>(0, p_start - w + 1);
        j_first = (lo / kKeyTile) * kKeyTile;
        const int64_t j_last = p_start + tile_rows - 1;
        n_tiles_total = (w > 0) ? (int)((j_last - j_first) / kKeyTile + 1) : 0;
    }

    // iterator over key tiles: (sub-bucket, tile) for the group pass
    int it_sub = 0, it_tile = 0;
    // (values read from LDS are block-uniform: keep them in scalar registers)
    auto uniform = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    auto tile_origin = [&](int &valid, int &owner) -> int64_t {
        if (GROUP) {
            while (it_tile * kKeyTile >= uniform(sub_count[it_sub])) {
                ++it_sub;
                it_tile = 0;
            }
            valid = min(kKeyTile, uniform(sub_count[it_sub]) - it_tile * kKeyTile);
            owner = uniform(sub_owner[it_sub]);
            return (int64_t)uniform(sub_start[it_sub]) + (int64_t)it_tile * kKeyTile;
        } else {
            valid = kKeyTile;
            owner = 0;
            return j_first + (int64_t)it_tile * kKeyTile;
        }
    };

    typename TL::Staged st;
    // Positions (and, where an owner test is needed, group bits) of a tile's
    // keys live next to its K and V^T data.  They are read from global
    // memory into registers when the tile's loads are issued and written to
    // LDS only after the current tile's compute: writing them at once would
    // make the wavefront wait for every load issued before them.
    const uint32_t *egh = GROUP ? p.egm + (int64_t)kvh * p.E : nullptr;
    auto load_keys = [&](int64_t origin, int valid, int owner, int &pos, uint32_t &gm) {
        pos = 0;
        gm = 0u;
        if (threadIdx.x < kKeyTile) {
            const int i = threadIdx.x;
            if (GROUP) {
                pos = i < valid ? tok[origin + i] : 0x7fffffff;
                gm = (i < valid && owner) ? egh[origin + i] : 0u;
            } else {
                pos = (int)(origin + i);
            }
        }
    };
    auto store_keys = [&](char *buf, int pos, uint32_t gm) {
        int *kpos = reinterpret_cast<int *>(buf + TL::K_BYTES + TL::V_BYTES);
        uint32_t *kgm = reinterpret_cast<uint32_t *>(kpos + kKeyTile);
        if (threadIdx.x < kKeyTile) {
            kpos[threadIdx.x] = pos;
            kgm[threadIdx.x] = gm;
        }
    };
    int cur_valid = 0, cur_owner = 0;
    if (n_tiles_total > 0) {
        const int64_t origin = tile_origin(cur_valid, cur_owner);
        int pos;
        uint32_t gm;
        load_keys(origin, cur_valid, cur_owner, pos, gm);
        TL::prefetch(st, p, kvh, origin, smem0, smem0 + TL::K_BYTES);
        TL::land(st, smem0, smem0 + TL::K_BYTES);
        store_keys(smem0, pos, gm);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // One key tile: compute on `cur` while the next tile streams into `nxt`.
    // The two LDS buffers are distinct arrays and the loop below is unrolled
    // by two, so each LDS read names one buffer and each LDS-DMA write the
    // other: the compiler can then see they do not overlap and does not wait
    // for the in-flight loads before reading the current tile.
    auto step = [&](int t, char *cur, char *nxt) {
        const int valid = cur_valid;
        const int owner = cur_owner;
        // start loading the next tile; it lands in the other buffer while
        // this one is computed
        const bool has_next = t + 1 < n_tiles_total;
        int nx_pos = 0;
        uint32_t nx_gm = 0u;
        if (has_next) {
            ++it_tile;
            const int64_t origin = tile_origin(cur_valid, cur_owner);
            load_keys(origin, cur_valid, cur_owner, nx_pos, nx_gm);
            TL::prefetch(st, p, kvh, origin, nxt, nxt + TL::K_BYTES);
        }

        const int *kpos = reinterpret_cast<const int *>(cur + TL::K_BYTES + TL::V_BYTES);
        const uint32_t *kgm = reinterpret_cast<const uint32_t *>(kpos + kKeyTile);
        // Every wavefront computes, including one whose rows all lie past a
        // ragged tile's end (its rows are masked and never stored): a branch
        // here would split the accumulator's live range and cost a register
        // copy of O per tile.
        {
            f32x16 s[2];
            TL::qk(s, qf, cur, m, h);
            // does any pair of this tile x wavefront need a mask?
            bool masked;
            if (GROUP) {
                const int last_key = kpos[valid - 1];
                masked = (valid < kKeyTile) || owner || ((int64_t)last_key > (int64_t)wq_min - w);
            } else {
                const int64_t j0 = kpos[0];
                masked = !((j0 + kKeyTile - 1 <= wq_min) && (j0 > (int64_t)wq_max - w));
            }
            if (masked) {
                // kgm holds zero unless this sub-bucket pair needs the owner
                // test, so the test below is a no-op elsewhere
                const int64_t lim = (int64_t)qpos - w;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int4 *kp4 = reinterpret_cast<const int4 *>(kpos + kb * 32 + h * 16);
                    const uint4 *kg4 = reinterpret_cast<const uint4 *>(kgm + kb * 32 + h * 16);
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int4 kp = kp4[r4];
                        const uint4 kg = kg4[r4];
                        const int kv[4] = {kp.x, kp.y, kp.z, kp.w};
                        const uint32_t kgv[4] = {kg.x, kg.y, kg.z, kg.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            bool keep;
                            if (GROUP)
                                keep = qvalid && ((int64_t)kv[e] <= lim) &&
                                       ((kgv[e] & qlow) == 0u);
                            else
                                keep = qvalid && (kv[e] <= qpos) && ((int64_t)kv[e] > lim);
                            s[kb][r4 * 4 + e] = keep ? s[kb][r4 * 4 + e] : -INFINITY;
                        }
                    }
                }
            }
            typename TL::PFrag pf;
            acc.softmax(s, p.c, pf);
            TL::pv(acc.o, pf, cur + TL::K_BYTES, m, h);
        }

        if (has_next) {
            TL::land(st, nxt, nxt + TL::K_BYTES);
            store_keys(nxt, nx_pos, nx_gm);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    for (int t = 0; t < n_tiles_total; t += 2) {
        step(t, smem0, smem1);
        if (t + 1 < n_tiles_total)
            step(t + 1, smem1, smem0);
    }

    if (!wave_active)
        return;

    // ---- epilogue
    const float l_tot = swap_halves_sum(acc.l);
    // log2-domain log-sum-exp of the scaled logits
    const float lse2 = (l_tot > 0.f) ? acc.m + __builtin_amdgcn_logf(l_tot) : -INFINITY;

    if (GROUP) {
        // normalised partial O (fp32) and natural-log LSE at the query's entry
        if (!qvalid)
            return;
        const int64_t e = e_start + qr;
        const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
        float *po = p.part_o + ((int64_t)hq * p.E + e) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                float4 v;
                v.x = acc.o[db][a * 4 + 0] * inv;
                v.y = acc.o[db][a * 4 + 1] * inv;
                v.z = acc.o[db][a * 4 + 2] * inv;
                v.w = acc.o[db][a * 4 + 3] * inv;
                *reinterpret_cast<float4 *>(po + db * 32 + a * 8 + h * 4) = v;
            }
        if (h == 0)
            p.part_lse[(int64_t)hq * p.E + e] = lse2 * kLn2;
        return;
    }

    // window pass: merge with the k group partials of the row, write O, LSE
    if (!qvalid)
        return;
    const int64_t i = qpos;
    const int ns = p.merge ? p.topk : 0;
    const int32_t *slots = p.slot_entry + ((int64_t)kvh * p.n + i) * p.topk;
    const float *plse = p.part_lse + (int64_t)hq * p.E;
    float M = lse2;
    for (int s_ = 0; s_ < ns; ++s_)
        M = fmaxf(M, plse[slots[s_]] * kLog2e);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    const float w_win = (l_tot > 0.f) ? __builtin_amdgcn_exp2f(lse2 - Mu) : 0.f;
    const float a_w = (l_tot > 0.f) ? w_win / l_tot : 0.f;
    float wsum = w_win;
    float res[DB][16];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            res[db][r] = acc.o[db][r] * a_w;
    for (int s_ = 0; s_ < ns; ++s_) {
        const int32_t ent = slots[s_];
        const float a_s = __builtin_amdgcn_exp2f(plse[ent] * kLog2e - Mu);
        if (a_s == 0.f)
            continue;
        wsum += a_s;
        const float *po = p.part_o + ((int64_t)hq * p.E + ent) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const float4 v = *reinterpret_cast<const float4 *>(po + db * 32 + a * 8 + h * 4);
                res[db][a * 4 + 0] += a_s * v.x;
                res[db][a * 4 + 1] += a_s * v.y;
                res[db][a * 4 + 2] += a_s * v.z;
                res[db][a * 4 + 3] += a_s * v.w;
            }
    }
    const float inv = (wsum > 0.f) ? 1.f / wsum : 0.f;
    T *orow = static_cast<T *>(p.out) + ((int64_t)hq * p.n + i) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            T *dst = orow + db * 32 + a * 8 + h * 4;
            if (BF16) {
                typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
                bf16x4 v;
                v[0] = (__bf16)(res[db][a * 4 + 0] * inv);
                v[1] = (__bf16)(res[db][a * 4 + 1] * inv);
                v[2] = (__bf16)(res[db][a * 4 + 2] * inv);
                v[3] = (__bf16)(res[db][a * 4 + 3] * inv);
                *reinterpret_cast<bf16x4 *>(dst) = v;
            } else {
                float4 v;
                v.x = res[db][a * 4 + 0] * inv;
                v.y = res[db][a * 4 + 1] * inv;
                v.z = res[db][a * 4 + 2] * inv;
                v.w = res[db][a * 4 + 3] * inv;
                *reinterpret_cast<float4 *>(dst) = v;
            }
        }
    if (h == 0)
        p.lse[(int64_t)hq * p.n + i] =
            (wsum > 0.f) ? (Mu + __builtin_amdgcn_logf(wsum)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// prepare: gather rows into bucket order (and transpose values for bf16)

// dst[h][row][:] = src[h][idx(row)][:] for row < rows (idx = tokens or
// identity), zero for rows in [rows, rows_pad).
template <typename T, int D>
__global__ __launch_bounds__(256) void gather_rows_kernel(const T *__restrict__ src,
                                                          const int32_t *__restrict__ tokens,
                                                          int64_t n, int64_t rows, int64_t rows_pad,
                                                          int H, T *__restrict__ dst)
{
    constexpr int CH = D * (int)sizeof(T) / 16;
    const int64_t total = (int64_t)H * rows_pad * CH;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(i % CH);
        const int64_t hr = i / CH;
        const int64_t row = hr % rows_pad;
        const int64_t h = hr / rows_pad;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < rows) {
            const int64_t srow = tokens ? tokens[h * rows + row] : row;
            v = reinterpret_cast<const uint4 *>(src + (h * n + srow) * D)[c];
        }
        reinterpret_cast<uint4 *>(dst + (h * rows_pad + row) * D)[c] = v;
    }
}

// bf16 transpose-gather: dst[h][d][col] = src[h][idx(col)][d] for col < cols,
// zero up to cols_pad.  One block per (head, 64-column tile).
template <int D>
__global__ __launch_bounds__(256) void gather_transpose_kernel(
    const __bf16 *__restrict__ src, const int32_t *__restrict__ tokens, int64_t n,
    int64_t cols, int64_t cols_pad, __bf16 *__restrict__ dst)
{
    __shared__ uint16_t tile[64][D + 8];
    const int h = blockIdx.y;
    const int64_t col0 = (int64_t)blockIdx.x * 64;
    constexpr int CH = D / 8;
    for (int i = threadIdx.x; i < 64 * CH; i += 256) {
        const int r = i / CH, c = i % CH;
        const int64_t col = col0 + r;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (col < cols) {
            const int64_t srow = tokens ? tokens[(int64_t)h * cols + col] : col;
            v = reinterpret_cast<const uint4 *>(src + ((int64_t)h * n + srow) * D)[c];
        }
        const uint16_t *pv = reinterpret_cast<const uint16_t *>(&v);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            tile[r][c * 8 + e] = pv[e];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < D * 8; i += 256) {
        const int d = i / 8, c = i % 8;
        uint16_t vals[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            vals[e] = tile[c * 8 + e][d];
        uint4 v;
        memcpy(&v, vals, 16);
        reinterpret_cast<uint4 *>(dst + ((int64_t)h * D + d) * cols_pad + col0)[c] = v;
    }
}

// egm[h][e] = gmask[h][tokens[h][e]]: the group bits of every bucket entry, in
// bucket order, so a tile's owner test reads them without a dependent load.
__global__ __launch_bounds__(256) void gather_gmask_kernel(const uint32_t *__restrict__ gmask,
                                                           const int32_t *__restrict__ tokens,
                                                           int64_t n, int64_t E, int H,
                                                           uint32_t *__restrict__ egm)
{
    const int64_t total = (int64_t)H * E;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t h = i / E;
        egm[i] = gmask[h * n + tokens[i]];
    }
}

// Tile list of the group pass: for routing head h, every sub-bucket cut into
// query tiles of `rows` entries, last tile (latest positions, most keys)
// first.  tiles[h][i] = {sub-bucket, first entry, entry count, 0}.
__global__ __launch_bounds__(256) void plan_kernel(const int32_t *__restrict__ offsets, int nsb,
                                                   int rows, int max_tiles,
                                                   int4 *__restrict__ tiles,
                                                   int32_t *__restrict__ ntiles)
{
    __shared__ int start[kMaxGroups * (kMaxGroups + 1) + 1];
    const int h = blockIdx.x;
    const int32_t *off = offsets + (int64_t)h * (nsb + 1);
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int sb = 0; sb < nsb; ++sb) {
            start[sb] = acc;
            acc += (off[sb + 1] - off[sb] + rows - 1) / rows;
        }
        start[nsb] = acc;
        ntiles[h] = acc;
    }
    __syncthreads();
    int4 *th = tiles + (int64_t)h * max_tiles;
    for (int sb = 0; sb < nsb; ++sb) {
        const int nt = start[sb + 1] - start[sb];
        const int cnt = off[sb + 1] - off[sb];
        for (int j = threadIdx.x; j < nt; j += blockDim.x) {
            const int jj = nt - 1 - j;
            th[start[sb] + j] = make_int4(sb, off[sb] + jj * rows, min(rows, cnt - jj * rows), 0);
        }
    }
}

// ---------------------------------------------------------------------------
// host side

struct Layout {
    int hpb, nhg, rows_group, max_tiles;
    int64_t E, e_pad, n_pad;
    size_t kb, vb, vt, egm, po, pl, tiles, ntiles, total;
};

int heads_per_block(int ratio)
{
    if (ratio % 4 == 0)
        return 4;
    if (ratio % 2 == 0)
        return 2;
    return 1;
}

Layout make_layout(const AttnShape &sh)
{
    Layout L{};
    const size_t es = sh.dt == FOCUS_BF16 ? 2 : 4;
    const int ratio = sh.hq / sh.hkv;
    L.hpb = heads_per_block(ratio);
    L.nhg = ratio / L.hpb;
    L.rows_group = kRowsPerBlock / L.hpb;
    L.E = sh.n * sh.topk;
    L.e_pad = (L.E + kKeyTile - 1) / kKeyTile * kKeyTile + kKeyTile;
    L.n_pad = (sh.n + kKeyTile - 1) / kKeyTile * kKeyTile + kKeyTile;
    L.max_tiles = (int)((L.E + L.rows_group - 1) / L.rows_group) + num_subbuckets(sh.K);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    L.kb = take((size_t)sh.hkv * L.e_pad * sh.d * es);
    L.vb = take((size_t)sh.hkv * L.e_pad * sh.d * es);
    L.vt = take(sh.dt == FOCUS_BF16 ? (size_t)sh.hkv * sh.d * L.n_pad * 2 : 0);
    L.egm = take((size_t)sh.hkv * L.E * 4);
    L.po = take((size_t)sh.hq * L.E * sh.d * 4);
    L.pl = take((size_t)sh.hq * L.E * 4);
    L.tiles = take((size_t)sh.hkv * L.max_tiles * sizeof(int4));
    L.ntiles = take((size_t)sh.hkv * sizeof(int32_t));
    L.total = off;
    return L;
}

template <int D, bool BF16, bool GROUP>
hipError_t launch_attn_kernel(const Params &p, hipStream_t s)
{
    const int grid = (p.total_blocks + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((attn_kernel<D, BF16, GROUP>), dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <bool GROUP>
hipError_t dispatch_attn(int d, bool bf16, const Params &p, hipStream_t s)
{
    if (bf16)
        return d == 64 ? launch_attn_kernel<64, true, GROUP>(p, s)
                       : launch_attn_kernel<128, true, GROUP>(p, s);
    return d == 64 ? launch_attn_kernel<64, false, GROUP>(p, s)
                   : launch_attn_kernel<128, false, GROUP>(p, s);
}

Params base_params(const AttnShape &sh, const Layout &L)
{
    Params p{};
    p.hq = sh.hq;
    p.hkv = sh.hkv;
    p.ratio = sh.hq / sh.hkv;
    p.hpb = L.hpb;
    p.nhg = L.nhg;
    p.n = sh.n;
    p.K = sh.K;
    p.topk = sh.topk;
    p.window = (int)std::min<int64_t>(sh.window, sh.n);
    p.c = sh.scale * kLog2e;
    p.E = L.E;
    return p;
}

template <typename T>
hipError_t launch_gather(int d, const T *src, const int32_t *tokens, int64_t n, int64_t rows,
                         int64_t rows_pad, int H, T *dst, hipStream_t s)
{
    const int64_t chunks = (int64_t)H * rows_pad * d * (int64_t)sizeof(T) / 16;
    const int blocks = (int)std::min<int64_t>((chunks + 255) / 256, 16384);
    if (d == 64)
        hipLaunchKernelGGL((gather_rows_kernel<T, 64>), dim3(blocks), dim3(256), 0, s, src, tokens,
                           n, rows, rows_pad, H, dst);
    else
        hipLaunchKernelGGL((gather_rows_kernel<T, 128>), dim3(blocks), dim3(256), 0, s, src,
                           tokens, n, rows, rows_pad, H, dst);
    return hipGetLastError();
}

hipError_t launch_transpose(int d, const __bf16 *src, const int32_t *tokens, int64_t n,
                            int64_t cols, int64_t cols_pad, int H, __bf16 *dst,
                            hipStream_t s)
{
    const dim3 grid((unsigned)(cols_pad / 64), (unsigned)H);
    if (d == 64)
        hipLaunchKernelGGL(gather_transpose_kernel<64>, grid, dim3(256), 0, s, src, tokens, n, cols,
                           cols_pad, dst);
    else
        hipLaunchKernelGGL(gather_transpose_kernel<128>, grid, dim3(256), 0, s, src, tokens, n,
                           cols, cols_pad, dst);
    return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(const AttnShape &sh) { return make_layout(sh).total; }

size_t dense_workspace_bytes(const AttnShape &sh)
{
    if (sh.dt != FOCUS_BF16)
        return 256;
    const int64_t n_pad = (sh.n + kKeyTile - 1) / kKeyTile * kKeyTile + kKeyTile;
    return align_up((size_t)sh.hkv * sh.d * n_pad * 2, 256);
}

hipError_t launch_attn(const AttnShape &sh, const void *q, const void *k, const void *v,
                       const uint32_t *gmask, const int32_t *offsets, const int32_t *tokens,
                       const int32_t *slot_entry, void *out, float *lse, void *ws, int parts,
                       hipStream_t s)
{
    const Layout L = make_layout(sh);
    char *w = static_cast<char *>(ws);
    const bool bf16 = sh.dt == FOCUS_BF16;
    int4 *tiles = reinterpret_cast<int4 *>(w + L.tiles);
    int32_t *ntiles = reinterpret_cast<int32_t *>(w + L.ntiles);
    hipError_t e = hipSuccess;

    if (parts & FOCUS_PART_PREPARE) {
        if (bf16) {
            auto K = static_cast<const __bf16 *>(k);
            auto V = static_cast<const __bf16 *>(v);
            e = launch_gather(sh.d, K, tokens, sh.n, L.E, L.e_pad, sh.hkv,
                              reinterpret_cast<__bf16 *>(w + L.kb), s);
            if (e == hipSuccess)
                e = launch_transpose(sh.d, V, tokens, sh.n, L.E, L.e_pad, sh.hkv,
                                     reinterpret_cast<__bf16 *>(w + L.vb), s);
            if (e == hipSuccess)
                e = launch_transpose(sh.d, V, nullptr, sh.n, sh.n, L.n_pad, sh.hkv,
                                     reinterpret_cast<__bf16 *>(w + L.vt), s);
        } else {
            auto K = static_cast<const float *>(k);
            auto V = static_cast<const float *>(v);
            e = launch_gather(sh.d, K, tokens, sh.n, L.E, L.e_pad, sh.hkv,
                              reinterpret_cast<float *>(w + L.kb), s);
            if (e == hipSuccess)
                e = launch_gather(sh.d, V, tokens, sh.n, L.E, L.e_pad, sh.hkv,
                                  reinterpret_cast<float *>(w + L.vb), s);
        }
        if (e != hipSuccess)
            return e;
        {
            const int64_t total = (int64_t)sh.hkv * L.E;
            const int blocks = (int)std::min<int64_t>((total + 255) / 256, 8192);
            hipLaunchKernelGGL(gather_gmask_kernel, dim3(blocks), dim3(256), 0, s, gmask, tokens,
                               sh.n, L.E, sh.hkv, reinterpret_cast<uint32_t *>(w + L.egm));
            e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
        hipLaunchKernelGGL(plan_kernel, dim3(sh.hkv), dim3(256), 0, s, offsets,
                           num_subbuckets(sh.K), L.rows_group, L.max_tiles, tiles, ntiles);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }

    Params p = base_params(sh, L);
    p.q = q;
    p.tokens = tokens;
    p.offsets = offsets;
    p.gmask = gmask;
    p.egm = reinterpret_cast<const uint32_t *>(w + L.egm);
    p.part_o = reinterpret_cast<float *>(w + L.po);
    p.part_lse = reinterpret_cast<float *>(w + L.pl);
    p.slot_entry = slot_entry;
    p.out = out;
    p.lse = lse;

    if (parts & FOCUS_PART_GROUP) {
        Params g = p;
        g.kmat = w + L.kb;
        g.vmat = w + L.vb;
        g.krows = L.e_pad;
        g.vcols = L.e_pad;
        g.tiles = tiles;
        g.ntiles = ntiles;
        g.max_tiles = L.max_tiles;
        g.total_blocks = sh.hkv * L.nhg * L.max_tiles;
        e = dispatch_attn<true>(sh.d, bf16, g, s);
        if (e != hipSuccess)
            return e;
    }
    if (parts & FOCUS_PART_WINDOW) {
        Params wp = p;
        wp.kmat = k;
        wp.vmat = bf16 ? (const void *)(w + L.vt) : v;
        wp.krows = sh.n;
        wp.vcols = L.n_pad;
        wp.merge = 1;
        wp.row_tiles = (int)((sh.n + (kRowsPerBlock / L.hpb) - 1) / (kRowsPerBlock / L.hpb));
        wp.total_blocks = sh.hkv * L.nhg * wp.row_tiles;
        e = dispatch_attn<false>(sh.d, bf16, wp, s);
    }
    return e;
}

hipError_t launch_dense(const AttnShape &sh, const void *q, const void *k, const void *v,
                        void *out, float *lse, void *ws, hipStream_t s)
{
    AttnShape d = sh;
    d.window = sh.n;
    d.K = 1;
    d.topk = 1;
    Layout L = make_layout(d);
    const bool bf16 = sh.dt == FOCUS_BF16;
    const int64_t n_pad = (sh.n + kKeyTile - 1) / kKeyTile * kKeyTile + kKeyTile;
    hipError_t e = hipSuccess;
    if (bf16) {
        e = launch_transpose(sh.d, static_cast<const __bf16 *>(v), nullptr, sh.n, sh.n,
                             n_pad, sh.hkv, static_cast<__bf16 *>(ws), s);
        if (e != hipSuccess)
            return e;
    }
    Params p = base_params(d, L);
    p.q = q;
    p.kmat = k;
    p.vmat = bf16 ? ws : v;
    p.krows = sh.n;
    p.vcols = n_pad;
    p.merge = 0;
    p.out = out;
    p.lse = lse;
    p.row_tiles = (int)((sh.n + (kRowsPerBlock / L.hpb) - 1) / (kRowsPerBlock / L.hpb));
    p.total_blocks = sh.hkv * L.nhg * p.row_tiles;
    return dispatch_attn<false>(sh.d, bf16, p, s);
}

}  // namespace focus
