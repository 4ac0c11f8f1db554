// Focus attention backward: gradients of the exact softmax over A(i) with
// respect to q, k and v, for the hard set (no gradient reaches the routing).
//
// What is differentiated: the forward of attn.hip (gist.science Technical
// Summary, section 2, Gated Attention and Inference Efficiency (Top-k)),
//     A(i) = { j <= i : i - j < w  or  G(i) and G(j) share a group },
// O_i = sum_{j in A(i)} P_ij v_j with P_ij = exp(s_ij - L_i), s_ij =
// scale q_i.k_j.  Training and fine-tuning through Focus (thelatestinai.com
// Table 5, all parameters fine-tuned; Technical Summary, from-scratch
// training) need these gradients.  With D_i = dO_i . O_i, dP_ij = dO_i . v_j
// and dS_ij = P_ij (dP_ij - D_i):
//     dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
//     dv_j = sum_i P_ij dO_i,
// the sums over i running over every query head that reads the key/value
// head.  L_i is the forward's log-sum-exp, so P_ij needs no second softmax.
//
// Every pair contributes independently once L_i and D_i are known, so the
// forward's partition carries over: pairs with i - j < w go to the window
// kernels, the others to the group kernels of the lowest group the two tokens
// share.  Two passes per partition, neither with atomics:
//   * dq pass (query-major, like the forward): a block owns 128 query rows
//     and walks their key tiles; S^T = K Q^T and dP^T = V dO^T put one query
//     per lane column, dS^T feeds dq^T += K^T dS^T from registers.
//   * dk/dv pass (key-major): a block owns 128 keys with K and V in
//     registers and walks the query tiles that see them, for every query head
//     of the key/value head; S = Q K^T and dP = dO V^T put one key per lane
//     column, P and dS feed dv^T += dO^T P and dk^T += Q^T dS.
// Each pass writes fp32 partials (per position for the window, per bucket
// entry for the groups); a merge kernel adds a row's window part and its k
// group parts and rounds to bf16.
//
// Operands on v_mfma_f32_32x32x16_bf16 need both fragments contiguous along
// the reduction index.  Tiles are staged through LDS by plain loads; the
// transposed operands (K^T in the dq pass, Q^T and dO^T in the dk/dv pass)
// are written transposed into LDS at staging time, so no transposed copy is
// kept in HBM.  The group passes read rows through the bucket's token list.
#include <algorithm>

#include "attn_common.hpp"

namespace focus {
namespace {
using namespace attn;

constexpr int kBwdThreads = 256;  // 4 wavefronts
constexpr int kBwdRows = 128;     // query rows (dq pass) or keys (dk/dv pass) per block
constexpr int kQKeys = 64;        // dq pass: keys per staged tile
constexpr int kKQueries = 32;     // dk/dv pass: queries per staged tile
constexpr int kNoPos = 0x7fffffff;

struct BwdParams {
    int hq, hkv, ratio, K, topk, window;
    int64_t n, E;
    float c;      // scale * log2(e)
    float scale;
    const __bf16 *q, *k, *v, *dout;
    const float *lse;
    const float *drow;  // D_i = dO_i . O_i, [hq][n]
    // group pass
    const int32_t *tokens;   // [hkv][E]
    const int32_t *offsets;  // [hkv][K(K+1)+1]
    const uint32_t *gmask;   // [hkv][n]
    const int4 *tiles;       // [hkv][max_tiles]: (sub-bucket, first entry, rows)
    const int32_t *ntiles;
    int max_tiles;
    int row_tiles;  // window: 128-row tiles per head
    // outputs (fp32 partials): rows are positions (window) or entries (group)
    float *dq;      // [hq][rows][D]
    float *dk, *dv; // [hkv][rows][D]
};

// XOR swizzles of 16-byte LDS slots.  Row-major tiles ([rows][D], read as
// A fragments row sigma(m), chunk 2ks+h) and transposed tiles ([D][cols],
// read row d, chunk c) are laid out so that the 8 lanes served together read
// distinct banks.
template <int D>
__device__ __forceinline__ int rswz(int row)
{
    if (D == 128)
        return (row & 3) | (((row >> 4) & 1) << 2) | (((row >> 2) & 1) << 3);
    return ((row & 3) | (((row >> 4) & 1) << 2)) ^ ((row >> 2) & 1);
}
template <int D>
__device__ __forceinline__ int rslot(int row, int c)  // row-major [rows][D]
{
    return row * (D / 8) + (c ^ rswz<D>(row));
}
// transposed tile with CH 16-byte chunks per row
template <int CH>
__device__ __forceinline__ int tslot(int d, int c)
{
    if (CH == 8)
        return d * 8 + (c ^ ((d & 7) ^ ((d >> 3) & 1)));
    return d * 4 + (c ^ ((d >> 2) & 3));  // CH == 4
}

__device__ __forceinline__ bf16x8 lds16(const char *base, int slot)
{
    return *reinterpret_cast<const bf16x8 *>(base + slot * 16);
}

// fp32 accumulator registers 8t .. 8t+7 as one bf16 B fragment
__device__ __forceinline__ bf16x8 pack8(const f32x16 &x, int t)
{
    bf16x8 r;
#pragma unroll
    for (int u = 0; u < 8; ++u)
        r[u] = (__bf16)x[8 * t + u];
    return r;
}

// Stores one chunk (8 values of row `row`, columns 8c..8c+7) transposed into
// a [D][cols] tile with CH chunks per row.
template <int CH>
__device__ __forceinline__ void store_transposed(char *tl, const uint4 &v, int row, int c)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const int kc = row >> 3, ke = row & 7;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int d = 8 * c + u;
        const uint16_t bits = (uint16_t)((u & 1) ? (w[u >> 1] >> 16) : (w[u >> 1] & 0xffffu));
        *reinterpret_cast<uint16_t *>(tl + tslot<CH>(d, kc) * 16 + ke * 2) = bits;
    }
}

// ---------------------------------------------------------------------------
// dq pass

template <int D, bool GROUP>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dq_kernel(BwdParams p)
{
    constexpr int KS = D / 16;   // k-steps over d
    constexpr int DB = D / 32;   // 32-row blocks of d
    constexpr int KCH = D / 8;   // 16-byte chunks per row
    constexpr int CHUNKS = kQKeys * KCH / kBwdThreads;  // per thread per matrix
    __shared__ __attribute__((aligned(16))) char k_lds[kQKeys * D * 2];
    __shared__ __attribute__((aligned(16))) char v_lds[kQKeys * D * 2];
    __shared__ __attribute__((aligned(16))) char kt_lds[D * kQKeys * 2];
    __shared__ int kpos_lds[kQKeys];
    __shared__ uint32_t kgm_lds[kQKeys];
    __shared__ int sub_start[kMaxGroups + 1], sub_count[kMaxGroups + 1], sub_owner[kMaxGroups + 1];

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int m = lane % 32;
    const int h = lane / 32;

    // ---- work item: (query head, tile)
    int hq, kvh, slot;
    if (GROUP) {
        slot = blockIdx.x % p.max_tiles;
        hq = blockIdx.x / p.max_tiles;
        kvh = hq / p.ratio;
        if (slot >= p.ntiles[kvh])
            return;
    } else {
        slot = blockIdx.x % p.row_tiles;
        hq = blockIdx.x / p.row_tiles;
        kvh = hq / p.ratio;
    }
    int g = 0, mq = 0, e_start = 0, tile_rows;
    int64_t p_start = 0;
    if (GROUP) {
        const int4 t = p.tiles[(int64_t)kvh * p.max_tiles + slot];
        g = t.x / (p.K + 1);
        mq = t.x % (p.K + 1);
        e_start = t.y;
        tile_rows = t.z;
    } else {
        p_start = (int64_t)slot * kBwdRows;
        tile_rows = (int)std::min<int64_t>(kBwdRows, p.n - p_start);
    }
    const int32_t *tok = GROUP ? p.tokens + (int64_t)kvh * p.E : nullptr;
    const uint32_t *gmh = p.gmask + (int64_t)kvh * p.n;

    // ---- this lane's query (column m of the wavefront's 32 rows)
    const int qr = wave * 32 + m;
    const bool qvalid = qr < tile_rows;
    const int qrc = qvalid ? qr : 0;
    const int qpos = GROUP ? tok[e_start + qrc] : (int)(p_start + qrc);
    const int64_t qrow = (int64_t)hq * p.n + qpos;
    bf16x8 qf[KS], dof[KS];
    {
        const bf16x8 *qs = reinterpret_cast<const bf16x8 *>(p.q + qrow * D);
        const bf16x8 *ds = reinterpret_cast<const bf16x8 *>(p.dout + qrow * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qf[ks] = qs[ks * 2 + h];
            dof[ks] = ds[ks * 2 + h];
        }
    }
    const float l2 = p.lse[qrow] * kLog2e;
    const float dq_d = p.drow[qrow];
    const uint32_t qgm = gmh[qpos];
    const int w = p.window;

    // ---- key tiles
    int n_tiles = 0;
    int64_t j_first = 0;
    if (GROUP) {
        const int bq_max = tok[e_start + tile_rows - 1];
        if (threadIdx.x <= p.K) {
            const int mk = threadIdx.x;
            const int sbk = g * (p.K + 1) + mk;
            const int32_t *offh = p.offsets + (int64_t)kvh * (num_subbuckets(p.K) + 1);
            const int lo0 = offh[sbk], hi0 = offh[sbk + 1];
            const bool skip = (p.topk >= 2) && (mk == mq) && (mq < g);
            int cnt = 0;
            if (!skip && hi0 > lo0) {
                const int64_t lim = (int64_t)bq_max - w;  // keys at or before lim
                int lo = lo0, hi = hi0;
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
            n_tiles += (sub_count[i] + kQKeys - 1) / kQKeys;
    } else if (w > 0) {
        const int64_t lo = std::max<int64_t>(0, p_start - w + 1);
        j_first = (lo / kQKeys) * kQKeys;
        const int64_t j_last = p_start + tile_rows - 1;
        n_tiles = (int)((j_last - j_first) / kQKeys + 1);
    }
    n_tiles = __builtin_amdgcn_readfirstlane(n_tiles);

    int it_sub = 0, it_tile = 0;
    // origin, valid key count and owner flag of the next tile, in order
    struct TileDesc {
        int64_t origin;
        int valid, owner;
    };
    auto next_tile = [&]() -> TileDesc {
        TileDesc t;
        if (GROUP) {
            while (it_tile * kQKeys >= sub_count[it_sub]) {
                ++it_sub;
                it_tile = 0;
            }
            t.valid = std::min(kQKeys, sub_count[it_sub] - it_tile * kQKeys);
            t.owner = sub_owner[it_sub];
            t.origin = (int64_t)sub_start[it_sub] + (int64_t)it_tile * kQKeys;
        } else {
            t.origin = j_first + (int64_t)it_tile * kQKeys;
            t.valid = (int)std::min<int64_t>(kQKeys, p.n - t.origin);
            t.owner = 0;
        }
        ++it_tile;
        return t;
    };

    // Staging: thread t stages key row (t % 64) of a tile, chunks c = 4 i + t / 64 of
    // its K and V rows.  The key's position (a bucket lookup in the group pass)
    // is fetched one tile ahead of its rows, so no load waits on another in
    // the loop.
    const int srow = threadIdx.x % kQKeys;
    const int sc0 = threadIdx.x / kQKeys;
    auto key_pos = [&](const TileDesc &t) -> int {
        const int r = std::min(srow, t.valid - 1);
        return GROUP ? tok[t.origin + r] : (int)(t.origin + r);
    };
    // (rows past the tile's end load a valid row and are zeroed when they
    // land, so that no load has to complete before the next is issued)
    uint4 kr[CHUNKS], vr[CHUNKS];
    int kp = kNoPos;
    uint32_t kg = 0;
    auto fetch = [&](const TileDesc &t, int pos) {
        const int64_t base = ((int64_t)kvh * p.n + pos) * D;
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int c = 4 * i + sc0;
            kr[i] = *reinterpret_cast<const uint4 *>(p.k + base + c * 8);
            vr[i] = *reinterpret_cast<const uint4 *>(p.v + base + c * 8);
        }
        kg = gmh[pos];
        kp = srow < t.valid ? pos : kNoPos;
    };
    auto land = [&]() {
        const bool ok = kp != kNoPos;
        const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int c = 4 * i + sc0;
            const uint4 kx = ok ? kr[i] : z, vx = ok ? vr[i] : z;
            *reinterpret_cast<uint4 *>(k_lds + rslot<D>(srow, c) * 16) = kx;
            *reinterpret_cast<uint4 *>(v_lds + rslot<D>(srow, c) * 16) = vx;
            store_transposed<kQKeys / 8>(kt_lds, kx, srow, c);
        }
        if (threadIdx.x < kQKeys) {
            kpos_lds[srow] = kp;
            kgm_lds[srow] = kp == kNoPos ? 0u : kg;
        }
    };

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[db][r] = 0.f;

    const uint32_t low = GROUP ? ((1u << g) - 1u) : 0u;
    // tiles it (rows in registers), it + 1 (position known), it + 2
    // Tile it's rows sit in registers while tile it+1's position is known;
    // past the last tile the descriptors repeat it, so every load in the
    // loop is unconditional (no register copy of a load in flight).
    TileDesc t_cur{}, t_next{};
    int pos_next = 0;
    if (n_tiles > 0) {
        t_cur = next_tile();
        const int pos0 = key_pos(t_cur);
        t_next = n_tiles > 1 ? next_tile() : t_cur;
        pos_next = key_pos(t_next);
        fetch(t_cur, pos0);
    }
    // per-lane LDS slots of the MFMA A fragments: K and V rows (row sigma(m)
    // of each 32-key block, chunk 2ks+h; the second block is 32 rows on) and
    // K^T (row db*32+m, chunk 4kb+2h+t; later row blocks are 256 slots on)
    int koff[KS], ktoff[4];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        koff[ks] = rslot<D>(sigma(m), 2 * ks + h);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        ktoff[j] = tslot<kQKeys / 8>(m, 4 * (j >> 1) + 2 * h + (j & 1));

    for (int it = 0; it < n_tiles; ++it) {
        __syncthreads();
        land();
        const int owner = __builtin_amdgcn_readfirstlane(t_cur.owner);
        const int valid = __builtin_amdgcn_readfirstlane(t_cur.valid);
        const int origin = __builtin_amdgcn_readfirstlane((int)t_cur.origin);
        __syncthreads();
        fetch(t_next, pos_next);
        t_cur = t_next;
        if (it + 2 < n_tiles)
            t_next = next_tile();
        pos_next = key_pos(t_next);

        // The keys this lane's query takes form one interval [klo, khi] of
        // the tile: in the window pass positions origin + kk with
        // 0 <= qpos - kpos < w; in the group pass the keys ascend and the
        // far ones (kpos <= qpos - w) are a prefix.
        int klo = 0, khi = -1;
        if (qvalid) {
            if (GROUP) {
                const int lim = qpos - w;
                if (lim >= kpos_lds[valid - 1]) {
                    khi = valid - 1;
                } else {
                    int lo = 0, hi = valid;
                    while (lo < hi) {
                        const int mid = (lo + hi) >> 1;
                        if (kpos_lds[mid] <= lim)
                            lo = mid + 1;
                        else
                            hi = mid;
                    }
                    khi = lo - 1;
                }
            } else {
                klo = std::max(0, qpos - origin - w + 1);
                khi = std::min(qpos - origin, valid - 1);
            }
        }
        const bool full = !owner && __builtin_amdgcn_ballot_w64(!(klo <= 0 && khi >= kQKeys - 1)) == 0;

        // S^T and dP^T for the two 32-key blocks.  LDS fragments are read a
        // block ahead: block 1's between block 0's MFMAs (into the same
        // registers), K^T's between block 1's; the fences keep that order.
        f32x16 s[2], dp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[kb][r] = dp[kb][r] = 0.f;
        bf16x8 fa[KS], fb[KS], ktf[DB][4];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            fa[ks] = lds16(k_lds, koff[ks]);
            fb[ks] = lds16(v_lds, koff[ks]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks], qf[ks], s[0], 0, 0, 0);
            dp[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks], dof[ks], dp[0], 0, 0, 0);
            fa[ks] = lds16(k_lds, koff[ks] + 32 * KCH);
            fb[ks] = lds16(v_lds, koff[ks] + 32 * KCH);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks], qf[ks], s[1], 0, 0, 0);
            dp[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks], dof[ks], dp[1], 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4 * DB / KS; ++q) {
                const int f = ks * (4 * DB / KS) + q;
                ktf[f / 4][f % 4] = lds16(kt_lds, ktoff[f % 4] + (f / 4) * 32 * (kQKeys / 8));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // dS^T = P^T (dP^T - D) as bf16 B fragments
        bf16x8 dsf[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float pr = __builtin_amdgcn_exp2f(s[kb][r] * p.c - l2);
                if (!full) {
                    const int kk = kb * 32 + 16 * h + r;
                    bool ok = kk >= klo && kk <= khi;
                    if (GROUP && owner)
                        ok = ok && ((qgm & kgm_lds[kk] & low) == 0u);
                    pr = ok ? pr : 0.f;
                }
                s[kb][r] = pr * (dp[kb][r] - dq_d);
            }
            dsf[kb][0] = pack8(s[kb], 0);
            dsf[kb][1] = pack8(s[kb], 1);
        }
        // dq^T += K^T dS^T
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktf[db][j], dsf[j >> 1][j & 1],
                                                                 acc[db], 0, 0, 0);
    }

    // ---- store: lane (m, h), register r of block db holds dq[query m][d]
    if (qvalid) {
        const int64_t row = GROUP ? (int64_t)e_start + qr : p_start + qr;
        const int64_t rows = GROUP ? p.E : p.n;
        float *dst = p.dq + ((int64_t)hq * rows + row) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<float4 *>(dst + db * 32 + 8 * j + 4 * h) =
                    make_float4(acc[db][4 * j] * p.scale, acc[db][4 * j + 1] * p.scale,
                                acc[db][4 * j + 2] * p.scale, acc[db][4 * j + 3] * p.scale);
    }
}

// ---------------------------------------------------------------------------
// dk/dv pass

template <int D, bool GROUP>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkv_kernel(BwdParams p)
{
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int KCH = D / 8;
    constexpr int CHUNKS = kKQueries * KCH / kBwdThreads;  // per thread per matrix
    __shared__ __attribute__((aligned(16))) char q_lds[kKQueries * D * 2];
    __shared__ __attribute__((aligned(16))) char do_lds[kKQueries * D * 2];
    __shared__ __attribute__((aligned(16))) char qt_lds[D * kKQueries * 2];
    __shared__ __attribute__((aligned(16))) char dot_lds[D * kKQueries * 2];
    __shared__ int qpos_lds[kKQueries];
    __shared__ __attribute__((aligned(16))) float ql2_lds[kKQueries];
    __shared__ __attribute__((aligned(16))) float qd_lds[kKQueries];
    __shared__ uint32_t qgm_lds[kKQueries];
    __shared__ int sub_start[kMaxGroups + 1], sub_count[kMaxGroups + 1], sub_owner[kMaxGroups + 1];

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int m = lane % 32;
    const int h = lane / 32;

    // ---- work item: (key/value head, tile of 128 keys)
    int kvh, slot;
    if (GROUP) {
        slot = blockIdx.x % p.max_tiles;
        kvh = blockIdx.x / p.max_tiles;
        if (slot >= p.ntiles[kvh])
            return;
    } else {
        slot = blockIdx.x % p.row_tiles;
        kvh = blockIdx.x / p.row_tiles;
    }
    int g = 0, mk = 0, e_start = 0, tile_keys;
    int64_t p_start = 0;
    if (GROUP) {
        const int4 t = p.tiles[(int64_t)kvh * p.max_tiles + slot];
        g = t.x / (p.K + 1);
        mk = t.x % (p.K + 1);
        e_start = t.y;
        tile_keys = t.z;
    } else {
        p_start = (int64_t)slot * kBwdRows;
        tile_keys = (int)std::min<int64_t>(kBwdRows, p.n - p_start);
    }
    const int32_t *tok = GROUP ? p.tokens + (int64_t)kvh * p.E : nullptr;
    const uint32_t *gmh = p.gmask + (int64_t)kvh * p.n;

    // ---- this lane's key (column m of the wavefront's 32 keys)
    const int kr = wave * 32 + m;
    const bool kvalid = kr < tile_keys;
    const int krc = kvalid ? kr : 0;
    const int kpos = GROUP ? tok[e_start + krc] : (int)(p_start + krc);
    bf16x8 kf[KS], vf[KS];
    {
        const int64_t row = (int64_t)kvh * p.n + kpos;
        const bf16x8 *ks_ = reinterpret_cast<const bf16x8 *>(p.k + row * D);
        const bf16x8 *vs_ = reinterpret_cast<const bf16x8 *>(p.v + row * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kf[ks] = ks_[ks * 2 + h];
            vf[ks] = vs_[ks * 2 + h];
        }
    }
    const uint32_t kgm = gmh[kpos];
    const int w = p.window;

    // ---- query tiles, per query head
    int tiles_per_head = 0;
    int64_t i_first = 0;
    if (GROUP) {
        const int bk_min = tok[e_start];  // keys ascend inside the sub-bucket
        if (threadIdx.x <= p.K) {
            const int mq = threadIdx.x;
            const int sbq = g * (p.K + 1) + mq;
            const int32_t *offh = p.offsets + (int64_t)kvh * (num_subbuckets(p.K) + 1);
            const int lo0 = offh[sbq], hi0 = offh[sbq + 1];
            const bool skip = (p.topk >= 2) && (mq == mk) && (mk < g);
            int first = hi0;
            if (!skip && hi0 > lo0) {
                const int64_t lim = (int64_t)bk_min + w;  // queries at or after lim
                int lo = lo0, hi = hi0;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if ((int64_t)tok[mid] < lim)
                        lo = mid + 1;
                    else
                        hi = mid;
                }
                first = lo;
            }
            sub_start[mq] = first;
            sub_count[mq] = hi0 - first;
            sub_owner[mq] = (p.topk >= 3) && (mq < g) && (mk < g) && (mk != mq);
        }
        __syncthreads();
        for (int i = 0; i <= p.K; ++i)
            tiles_per_head += (sub_count[i] + kKQueries - 1) / kKQueries;
    } else if (w > 0) {
        i_first = p_start;
        const int64_t i_last = std::min<int64_t>(p.n - 1, p_start + tile_keys - 1 + w - 1);
        tiles_per_head = (int)((i_last - i_first) / kKQueries + 1);
    }
    tiles_per_head = __builtin_amdgcn_readfirstlane(tiles_per_head);
    const int n_tiles = tiles_per_head * p.ratio;

    int it_head = 0, it_sub = 0, it_tile = 0, it_count = 0;
    struct TileDesc {
        int64_t origin;
        int valid, owner, head;
    };
    auto next_tile = [&]() -> TileDesc {
        if (it_count == tiles_per_head) {  // next query head
            ++it_head;
            it_sub = 0;
            it_tile = 0;
            it_count = 0;
        }
        ++it_count;
        TileDesc t;
        t.head = kvh * p.ratio + it_head;
        if (GROUP) {
            while (it_tile * kKQueries >= sub_count[it_sub]) {
                ++it_sub;
                it_tile = 0;
            }
            t.valid = std::min(kKQueries, sub_count[it_sub] - it_tile * kKQueries);
            t.owner = sub_owner[it_sub];
            t.origin = (int64_t)sub_start[it_sub] + (int64_t)it_tile * kKQueries;
        } else {
            t.origin = i_first + (int64_t)it_tile * kKQueries;
            t.valid = (int)std::min<int64_t>(kKQueries, p.n - t.origin);
            t.owner = 0;
        }
        ++it_tile;
        return t;
    };

    // Staging: thread t stages query row (t % 32), chunks c = 8 i + t / 32 of
    // its Q and dO rows, and (t < 32) the row's position, log2-domain LSE, D
    // and group bits.  Positions are fetched one tile ahead of the rows.
    const int srow = threadIdx.x % kKQueries;
    const int sc0 = threadIdx.x / kKQueries;
    auto query_pos = [&](const TileDesc &t) -> int {
        const int r = std::min(srow, t.valid - 1);
        return GROUP ? tok[t.origin + r] : (int)(t.origin + r);
    };
    uint4 qr_[CHUNKS], dr_[CHUNKS];
    int qp = kNoPos;
    float ql2 = 0.f, qd = 0.f;
    uint32_t qg = 0;
    auto fetch = [&](const TileDesc &t, int pos) {
        const int64_t qrow = (int64_t)t.head * p.n + pos;
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int c = 8 * i + sc0;
            qr_[i] = *reinterpret_cast<const uint4 *>(p.q + qrow * D + c * 8);
            dr_[i] = *reinterpret_cast<const uint4 *>(p.dout + qrow * D + c * 8);
        }
        ql2 = p.lse[qrow] * kLog2e;
        qd = p.drow[qrow];
        qg = gmh[pos];
        qp = srow < t.valid ? pos : kNoPos;
    };
    auto land = [&]() {
        const bool ok = qp != kNoPos;
        const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int c = 8 * i + sc0;
            const uint4 qx = ok ? qr_[i] : z, dx = ok ? dr_[i] : z;
            *reinterpret_cast<uint4 *>(q_lds + rslot<D>(srow, c) * 16) = qx;
            *reinterpret_cast<uint4 *>(do_lds + rslot<D>(srow, c) * 16) = dx;
            store_transposed<kKQueries / 8>(qt_lds, qx, srow, c);
            store_transposed<kKQueries / 8>(dot_lds, dx, srow, c);
        }
        if (threadIdx.x < kKQueries) {
            qpos_lds[srow] = qp;
            ql2_lds[srow] = ok ? ql2 : 0.f;
            qd_lds[srow] = ok ? qd : 0.f;
            qgm_lds[srow] = ok ? qg : 0u;
        }
    };

    f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dk_acc[db][r] = dv_acc[db][r] = 0.f;

    const uint32_t low = GROUP ? ((1u << g) - 1u) : 0u;
    TileDesc t_cur{}, t_next{};
    int pos_next = 0;
    if (n_tiles > 0) {
        t_cur = next_tile();
        const int pos0 = query_pos(t_cur);
        t_next = n_tiles > 1 ? next_tile() : t_cur;
        pos_next = query_pos(t_next);
        fetch(t_cur, pos0);
    }
    // per-lane LDS slots: Q and dO rows (row sigma(m), chunk 2ks+h) and
    // Q^T / dO^T (row db*32+m, chunk 2h+t; later row blocks 128 slots on)
    int qoff[KS], qtoff[2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qoff[ks] = rslot<D>(sigma(m), 2 * ks + h);
#pragma unroll
    for (int t = 0; t < 2; ++t)
        qtoff[t] = tslot<kKQueries / 8>(m, 2 * h + t);

    for (int it = 0; it < n_tiles; ++it) {
        __syncthreads();
        land();
        const int owner = __builtin_amdgcn_readfirstlane(t_cur.owner);
        const int valid = __builtin_amdgcn_readfirstlane(t_cur.valid);
        const int origin = __builtin_amdgcn_readfirstlane((int)t_cur.origin);
        __syncthreads();
        fetch(t_next, pos_next);
        t_cur = t_next;
        if (it + 2 < n_tiles)
            t_next = next_tile();
        pos_next = query_pos(t_next);

        // The queries that see this lane's key form one interval [qlo, qhi]
        // of the tile: positions origin + qi with 0 <= qpos - kpos < w in the
        // window pass; in the group pass the queries ascend and the far ones
        // (qpos >= kpos + w) are a suffix.
        int qlo = 0, qhi = -1;
        if (kvalid) {
            if (GROUP) {
                const int lim = kpos + w;
                qhi = valid - 1;
                if (qpos_lds[0] < lim) {
                    int lo = 0, hi = valid;
                    while (lo < hi) {
                        const int mid = (lo + hi) >> 1;
                        if (qpos_lds[mid] < lim)
                            lo = mid + 1;
                        else
                            hi = mid;
                    }
                    qlo = lo;
                }
            } else {
                qlo = std::max(0, kpos - origin);
                qhi = std::min(valid - 1, kpos - origin + w - 1);
            }
        }
        const bool full =
            !owner && __builtin_amdgcn_ballot_w64(!(qlo <= 0 && qhi >= kKQueries - 1)) == 0;

        // S = Q K^T and dP = dO V^T: rows are queries (sigma), columns keys.
        // The Q / dO fragments are read first; the Q^T / dO^T fragments of
        // the second product are read between the MFMAs (fenced order).
        bf16x8 qfr[KS], dfr[KS], dtf[DB][2], qtf[DB][2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qfr[ks] = lds16(q_lds, qoff[ks]);
            dfr[ks] = lds16(do_lds, qoff[ks]);
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            s[r] = dp[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qfr[ks], kf[ks], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dfr[ks], vf[ks], dp, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 2 * DB / KS; ++q) {
                const int f = ks * (2 * DB / KS) + q;  // f / 2 = db, f % 2 = t
                dtf[f / 2][f % 2] = lds16(dot_lds, qtoff[f % 2] + (f / 2) * 32 * (kKQueries / 8));
                qtf[f / 2][f % 2] = lds16(qt_lds, qtoff[f % 2] + (f / 2) * 32 * (kKQueries / 8));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // P and dS, four queries at a time (their log2-domain LSE and D are
        // read as vectors: queries 16h + 4j .. 16h + 4j + 3)
        f32x16 ds;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 l4 = reinterpret_cast<const float4 *>(ql2_lds)[4 * h + j];
            const float4 d4 = reinterpret_cast<const float4 *>(qd_lds)[4 * h + j];
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
            const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = 4 * j + u;
                float pr = __builtin_amdgcn_exp2f(s[r] * p.c - lv[u]);
                if (!full) {
                    const int qi = 16 * h + r;
                    bool ok = qi >= qlo && qi <= qhi;
                    if (GROUP && owner)
                        ok = ok && ((qgm_lds[qi] & kgm & low) == 0u);
                    pr = ok ? pr : 0.f;
                }
                s[r] = pr;
                ds[r] = pr * (dp[r] - dv4[u]);
            }
        }
        const bf16x8 pf[2] = {pack8(s, 0), pack8(s, 1)};
        const bf16x8 dsf[2] = {pack8(ds, 0), pack8(ds, 1)};
        // dv^T += dO^T P, dk^T += Q^T dS
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                dv_acc[db] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(dtf[db][t], pf[t], dv_acc[db], 0, 0, 0);
                dk_acc[db] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(qtf[db][t], dsf[t], dk_acc[db], 0, 0, 0);
            }
    }

    if (kvalid) {
        const int64_t row = GROUP ? (int64_t)e_start + kr : p_start + kr;
        const int64_t rows = GROUP ? p.E : p.n;
        float *dk = p.dk + ((int64_t)kvh * rows + row) * D;
        float *dv = p.dv + ((int64_t)kvh * rows + row) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = db * 32 + 8 * j + 4 * h;
                *reinterpret_cast<float4 *>(dk + d) =
                    make_float4(dk_acc[db][4 * j] * p.scale, dk_acc[db][4 * j + 1] * p.scale,
                                dk_acc[db][4 * j + 2] * p.scale, dk_acc[db][4 * j + 3] * p.scale);
                *reinterpret_cast<float4 *>(dv + d) =
                    make_float4(dv_acc[db][4 * j], dv_acc[db][4 * j + 1], dv_acc[db][4 * j + 2],
                                dv_acc[db][4 * j + 3]);
            }
    }
}

// ---------------------------------------------------------------------------
// row statistics, plan and merge

// D_i = dO_i . O_i in fp32, one wavefront per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_drow_kernel(const __bf16 *__restrict__ out,
                                                       const __bf16 *__restrict__ dout,
                                                       int64_t rows, float *__restrict__ drow)
{
    const int lane = threadIdx.x % kWave;
    const int64_t r = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    if (r >= rows)
        return;
    float s = 0.f;
    for (int e = lane; e < D; e += kWave)
        s += (float)out[r * D + e] * (float)dout[r * D + e];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        s += __shfl_xor(s, off);
    if (lane == 0)
        drow[r] = s;
}

// Tiles of up to 128 entries inside each sub-bucket, one block per head.
__global__ __launch_bounds__(256) void bwd_plan_kernel(const int32_t *__restrict__ offsets,
                                                       int nsb, int max_tiles,
                                                       int4 *__restrict__ tiles,
                                                       int32_t *__restrict__ ntiles)
{
    __shared__ int base[1057];
    const int h = blockIdx.x;
    const int32_t *off = offsets + (int64_t)h * (nsb + 1);
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int sb = 0; sb < nsb; ++sb) {
            base[sb] = acc;
            acc += (off[sb + 1] - off[sb] + kBwdRows - 1) / kBwdRows;
        }
        base[nsb] = acc;
        ntiles[h] = acc;
    }
    __syncthreads();
    for (int sb = threadIdx.x; sb < nsb; sb += blockDim.x) {
        const int lo = off[sb], cnt = off[sb + 1] - lo;
        for (int t = 0; t * kBwdRows < cnt; ++t) {
            const int slot = base[sb] + t;
            if (slot < max_tiles)
                tiles[(int64_t)h * max_tiles + slot] =
                    make_int4(sb, lo + t * kBwdRows, std::min(kBwdRows, cnt - t * kBwdRows), 0);
        }
    }
}

// out[head][t] = win[head][t] + sum_s grp[head'][slot_entry[t][s]], in bf16;
// the bucket arrays are per key/value head (head' = head / ratio).
template <int D>
__global__ __launch_bounds__(256) void bwd_merge_kernel(const float *__restrict__ win,
                                                        const float *__restrict__ grp,
                                                        const int32_t *__restrict__ slot_entry,
                                                        int heads, int ratio, int64_t n,
                                                        int64_t E, int topk,
                                                        __bf16 *__restrict__ out)
{
    constexpr int V4 = D / 4;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)heads * n * V4)
        return;
    const int c = (int)(idx % V4);
    const int64_t ht = idx / V4;
    const int64_t head = ht / n, t = ht % n;
    const int64_t kvh = head / ratio;
    float4 a = reinterpret_cast<const float4 *>(win + ht * D)[c];
    for (int s = 0; s < topk; ++s) {
        const int64_t e = slot_entry[(kvh * n + t) * topk + s];
        const float4 b = reinterpret_cast<const float4 *>(grp + (head * E + e) * D)[c];
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
    __bf16 *o = out + ht * D + c * 4;
    o[0] = (__bf16)a.x;
    o[1] = (__bf16)a.y;
    o[2] = (__bf16)a.z;
    o[3] = (__bf16)a.w;
}

struct BwdLayout {
    size_t drow, dq_win, dk_win, dv_win, dq_grp, dk_grp, dv_grp, tiles, ntiles, total;
    int max_tiles;
};

BwdLayout bwd_layout(const AttnShape &sh)
{
    BwdLayout L{};
    const int64_t n = sh.n, E = n * sh.topk;
    const int nsb = num_subbuckets(sh.K);
    L.max_tiles = (int)((E + kBwdRows - 1) / kBwdRows + nsb);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes, 256);
        return o;
    };
    L.drow = take(sizeof(float) * sh.hq * n);
    L.dq_win = take(sizeof(float) * sh.hq * n * sh.d);
    L.dk_win = take(sizeof(float) * sh.hkv * n * sh.d);
    L.dv_win = take(sizeof(float) * sh.hkv * n * sh.d);
    L.dq_grp = take(sizeof(float) * sh.hq * E * sh.d);
    L.dk_grp = take(sizeof(float) * sh.hkv * E * sh.d);
    L.dv_grp = take(sizeof(float) * sh.hkv * E * sh.d);
    L.tiles = take(sizeof(int4) * sh.hkv * (size_t)L.max_tiles);
    L.ntiles = take(sizeof(int32_t) * sh.hkv);
    L.total = off;
    return L;
}

template <int D>
hipError_t launch_bwd_d(const AttnShape &sh, const void *q, const void *k, const void *v,
                        const void *out, const float *lse, const void *dout,
                        const uint32_t *gmask, const int32_t *offsets, const int32_t *tokens,
                        const int32_t *slot_entry, void *dq, void *dk, void *dv, void *ws,
                        hipStream_t s)
{
    const BwdLayout L = bwd_layout(sh);
    char *base = static_cast<char *>(ws);
    const int64_t n = sh.n, E = n * sh.topk;
    BwdParams p{};
    p.hq = sh.hq;
    p.hkv = sh.hkv;
    p.ratio = sh.hq / sh.hkv;
    p.K = sh.K;
    p.topk = sh.topk;
    p.window = (int)std::min<int64_t>(sh.window, n);
    p.n = n;
    p.E = E;
    p.scale = sh.scale;
    p.c = sh.scale * kLog2e;
    p.q = static_cast<const __bf16 *>(q);
    p.k = static_cast<const __bf16 *>(k);
    p.v = static_cast<const __bf16 *>(v);
    p.dout = static_cast<const __bf16 *>(dout);
    p.lse = lse;
    p.drow = reinterpret_cast<float *>(base + L.drow);
    p.tokens = tokens;
    p.offsets = offsets;
    p.gmask = gmask;
    p.tiles = reinterpret_cast<const int4 *>(base + L.tiles);
    p.ntiles = reinterpret_cast<const int32_t *>(base + L.ntiles);
    p.max_tiles = L.max_tiles;
    p.row_tiles = (int)((n + kBwdRows - 1) / kBwdRows);

    const int64_t qrows = (int64_t)sh.hq * n;
    hipLaunchKernelGGL(bwd_drow_kernel<D>, dim3((unsigned)((qrows + 3) / 4)), dim3(256), 0, s,
                       static_cast<const __bf16 *>(out), p.dout, qrows,
                       reinterpret_cast<float *>(base + L.drow));
    hipLaunchKernelGGL(bwd_plan_kernel, dim3(sh.hkv), dim3(256), 0, s, offsets,
                       num_subbuckets(sh.K), L.max_tiles,
                       reinterpret_cast<int4 *>(base + L.tiles),
                       reinterpret_cast<int32_t *>(base + L.ntiles));

    // window pass
    p.dq = reinterpret_cast<float *>(base + L.dq_win);
    p.dk = reinterpret_cast<float *>(base + L.dk_win);
    p.dv = reinterpret_cast<float *>(base + L.dv_win);
    hipLaunchKernelGGL((bwd_dq_kernel<D, false>), dim3((unsigned)(sh.hq * p.row_tiles)),
                       dim3(kBwdThreads), 0, s, p);
    hipLaunchKernelGGL((bwd_dkv_kernel<D, false>), dim3((unsigned)(sh.hkv * p.row_tiles)),
                       dim3(kBwdThreads), 0, s, p);
    // group pass
    p.dq = reinterpret_cast<float *>(base + L.dq_grp);
    p.dk = reinterpret_cast<float *>(base + L.dk_grp);
    p.dv = reinterpret_cast<float *>(base + L.dv_grp);
    hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3((unsigned)(sh.hq * L.max_tiles)),
                       dim3(kBwdThreads), 0, s, p);
    hipLaunchKernelGGL((bwd_dkv_kernel<D, true>), dim3((unsigned)(sh.hkv * L.max_tiles)),
                       dim3(kBwdThreads), 0, s, p);
    // merge
    const int64_t qv = qrows * (D / 4), kv = (int64_t)sh.hkv * n * (D / 4);
    hipLaunchKernelGGL(bwd_merge_kernel<D>, dim3((unsigned)((qv + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const float *>(base + L.dq_win),
                       reinterpret_cast<const float *>(base + L.dq_grp), slot_entry, sh.hq,
                       p.ratio, n, E, sh.topk, static_cast<__bf16 *>(dq));
    hipLaunchKernelGGL(bwd_merge_kernel<D>, dim3((unsigned)((kv + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const float *>(base + L.dk_win),
                       reinterpret_cast<const float *>(base + L.dk_grp), slot_entry, sh.hkv, 1,
                       n, E, sh.topk, static_cast<__bf16 *>(dk));
    hipLaunchKernelGGL(bwd_merge_kernel<D>, dim3((unsigned)((kv + 255) / 256)), dim3(256), 0, s,
                       reinterpret_cast<const float *>(base + L.dv_win),
                       reinterpret_cast<const float *>(base + L.dv_grp), slot_entry, sh.hkv, 1,
                       n, E, sh.topk, static_cast<__bf16 *>(dv));
    return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace_bytes(const AttnShape &sh) { return bwd_layout(sh).total; }

hipError_t launch_attn_bwd(const AttnShape &sh, const void *q, const void *k, const void *v,
                           const void *out, const float *lse, const void *dout,
                           const uint32_t *gmask, const int32_t *offsets, const int32_t *tokens,
                           const int32_t *slot_entry, void *dq, void *dk, void *dv, void *ws,
                           hipStream_t s)
{
    if (sh.d == 128)
        return launch_bwd_d<128>(sh, q, k, v, out, lse, dout, gmask, offsets, tokens,
                                 slot_entry, dq, dk, dv, ws, s);
    return launch_bwd_d<64>(sh, q, k, v, out, lse, dout, gmask, offsets, tokens, slot_entry, dq,
                            dk, dv, ws, s);
}

}  // namespace focus
