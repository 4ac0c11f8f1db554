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
//   * dq pass (query-major, like the forward): a block of 8 wavefronts owns
//     128 query rows and walks their 64-key tiles, the two wavefronts of a
//     SIMD sharing 32 queries and splitting each tile's keys in halves;
//     S^T = K Q^T and dP^T = V dO^T put one query per lane column, dS^T
//     feeds dq^T += K^T dS^T from registers, and the halves' sums are added
//     at the end.
//   * dk/dv pass (key-major): a block of 4 wavefronts walks the 32-query
//     tiles that see its keys, for every query head of the key/value head;
//     S = Q K^T and dP = dO V^T put one key per lane column, P and dS feed
//     dv^T += dO^T P and dk^T += Q^T dS.  The window pass gives each
//     wavefront 32 keys (K and V in registers); the group pass gives it 64
//     (two column blocks sharing every LDS fragment read, the dK / dV sums
//     in AGPRs, K in LDS).
// The group passes run first and write fp32 partials per bucket entry; the
// window passes then add, in their epilogues, a row's window part and its k
// group parts (found through slot_entry) and round the sum to bf16, so the
// window parts never go to memory.
//
// Data movement.  The group passes read copies of their rows gathered into
// bucket (entry) order by a prepare kernel, so that every staged tile, in
// both partitions, is a run of consecutive rows.  Tiles go straight from HBM
// into a four-stage LDS ring by LDS-DMA (three tiles in flight while one is
// computed; one barrier per tile), row-major with 16-byte chunks XOR-swizzled.
// v_mfma_f32_32x32x16_bf16 needs both operands contiguous along the
// reduction index: the row operands (K and V in the dq pass, Q and dO in the
// dk/dv pass) are read as 16-byte fragments, the transposed ones (K^T, and
// Q^T and dO^T) with the LDS transpose read ds_read_b64_tr_b16 from the same
// row-major tile.
#include <algorithm>
#include <cstddef>

#include "attn_common.hpp"

namespace focus {
namespace {
using namespace attn;

constexpr int kBwdThreads = 256;  // dk/dv pass: 4 wavefronts
constexpr int kDqThreads = 512;   // dq pass: 8 wavefronts, 2 per SIMD
constexpr int kBwdRows = 128;     // query rows (dq pass) or keys (dk/dv pass) per block
constexpr int kWideKeys = 256;    // keys per block of the wide dk/dv group pass
constexpr int kQKeys = 64;        // dq pass: keys per staged tile
constexpr int kKQueries = 32;     // dk/dv pass: queries per staged tile
constexpr int kDqStages = 4;      // LDS ring depth (dq pass)
constexpr int kDkvStages = 4;     // LDS ring depth (dk/dv pass)

struct BwdParams {
    int hq, hkv, ratio, K, topk, window;
    int64_t n, E;
    float c;      // scale * log2(e)
    float scale;
    // rows in position order (window pass) or gathered in entry order (group
    // pass): [heads][rows][D] with rows = n or E
    const __bf16 *q, *k, *v, *dout;
    const float *l2;    // forward log-sum-exp times log2(e), [hq][rows]
    const float *drow;  // D_i = dO_i . O_i, [hq][rows]
    // group pass
    const uint32_t *egm;     // group bits per entry [hkv][E]
    const int32_t *tokens;   // [hkv][E]
    const int32_t *offsets;  // [hkv][num_subbuckets(K, topk) + 1]
    const int4 *tiles;       // [hkv][max_tiles]: (sub-bucket, first entry, rows, group)
    const int32_t *ntiles;
    int max_tiles;
    const int4 *tiles_w;     // the same for the wide dk/dv pass's tiles of 256 keys
    const int32_t *ntiles_w;
    int max_tiles_w;
    int row_tiles;  // window: 128-row tiles per head
    // group passes: fp32 partials per entry, [hq][E][D] and [hkv][E][D]
    float *dq;
    float *dk, *dv;
    // window passes: the group partials to add, each row's entries, and the
    // bf16 results [hq][n][D] and [hkv][n][D]
    const float *grp_dq, *grp_dk, *grp_dv;
    const int32_t *slot_entry;
    __bf16 *out_dq, *out_dk, *out_dv;
};

// XOR swizzle of the 16-byte chunks of a row-major [rows][D] tile (chunk c of
// row r sits in slot c ^ rswz(r)).  With 64 banks of 4 bytes it keeps three
// access patterns free of bank conflicts: 16-byte fragment reads of rows
// sigma(m) (16 lanes, rows differing in bits 0, 1, 2 and 4), transpose reads
// (32 lanes, 4 consecutive rows times 64 bytes) and the row writes of the
// DMA (16 lanes, one row).
template <int D>
__device__ __forceinline__ int rswz(int row)
{
    if (D == 128)  // row bits 0,1 -> chunk bits 2,3; bit 2 -> 0; bit 4 -> 1
        return ((row & 3) << 2) | ((row >> 2) & 1) | (((row >> 4) & 1) << 1);
    // 128-byte rows: bit 0 already picks the bank half; bit 1 -> 2, 2 -> 0, 4 -> 1
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 1) | (((row >> 4) & 1) << 1);
}
template <int D>
__device__ __forceinline__ uint32_t rbyte(int row, int c)  // byte offset of chunk c of row
{
    return (uint32_t)((row * (D / 8) + (c ^ rswz<D>(row))) * 16);
}

__device__ __forceinline__ bf16x8 lds16(const char *base, uint32_t off)
{
    return *reinterpret_cast<const bf16x8 *>(base + off);
}

// ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte pieces addressed by lanes 4v + i / 4 (v = 0..3).  With
// lane 4a + b addressing row r0 + a, columns c0 + 4b .. c0 + 4b + 3 of a
// row-major tile, lane i thus holds rows r0 .. r0 + 3 of column c0 + i.
typedef short s16x4 __attribute__((vector_size(8)));
__device__ __forceinline__ uint2 lds_tr(const char *p)
{
    const s16x4 r =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p);
    return __builtin_bit_cast(uint2, r);
}
// A fragment of a transposed operand: lane (m, h) gets column m of rows
// r0 + 8h .. r0 + 8h + 7 (the two halves of 4 rows from two transpose reads)
__device__ __forceinline__ bf16x8 tr_frag(const char *tile, uint32_t o0, uint32_t o1)
{
    const uint2 a = lds_tr(tile + o0), b = lds_tr(tile + o1);
    return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
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

// LDS-DMA of a [ROWS][D] tile of consecutive rows: load i of wavefront w
// fills the 1024 LDS bytes (w L + i) * 1024 ..., i.e. rows (w L + i) R ..
// (R rows per load), lane l slot l % KCH of its row, so it fetches the chunk
// the swizzle keeps there.  Rows at or past `valid` re-read row valid - 1 (the
// kernels mask them), so no load leaves the tile's rows.
template <int D, int ROWS, int WAVES = kBwdThreads / kWave>
struct TileDma {
    static constexpr int RB = D * 2;
    static constexpr int KCH = D / 8;
    static constexpr int R = 1024 / RB;
    static constexpr int LOADS = ROWS / R / WAVES;
    static_assert(LOADS >= 1 && LOADS * R * WAVES == ROWS, "tile shape");
    int row[LOADS];
    uint32_t cofs[LOADS];
    __device__ void init(int wave, int lane)
    {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            row[i] = (wave * LOADS + i) * R + lane / KCH;
            cofs[i] = (uint32_t)(((lane % KCH) ^ rswz<D>(row[i])) * 16);
        }
    }
    __device__ void issue(const void *base, int valid, uint32_t lds, int wave) const
    {
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
            dma16(base, (uint32_t)(std::min(row[i], valid - 1) * RB) + cofs[i],
                  lds + (uint32_t)(wave * LOADS + i) * 1024u);
    }
};

// LDS byte address of the member at byte offset `off` of stage S of a
// __shared__ stage ring, from the ring's own address: indexing the ring
// with a run-time S and converting the member's generic pointer back would
// cost a shared-aperture add and a null test per address.
template <class StageT, int N>
__device__ __forceinline__ uint32_t stage_lds(StageT (&ring)[N], int S, size_t off)
{
    return lds_address(ring) + (uint32_t)S * (uint32_t)sizeof(StageT) + (uint32_t)off;
}

// "s_waitcnt vmcnt(n) lgkmcnt(0)" for a wave-uniform n in 0..47 (larger n
// waits for 47, which is only more conservative)
__device__ __forceinline__ void wait_vm_n(int n)
{
#define FOCUS_WAIT_CASE(k) \
    case k:                \
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(k)); \
        break;
    switch (n) {
        FOCUS_WAIT_CASE(0) FOCUS_WAIT_CASE(1) FOCUS_WAIT_CASE(2) FOCUS_WAIT_CASE(3)
        FOCUS_WAIT_CASE(4) FOCUS_WAIT_CASE(5) FOCUS_WAIT_CASE(6) FOCUS_WAIT_CASE(7)
        FOCUS_WAIT_CASE(8) FOCUS_WAIT_CASE(9) FOCUS_WAIT_CASE(10) FOCUS_WAIT_CASE(11)
        FOCUS_WAIT_CASE(12) FOCUS_WAIT_CASE(13) FOCUS_WAIT_CASE(14) FOCUS_WAIT_CASE(15)
        FOCUS_WAIT_CASE(16) FOCUS_WAIT_CASE(17) FOCUS_WAIT_CASE(18) FOCUS_WAIT_CASE(19)
        FOCUS_WAIT_CASE(20) FOCUS_WAIT_CASE(21) FOCUS_WAIT_CASE(22) FOCUS_WAIT_CASE(23)
        FOCUS_WAIT_CASE(24) FOCUS_WAIT_CASE(25) FOCUS_WAIT_CASE(26) FOCUS_WAIT_CASE(27)
        FOCUS_WAIT_CASE(28) FOCUS_WAIT_CASE(29) FOCUS_WAIT_CASE(30) FOCUS_WAIT_CASE(31)
        FOCUS_WAIT_CASE(32) FOCUS_WAIT_CASE(33) FOCUS_WAIT_CASE(34) FOCUS_WAIT_CASE(35)
        FOCUS_WAIT_CASE(36) FOCUS_WAIT_CASE(37) FOCUS_WAIT_CASE(38) FOCUS_WAIT_CASE(39)
        FOCUS_WAIT_CASE(40) FOCUS_WAIT_CASE(41) FOCUS_WAIT_CASE(42) FOCUS_WAIT_CASE(43)
        FOCUS_WAIT_CASE(44) FOCUS_WAIT_CASE(45) FOCUS_WAIT_CASE(46)
    default:
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(47));
        break;
    }
#undef FOCUS_WAIT_CASE
}

// a += the group partials of a row's entries, in slot order, at one float4
// of d: grp points at element d of the head's entry 0, rows D floats apart
template <int D>
__device__ __forceinline__ void add_group_parts(float4 &a, const float *grp,
                                                const int32_t *slot_entry, int topk)
{
    for (int s = 0; s < topk; ++s) {
        const float4 b = *reinterpret_cast<const float4 *>(grp + (int64_t)slot_entry[s] * D);
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
}
__device__ __forceinline__ void store_bf16x4(__bf16 *o, const float4 &a)
{
    o[0] = (__bf16)a.x;
    o[1] = (__bf16)a.y;
    o[2] = (__bf16)a.z;
    o[3] = (__bf16)a.w;
}

// ---------------------------------------------------------------------------
// dq pass

template <int D, bool GROUP>
__global__ __launch_bounds__(kDqThreads, 1) void bwd_dq_kernel(BwdParams p)
{
    constexpr int KS = D / 16;   // k-steps over d
    constexpr int DB = D / 32;   // 32-row blocks of d
    constexpr int RB = D * 2;    // bytes per row
    constexpr int WAVES = kDqThreads / kWave;
    using Dma = TileDma<D, kQKeys, WAVES>;
    struct Stage {
        char k[kQKeys * RB];
        char v[kQKeys * RB];
        int pos[kWave];       // key positions (group pass)
        uint32_t gm[kWave];   // key group bits (group pass)
    };
    __shared__ __attribute__((aligned(16))) Stage stg[kDqStages];
    __shared__ int sub_start[GROUP ? kMaxCodes : 1], sub_count[GROUP ? kMaxCodes : 1],
        sub_owner[GROUP ? kMaxCodes : 1], sub_tiles;

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int m = lane % 32;
    const int h = lane / 32;
    // waves w and w + 4 (one SIMD) share the 32 queries of group w % 4 and
    // take the two 32-key halves of every key tile
    const int qg = wave & 3;
    const int kh = wave >> 2;

    // ---- work item: (key/value head, tile, query head of that key/value
    // head), in that order, the query heads of one tile adjacent (they read
    // the same key tiles); each XCD takes one contiguous range of the list
    // (the grid is a multiple of 8 long), so neighbouring tiles share its L2
    const int b = xcd_remap(blockIdx.x, gridDim.x);
    const int tiles_per_kvh = GROUP ? p.max_tiles : p.row_tiles;
    if (b >= p.hkv * tiles_per_kvh * p.ratio)
        return;
    const int hr = b % p.ratio;
    const int slot = (b / p.ratio) % tiles_per_kvh;
    const int kvh = b / p.ratio / tiles_per_kvh;
    const int hq = kvh * p.ratio + hr;
    if (GROUP && slot >= p.ntiles[kvh])
        return;
    int g = 0, sbq = 0, tile_rows;
    int64_t row0;  // first query row (entry or position)
    if (GROUP) {
        const int4 t = p.tiles[(int64_t)kvh * p.max_tiles + slot];
        sbq = t.x;
        row0 = t.y;
        tile_rows = t.z;
        g = t.w;
    } else {
        row0 = (int64_t)slot * kBwdRows;
        tile_rows = (int)std::min<int64_t>(kBwdRows, p.n - row0);
    }
    const int64_t rows = GROUP ? p.E : p.n;
    const int32_t *tok = GROUP ? p.tokens + (int64_t)kvh * p.E : nullptr;
    const uint32_t *egm = GROUP ? p.egm + (int64_t)kvh * p.E : nullptr;

    // ---- this lane's query (column m of the wave pair's 32 rows)
    const int qr = qg * 32 + m;
    const bool qvalid = qr < tile_rows;
    const int qrc = qvalid ? qr : 0;
    const int qpos = GROUP ? tok[row0 + qrc] : (int)(row0 + qrc);
    const int64_t qrow = (int64_t)hq * rows + row0 + qrc;
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
    const float l2 = p.l2[qrow];
    const float dq_d = p.drow[qrow];
    const uint32_t qgm = GROUP ? egm[row0 + qrc] : 0u;
    const int w = p.window;

    // ---- key tiles
    int n_tiles = 0;
    int64_t j_first = 0;
    if (GROUP) {
        const int bq_max = tok[row0 + tile_rows - 1];
        // the key sub-buckets of group g whose lower sets miss the query
        // tile's (as in the forward's group pass), packed by wave 0
        if (wave == 0) {
            const int cm = code_members(p.K, p.topk);
            const LowerSet qs = decode_lower(g, sbq - group_base(g, cm));
            const int ncode = codes_of_group(g, cm);
            const int gb = group_base(g, cm);
            const int32_t *offh =
                p.offsets + (int64_t)kvh * (num_subbuckets(p.K, p.topk) + 1);
            const int64_t lim = (int64_t)bq_max - w;  // keys at or before lim
            const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
            int kept = 0, tiles = 0;
            for (int c0 = 0; c0 < ncode; c0 += 64) {
                const int c = c0 + lane;
                int cnt = 0, lo0 = 0, owner = 0;
                if (c < ncode) {
                    const LowerSet ks = decode_lower(g, c);
                    const bool meets = lower_sets_meet(qs, ks);
                    lo0 = offh[gb + c];
                    const int hi0 = offh[gb + c + 1];
                    if (!meets && hi0 > lo0) {
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
                    owner = owner_test_needed(p.topk, cm, qs, ks);
                }
                const uint64_t keep = __ballot(cnt > 0);
                if (cnt > 0) {
                    const int at = kept + __popcll(keep & below);
                    sub_start[at] = lo0;
                    sub_count[at] = cnt;
                    sub_owner[at] = owner;
                }
                kept += __popcll(keep);
                tiles += (cnt + kQKeys - 1) / kQKeys;
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1)
                tiles += __shfl_xor(tiles, o);
            if (lane == 0)
                sub_tiles = tiles;
        }
        __syncthreads();
        n_tiles = sub_tiles;
    } else if (w > 0) {
        const int64_t lo = std::max<int64_t>(0, row0 - w + 1);
        j_first = (lo / kQKeys) * kQKeys;
        const int64_t j_last = row0 + tile_rows - 1;
        n_tiles = (int)((j_last - j_first) / kQKeys + 1);
    }
    const int T = __builtin_amdgcn_readfirstlane(n_tiles);
    // a group tile whose last key is at or before this wave's smallest
    // qpos - w is taken whole by every query of the wave
    int wave_lim = qvalid ? qpos - w : 0x7fffffff;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        wave_lim = std::min(wave_lim, __shfl_xor(wave_lim, off));
    wave_lim = __builtin_amdgcn_readfirstlane(wave_lim);

    // ---- tiles in order (wave-uniform iterator; the issue side runs three
    // tiles ahead of the compute side)
    struct It {
        int sub, tile, cnt, start, owner;
    };
    auto it_next = [&](It &t, int &origin, int &valid, int &owner) {
        if (GROUP) {
            while (t.tile * kQKeys >= t.cnt) {
                ++t.sub;
                t.tile = 0;
                t.cnt = __builtin_amdgcn_readfirstlane(sub_count[t.sub]);
                t.start = __builtin_amdgcn_readfirstlane(sub_start[t.sub]);
                t.owner = __builtin_amdgcn_readfirstlane(sub_owner[t.sub]);
            }
            valid = std::min(kQKeys, t.cnt - t.tile * kQKeys);
            origin = t.start + t.tile * kQKeys;
            owner = t.owner;
        } else {
            origin = (int)(j_first + (int64_t)t.tile * kQKeys);
            valid = (int)std::min<int64_t>(kQKeys, p.n - origin);
            owner = 0;
        }
        ++t.tile;
    };
    It it_issue{-1, 0, 0, 0, 0}, it_comp{-1, 0, 0, 0, 0};

    // ---- staging: K and V tiles by LDS-DMA (all waves), key positions
    // (wave 0) and group bits (wave 1) of the group pass by 4-byte DMA
    Dma dma;
    dma.init(wave, lane);
    constexpr int DMA_KV = 2 * Dma::LOADS;
    const bool extra = GROUP && wave < 2;
    const int per_tile = DMA_KV + (extra ? 1 : 0);  // this wave's loads per tile
    constexpr int AHEAD = kDqStages - 1;             // tiles in flight ahead
    auto issue = [&](int S) {
        int origin, valid, owner;
        it_next(it_issue, origin, valid, owner);
        const int64_t r0 = (int64_t)kvh * rows + origin;
        dma.issue(p.k + r0 * D, valid, stage_lds(stg, S, offsetof(Stage, k)), wave);
        dma.issue(p.v + r0 * D, valid, stage_lds(stg, S, offsetof(Stage, v)), wave);
        if (GROUP) {
            const uint32_t lo = (uint32_t)std::min(lane, valid - 1) * 4u;
            if (wave == 0)
                dma4(tok + origin, lo, stage_lds(stg, S, offsetof(Stage, pos)));
            else if (wave == 1)
                dma4(egm + origin, lo, stage_lds(stg, S, offsetof(Stage, gm)));
        }
    };

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[db][r] = 0.f;

    // per-lane LDS byte offsets in this wave's 32-key half: K and V rows
    // (row 32 kh + sigma(m), chunk 2ks+h) and K^T by transpose reads
    // (d = 32 db + m, keys 32 kh + 16h + 8t + 4s + 0..3; t adds 8 rows)
    uint32_t koff[KS], tro[DB][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        koff[ks] = rbyte<D>(32 * kh + sigma(m), 2 * ks + h);
    {
        const int jj = lane & 15, gp = (lane >> 4) & 1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int row = 32 * kh + 16 * h + 4 * s + (jj >> 2);
                const int col = 32 * db + 16 * gp + 4 * (jj & 3);
                tro[db][s] = rbyte<D>(row, col >> 3) + (uint32_t)(col & 7) * 2u;
            }
    }

    const uint32_t low = GROUP ? ((1u << g) - 1u) : 0u;

    // One key tile in stage S: S^T = K Q^T, then dP^T = V dO^T with
    // P^T = exp2(S^T c - L log2 e) formed two elements per step (K^T
    // transpose reads in between), dS^T = P^T (dP^T - D), dq^T += K^T dS^T,
    // then the DMA of tile u + AHEAD and the end-of-tile barrier.
    auto body = [&](int S, int u) {
        int origin, valid, owner;
        it_next(it_comp, origin, valid, owner);
        const char *kl = stg[S].k;
        const char *vl = stg[S].v;
        const int klast = GROUP ? stg[S].pos[valid - 1] : 0;

        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            s[r] = dp[r] = 0.f;
        bf16x8 ktf[DB][2];
        bf16x8 fr[3];
        fr[0] = lds16(kl, koff[0]);
        fr[1] = lds16(kl, koff[1]);
        auto stream = [&](int i) {  // fragment i + 2 of the 2 KS sequence (K then V)
            if (i + 2 < 2 * KS) {
                const int n2 = i + 2;
                fr[n2 % 3] = lds16(n2 < KS ? kl : vl, koff[n2 % KS]);
            }
        };
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            stream(i);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % 3], qf[i], s, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }

        // Keys this lane's query takes, as a bit mask over the wave's half:
        // an interval (window: 0 <= qpos - kpos < w; group: the keys ascend,
        // the far ones kpos <= qpos - w are a prefix), in the group pass's
        // owner tiles also without a lower shared group.
        uint32_t kmask;
        if (GROUP) {
            int khi = valid - 1;
            if (__builtin_amdgcn_readfirstlane(klast) > wave_lim && qvalid) {
                const int lim = qpos - w;
                if (klast > lim) {
                    int lo = 0, hi = valid;
                    while (lo < hi) {
                        const int mid = (lo + hi) >> 1;
                        if (stg[S].pos[mid] <= lim)
                            lo = mid + 1;
                        else
                            hi = mid;
                    }
                    khi = lo - 1;
                }
            }
            // keys 32 kh .. 32 kh + 31 of the tile, at or below khi
            const int top = khi - 32 * kh;
            kmask = !qvalid || top < 0 ? 0u : top >= 31 ? 0xffffffffu : ((2u << top) - 1u);
            if (owner) {
                for (int kk = 0; kk < 32; ++kk)
                    if (32 * kh + kk < valid &&
                        (qgm & stg[S].gm[32 * kh + kk] & low) != 0u)
                        kmask &= ~(1u << kk);
            }
        } else {
            const int lo = std::max(0, qpos - origin - w + 1) - 32 * kh;
            const int hi = std::min(qpos - origin, valid - 1) - 32 * kh;
            const int clo = std::max(lo, 0), chi = std::min(hi, 31);
            kmask = qvalid && chi >= clo ? (uint32_t)((2ull << chi) - (1ull << clo)) : 0u;
        }
        // this lane's 16 keys are 16h .. 16h + 15 of the half; a wave whose
        // queries all take the whole half skips the mask
        const uint32_t mh = kmask >> (16 * h);
        const bool full = __builtin_amdgcn_ballot_w64(kmask != 0xffffffffu) == 0;
        __builtin_amdgcn_sched_barrier(0);

        // dP^T chain with P^T of registers 2i, 2i + 1 after step i, and the
        // K^T fragments read in between
        auto dp_chain = [&](auto masked) {
#pragma unroll
            for (int i = 0; i < KS; ++i) {
                stream(KS + i);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[(KS + i) % 3], dof[i], dp, 0, 0, 0);
                {
                    static_assert(2 * DB == KS, "one K^T fragment per step");
                    const int db = i / 2, t = i % 2;
                    const uint32_t step = (uint32_t)(8 * t * RB);
                    ktf[db][t] = tr_frag(kl, tro[db][0] + step, tro[db][1] + step);
                }
#pragma unroll
                for (int e = 0; e < 16 / KS; ++e) {
                    const int r = (16 / KS) * i + e;
                    const float pr = __builtin_amdgcn_exp2f(s[r] * p.c - l2);
                    if constexpr (decltype(masked)::value) {
                        const int keep = __builtin_amdgcn_sbfe((int)mh, r, 1);  // 0 or -1
                        s[r] = __int_as_float(__float_as_int(pr) & keep);
                    } else {
                        s[r] = pr;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if (full)
            dp_chain(std::false_type{});
        else
            dp_chain(std::true_type{});
        // dS^T = P^T (dP^T - D) as bf16 B fragments
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dp[r] = s[r] * (dp[r] - dq_d);
        const bf16x8 dsf[2] = {pack8(dp, 0), pack8(dp, 1)};
        // dq^T += K^T dS^T
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktf[db][t], dsf[t], acc[db], 0, 0, 0);
        // tile u + AHEAD into the stage tile u - 1 left, then: tile u + 1
        // landed (the tiles after it may still fly), every wave done with S
        if (u + AHEAD < T)
            issue(S == 0 ? kDqStages - 1 : S - 1);
        if (u + 1 < T) {
            // AHEAD - 1 tiles may fly on in the steady state (an immediate
            // count), fewer at the ring's tail
            if (u + AHEAD < T) {
                if (extra)
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((AHEAD - 1) * (DMA_KV + 1)));
                else
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((AHEAD - 1) * DMA_KV));
            } else {
                wait_vm_n((T - 2 - u) * per_tile);
            }
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
    };

    // the loads above have landed before any DMA is issued (the compiler's
    // own wait tracking then has nothing outstanding in the loop)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    asm volatile("" ::: "memory");
    for (int i = 0; i < AHEAD && i < T; ++i)
        issue(i);
    wait_vm_n((std::min(T, AHEAD) - 1) * per_tile);
    __syncthreads();
    for (int u = 0, S = 0; u < T; ++u, S = S == kDqStages - 1 ? 0 : S + 1)
        body(S, u);

    // ---- the two key halves' partial sums: the second wave of each pair
    // leaves its accumulators in LDS (the stage ring is free after the
    // barrier), the first adds them and stores.  Lane (m, h), register r of
    // block db holds dq[query m][d].
    __syncthreads();
    static_assert(sizeof(stg) >= sizeof(float) * 4 * DB * 16 * kWave, "reduction fits the ring");
    float *red = reinterpret_cast<float *>(&stg[0]);  // [4 pairs][DB][16][64 lanes]
    if (kh == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                red[((qg * DB + db) * 16 + r) * kWave + lane] = acc[db][r];
    }
    __syncthreads();
    if (kh == 0 && qvalid) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[db][r] += red[((qg * DB + db) * 16 + r) * kWave + lane];
        if (GROUP) {
            float *dst = p.dq + ((int64_t)hq * rows + row0 + qr) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<float4 *>(dst + db * 32 + 8 * j + 4 * h) =
                        make_float4(acc[db][4 * j] * p.scale, acc[db][4 * j + 1] * p.scale,
                                    acc[db][4 * j + 2] * p.scale, acc[db][4 * j + 3] * p.scale);
        } else {
            // the row's window part plus its group parts, rounded once
            const int64_t t = row0 + qr;
            const int32_t *se = p.slot_entry + ((int64_t)kvh * p.n + t) * p.topk;
            __bf16 *dst = p.out_dq + ((int64_t)hq * p.n + t) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d = db * 32 + 8 * j + 4 * h;
                    float4 a = make_float4(acc[db][4 * j] * p.scale, acc[db][4 * j + 1] * p.scale,
                                           acc[db][4 * j + 2] * p.scale,
                                           acc[db][4 * j + 3] * p.scale);
                    add_group_parts<D>(a, p.grp_dq + (int64_t)hq * p.E * D + d, se, p.topk);
                    store_bf16x4(dst + d, a);
                }
        }
    }
}

// ---------------------------------------------------------------------------
// dk/dv window pass (32 keys per wavefront)

template <int D>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkv_window_kernel(BwdParams p)
{
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int RB = D * 2;
    using Dma = TileDma<D, kKQueries>;
    struct Stage {
        char q[kKQueries * RB];
        char d[kKQueries * RB];
        float l2[kWave];       // query log-sum-exp times log2(e)
        float dd[kWave];       // query D_i
    };
    __shared__ __attribute__((aligned(16))) Stage stg[kDkvStages];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int m = lane % 32;
    const int h = lane / 32;

    // ---- work item: (key/value head, tile of 128 keys); each XCD takes one
    // contiguous range (the grid is a multiple of 8 long), so neighbouring
    // key tiles, which stream the same query tiles, share its L2
    const int b = xcd_remap(blockIdx.x, gridDim.x);
    if (b >= p.hkv * p.row_tiles)
        return;
    const int slot = b % p.row_tiles;
    const int kvh = b / p.row_tiles;
    const int64_t row0 = (int64_t)slot * kBwdRows;
    const int tile_keys = (int)std::min<int64_t>(kBwdRows, p.n - row0);
    const int64_t rows = p.n;

    // ---- this lane's key (column m of the wavefront's 32 keys)
    const int kr = wave * 32 + m;
    const bool kvalid = kr < tile_keys;
    const int krc = kvalid ? kr : 0;
    const int kpos = (int)(row0 + krc);
    bf16x8 kf[KS], vf[KS];
    {
        const int64_t row = (int64_t)kvh * rows + row0 + krc;
        const bf16x8 *ks_ = reinterpret_cast<const bf16x8 *>(p.k + row * D);
        const bf16x8 *vs_ = reinterpret_cast<const bf16x8 *>(p.v + row * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kf[ks] = ks_[ks * 2 + h];
            vf[ks] = vs_[ks * 2 + h];
        }
    }
    const int w = p.window;

    // ---- query tiles, per query head: the queries i with 0 <= i - j < w of
    // the tile's keys j
    int tiles_per_head = 0;
    int64_t i_first = 0;
    if (w > 0) {
        i_first = row0;
        const int64_t i_last = std::min<int64_t>(p.n - 1, row0 + tile_keys - 1 + w - 1);
        tiles_per_head = (int)((i_last - i_first) / kKQueries + 1);
    }
    tiles_per_head = __builtin_amdgcn_readfirstlane(tiles_per_head);
    const int T = tiles_per_head * p.ratio;

    // ---- tiles in order, per query head (wave-uniform iterator; the issue
    // side runs two tiles ahead of the compute side)
    struct It {
        int head, tile, count;
    };
    auto it_next = [&](It &t, int &head, int &origin, int &valid) {
        if (t.count == tiles_per_head) {  // next query head
            ++t.head;
            t.tile = 0;
            t.count = 0;
        }
        ++t.count;
        head = kvh * p.ratio + t.head;
        origin = (int)(i_first + (int64_t)t.tile * kKQueries);
        valid = (int)std::min<int64_t>(kKQueries, p.n - origin);
        ++t.tile;
    };
    It it_issue{0, 0, 0}, it_comp{0, 0, 0};

    // ---- staging: Q and dO tiles by LDS-DMA (all waves); per query, the
    // log2-domain log-sum-exp (wave 1) and D (wave 2) by 4-byte DMA
    Dma dma;
    dma.init(wave, lane);
    constexpr int DMA_QD = 2 * Dma::LOADS;
    const bool extra = wave == 1 || wave == 2;
    const int per_tile = DMA_QD + (extra ? 1 : 0);  // this wave's loads per tile
    constexpr int AHEAD = kDkvStages - 1;             // tiles in flight ahead
    auto issue = [&](int S) {
        int head, origin, valid;
        it_next(it_issue, head, origin, valid);
        const int64_t r0 = (int64_t)head * rows + origin;
        dma.issue(p.q + r0 * D, valid, stage_lds(stg, S, offsetof(Stage, q)), wave);
        dma.issue(p.dout + r0 * D, valid, stage_lds(stg, S, offsetof(Stage, d)), wave);
        const uint32_t lo = (uint32_t)std::min(lane, valid - 1) * 4u;
        if (wave == 1)
            dma4(p.l2 + r0, lo, stage_lds(stg, S, offsetof(Stage, l2)));
        else if (wave == 2)
            dma4(p.drow + r0, lo, stage_lds(stg, S, offsetof(Stage, dd)));
    };

    f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dk_acc[db][r] = dv_acc[db][r] = 0.f;

    // per-lane LDS byte offsets: Q and dO rows (row sigma(m), chunk 2ks+h)
    // and Q^T / dO^T by transpose reads (d = 32 db + m, queries
    // 16h + 8t + 4s + 0..3; t adds 8 rows)
    uint32_t qoff[KS], tro[DB][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qoff[ks] = rbyte<D>(sigma(m), 2 * ks + h);
    {
        const int jj = lane & 15, gp = (lane >> 4) & 1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int row = 16 * h + 4 * s + (jj >> 2);
                const int col = 32 * db + 16 * gp + 4 * (jj & 3);
                tro[db][s] = rbyte<D>(row, col >> 3) + (uint32_t)(col & 7) * 2u;
            }
    }

    // One query tile in stage S, ordered so that the vector work overlaps
    // the matrix cores: S = Q K^T (16-byte fragments streamed two steps
    // ahead, the transpose reads of dO^T in between); the key's query mask;
    // dP = dO V^T with P = exp2(S c - L log2 e) formed two elements per step
    // (no mask where the wave's keys all see the whole tile); dv^T += dO^T P
    // with dS = P (dP - D) formed two elements per step and the Q^T
    // transpose reads in between; dk^T += Q^T dS; then the DMA of tile
    // u + AHEAD and the end-of-tile barrier.
    auto body = [&](int S, int u) {
        int head_c, origin, valid;
        it_next(it_comp, head_c, origin, valid);
        (void)head_c;
        const char *ql = stg[S].q;
        const char *dl = stg[S].d;

        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            s[r] = dp[r] = 0.f;
        bf16x8 dtf[DB][2], qtf[DB][2];
        bf16x8 fr[3];
        fr[0] = lds16(ql, qoff[0]);
        fr[1] = lds16(ql, qoff[1]);
        auto stream = [&](int i) {  // fragment i + 2 of the 2 KS sequence (Q then dO)
            if (i + 2 < 2 * KS) {
                const int n2 = i + 2;
                fr[n2 % 3] = lds16(n2 < KS ? ql : dl, qoff[n2 % KS]);
            }
        };
        auto transpose_reads = [&](int i) {  // dO^T during S
#pragma unroll
            for (int q = 0; q < 2 * DB / KS; ++q) {
                const int f = i * (2 * DB / KS) + q;  // f / 2 = db, f % 2 = t
                const int db = f / 2, t = f % 2;
                const uint32_t step = (uint32_t)(8 * t * RB);
                dtf[db][t] = tr_frag(dl, tro[db][0] + step, tro[db][1] + step);
            }
        };
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            stream(i);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % 3], kf[i], s, 0, 0, 0);
            transpose_reads(i);
            __builtin_amdgcn_sched_barrier(0);
        }
        // log2-domain log-sum-exp of this lane's queries 16h .. 16h + 15
        float4 l4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            l4[j] = reinterpret_cast<const float4 *>(stg[S].l2)[4 * h + j];

        // Queries this lane's key sees, as a bit mask over the tile: the
        // interval 0 <= qpos - kpos < w.
        const int qlo = std::max(0, kpos - origin);
        const int qhi = std::min(valid - 1, kpos - origin + w - 1);
        const uint32_t qmask =
            kvalid && qhi >= qlo ? (uint32_t)((2ull << qhi) - (1ull << qlo)) : 0u;
        // this lane's 16 queries are 16h .. 16h + 15; a wave whose valid
        // keys all see the whole tile skips the mask (the columns of keys
        // past the tile's end are never stored)
        const uint32_t mh = qmask >> (16 * h);
        const bool full = __builtin_amdgcn_ballot_w64(kvalid && qmask != 0xffffffffu) == 0;
        __builtin_amdgcn_sched_barrier(0);

        // dP chain; P of registers 2i, 2i + 1 after dP step i
        auto dp_chain = [&](auto masked) {
#pragma unroll
            for (int i = 0; i < KS; ++i) {
                stream(KS + i);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[(KS + i) % 3], vf[i], dp, 0, 0,
                                                             0);
#pragma unroll
                for (int e = 0; e < 16 / KS; ++e) {
                    const int r = (16 / KS) * i + e;
                    const float l = r % 4 == 0 ? l4[r / 4].x : r % 4 == 1 ? l4[r / 4].y
                                  : r % 4 == 2 ? l4[r / 4].z : l4[r / 4].w;
                    const float pr = __builtin_amdgcn_exp2f(s[r] * p.c - l);
                    if constexpr (decltype(masked)::value) {
                        const int keep = __builtin_amdgcn_sbfe((int)mh, r, 1);  // 0 or -1
                        s[r] = __int_as_float(__float_as_int(pr) & keep);
                    } else {
                        s[r] = pr;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if (full)
            dp_chain(std::false_type{});
        else
            dp_chain(std::true_type{});
        const bf16x8 pf[2] = {pack8(s, 0), pack8(s, 1)};
        float4 d4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            d4[j] = reinterpret_cast<const float4 *>(stg[S].dd)[4 * h + j];
        __builtin_amdgcn_sched_barrier(0);
        // dv^T += dO^T P; dS of registers 2i, 2i + 1 after MFMA i, and the Q^T
        // fragment of step i read into the registers dO^T fragment i leaves
#pragma unroll
        for (int i = 0; i < 2 * DB; ++i) {
            const int db = i / 2, t = i % 2;
            dv_acc[db] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(dtf[db][t], pf[t], dv_acc[db], 0, 0, 0);
            {
                const uint32_t step = (uint32_t)(8 * t * RB);
                qtf[db][t] = tr_frag(ql, tro[db][0] + step, tro[db][1] + step);
            }
#pragma unroll
            for (int e = 0; e < 16 / (2 * DB); ++e) {
                const int r = (16 / (2 * DB)) * i + e;
                const float dd = r % 4 == 0 ? d4[r / 4].x : r % 4 == 1 ? d4[r / 4].y
                               : r % 4 == 2 ? d4[r / 4].z : d4[r / 4].w;
                dp[r] = s[r] * (dp[r] - dd);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const bf16x8 dsf[2] = {pack8(dp, 0), pack8(dp, 1)};
        // dk^T += Q^T dS
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                dk_acc[db] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(qtf[db][t], dsf[t], dk_acc[db], 0, 0, 0);
        // tile u + AHEAD into the stage tile u - 1 left (every wave passed
        // the barrier after it), then: tile u + 1 landed (the tiles after it
        // may still fly) and every wave done with this stage
        if (u + AHEAD < T)
            issue(S == 0 ? kDkvStages - 1 : S - 1);
        if (u + 1 < T) {
            if (u + AHEAD < T) {
                if (extra)
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((AHEAD - 1) * (DMA_QD + 1)));
                else
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((AHEAD - 1) * DMA_QD));
            } else {
                wait_vm_n((T - 2 - u) * per_tile);
            }
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
    };

    // the loads above have landed before any DMA is issued (the compiler's
    // own wait tracking then has nothing outstanding in the loop)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    asm volatile("" ::: "memory");
    for (int i = 0; i < AHEAD && i < T; ++i)
        issue(i);
    wait_vm_n((std::min(T, AHEAD) - 1) * per_tile);
    __syncthreads();
    for (int u = 0, S = 0; u < T; ++u, S = S == kDkvStages - 1 ? 0 : S + 1)
        body(S, u);

    if (kvalid) {
        // the key's window part plus its group parts, rounded once
        const int32_t *se = p.slot_entry + ((int64_t)kvh * p.n + kpos) * p.topk;
        __bf16 *dk = p.out_dk + ((int64_t)kvh * p.n + kpos) * D;
        __bf16 *dv = p.out_dv + ((int64_t)kvh * p.n + kpos) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = db * 32 + 8 * j + 4 * h;
                float4 a = make_float4(dk_acc[db][4 * j] * p.scale, dk_acc[db][4 * j + 1] * p.scale,
                                       dk_acc[db][4 * j + 2] * p.scale,
                                       dk_acc[db][4 * j + 3] * p.scale);
                add_group_parts<D>(a, p.grp_dk + (int64_t)kvh * p.E * D + d, se, p.topk);
                store_bf16x4(dk + d, a);
                float4 b = make_float4(dv_acc[db][4 * j], dv_acc[db][4 * j + 1],
                                       dv_acc[db][4 * j + 2], dv_acc[db][4 * j + 3]);
                add_group_parts<D>(b, p.grp_dv + (int64_t)kvh * p.E * D + d, se, p.topk);
                store_bf16x4(dv + d, b);
            }
    }
}

// ---------------------------------------------------------------------------
// dk/dv group pass, wide form: 64 keys per wavefront
//
// Each wavefront holds two 32-key column blocks, so every Q / dO fragment
// and every Q^T / dO^T transpose fragment read from LDS feeds two products
// instead of one: fewer LDS reads, waits and per-tile bookkeeping per FLOP
// than the 32-key form.  The dK and dV sums of 64 keys take 256 registers
// per lane; they live in the AGPR file (one wavefront per SIMD has all 512
// registers), written by the products below.  V stays in VGPRs; K sits in
// LDS (64 KB per block), each lane reading back exactly the chunks it wrote,
// so S takes one more 16-byte read per product.

// One v_mfma_f32_32x32x16_bf16 accumulating into AGPRs.  The compiler does
// not see inside the statement, so it carries the wait states itself: two
// before the product, for an A/B operand a VALU instruction has just written
// (LDS loads are covered by the compiler's own lgkmcnt waits).  Dependent
// products into the same accumulator issue back to back; a read of the
// accumulator needs the product to have landed (agpr_settle).
__device__ __forceinline__ void mfma_agpr(f32x16 &acc, const bf16x8 &a, const bf16x8 &b)
{
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                 : "+a"(acc)
                 : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_agpr_zero(f32x16 &acc, const bf16x8 &z)
{
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(z));
}
// 32 wait states: more than a 32x32x16 product needs before its result is
// read by any other instruction
__device__ __forceinline__ void agpr_settle()
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// NE consecutive floats of an LDS array (NE = 2 or 4)
template <int NE>
__device__ __forceinline__ void lds_floats(const float *p, float (&out)[NE])
{
    if constexpr (NE == 2) {
        const float2 v = *reinterpret_cast<const float2 *>(p);
        out[0] = v.x;
        out[1] = v.y;
    } else {
        static_assert(NE == 4, "two or four values per step");
        const float4 v = *reinterpret_cast<const float4 *>(p);
        out[0] = v.x;
        out[1] = v.y;
        out[2] = v.z;
        out[3] = v.w;
    }
}

template <int D>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkv_wide_kernel(BwdParams p)
{
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int RB = D * 2;
    constexpr int KB = 2;                  // 32-key column blocks per wavefront
    constexpr int NP = 16 / KS;            // P elements per block per dP step
    constexpr int NS = 16 / (2 * DB);      // dS elements per block per dV step
    constexpr int NTR = 4 * DB;            // transpose fragments per tile (dO^T, then Q^T)
    using Dma = TileDma<D, kKQueries>;
    struct Stage {
        char q[kKQueries * RB];
        char d[kKQueries * RB];
        int pos[kWave];        // query positions
        float l2[kWave];       // query log-sum-exp times log2(e)
        float dd[kWave];       // query D_i
        uint32_t gm[kWave];    // query group bits
    };
    __shared__ __attribute__((aligned(16))) Stage stg[kDkvStages];
    __shared__ __attribute__((aligned(16))) char k_lds[kBwdThreads / kWave][32 * KB * RB];
    __shared__ int sub_start[kMaxCodes], sub_count[kMaxCodes], sub_owner[kMaxCodes], sub_tiles;

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int m = lane % 32;
    const int h = lane / 32;

    // ---- work item: (key/value head, tile of up to 256 keys of one
    // sub-bucket); each XCD takes one contiguous range
    const int b = xcd_remap(blockIdx.x, gridDim.x);
    if (b >= p.hkv * p.max_tiles_w)
        return;
    const int slot = b % p.max_tiles_w;
    const int kvh = b / p.max_tiles_w;
    if (slot >= p.ntiles_w[kvh])
        return;
    const int4 wt = p.tiles_w[(int64_t)kvh * p.max_tiles_w + slot];
    const int sbk = wt.x;
    const int64_t row0 = wt.y;
    const int tile_keys = wt.z;
    const int g = wt.w;
    const int64_t rows = p.E;
    const int32_t *tok = p.tokens + (int64_t)kvh * p.E;
    const uint32_t *egm = p.egm + (int64_t)kvh * p.E;
    const int w = p.window;

    // ---- this lane's keys: column m of key blocks c (keys 64 wave + 32 c + m)
    // per-lane LDS byte offsets: Q and dO rows (row sigma(m), chunk 2ks+h)
    // and Q^T / dO^T by transpose reads (d = 32 db + m, queries
    // 16h + 8t + 4s + 0..3; t adds 8 rows).  The swizzle only flips chunk
    // bits, so k-step ks is the ks = 0 offset XOR 32 ks, and d-block db the
    // db = 0 offset XOR 64 db.
    const uint32_t qoff0 = rbyte<D>(sigma(m), h);
    auto qoff = [&](int ks) { return qoff0 ^ (uint32_t)(32 * ks); };
    uint32_t tro0[2];
    {
        const int jj = lane & 15, gp = (lane >> 4) & 1;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int row = 16 * h + 4 * s + (jj >> 2);
            const int col = 16 * gp + 4 * (jj & 3);
            tro0[s] = rbyte<D>(row, col >> 3) + (uint32_t)(col & 7) * 2u;
        }
    }
    auto tro = [&](int db, int s) { return tro0[s] ^ (uint32_t)(64 * db); };
    // key (c, m) of this wave sits at row 32 c + sigma(m) of its LDS K block,
    // so the fragment reads use the Q offsets
    char *const kl = k_lds[wave];

    bool kvalid[KB];
    int kpos[KB];
    uint32_t kgm[KB];
    bf16x8 vf[KB][KS];
#pragma unroll
    for (int c = 0; c < KB; ++c) {
        const int kr = wave * 32 * KB + 32 * c + m;
        kvalid[c] = kr < tile_keys;
        const int krc = kvalid[c] ? kr : 0;
        kpos[c] = tok[row0 + krc];
        kgm[c] = egm[row0 + krc];
        const int64_t row = (int64_t)kvh * rows + row0 + krc;
        const bf16x8 *ks_ = reinterpret_cast<const bf16x8 *>(p.k + row * D);
        const bf16x8 *vs_ = reinterpret_cast<const bf16x8 *>(p.v + row * D);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            *reinterpret_cast<bf16x8 *>(kl + 32 * c * RB + qoff(ks)) = ks_[ks * 2 + h];
            vf[c][ks] = vs_[ks * 2 + h];
        }
    }

    // ---- the query sub-buckets of group g whose lower sets miss the key
    // tile's, with the queries at or after (first key position + w), packed
    // by wave 0
    {
        const int bk_min = tok[row0];  // keys ascend inside the sub-bucket
        if (wave == 0) {
            const int cm = code_members(p.K, p.topk);
            const LowerSet ks = decode_lower(g, sbk - group_base(g, cm));
            const int ncode = codes_of_group(g, cm);
            const int gb = group_base(g, cm);
            const int32_t *offh =
                p.offsets + (int64_t)kvh * (num_subbuckets(p.K, p.topk) + 1);
            const int64_t lim = (int64_t)bk_min + w;  // queries at or after lim
            const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
            int kept = 0, tiles = 0;
            for (int c0 = 0; c0 < ncode; c0 += 64) {
                const int c = c0 + lane;
                int cnt = 0, first = 0, owner = 0;
                if (c < ncode) {
                    const LowerSet qs = decode_lower(g, c);
                    const bool meets = lower_sets_meet(qs, ks);
                    const int lo0 = offh[gb + c], hi0 = offh[gb + c + 1];
                    first = hi0;
                    if (!meets && hi0 > lo0) {
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
                    cnt = hi0 - first;
                    owner = owner_test_needed(p.topk, cm, qs, ks);
                }
                const uint64_t keep = __ballot(cnt > 0);
                if (cnt > 0) {
                    const int at = kept + __popcll(keep & below);
                    sub_start[at] = first;
                    sub_count[at] = cnt;
                    sub_owner[at] = owner;
                }
                kept += __popcll(keep);
                tiles += (cnt + kKQueries - 1) / kKQueries;
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1)
                tiles += __shfl_xor(tiles, o);
            if (lane == 0)
                sub_tiles = tiles;
        }
        __syncthreads();
    }
    const int tiles_per_head = __builtin_amdgcn_readfirstlane(sub_tiles);
    const int T = tiles_per_head * p.ratio;
    // a tile whose first query is at or after this wave's largest kpos + w
    // is seen by every key of the wave
    int wave_lim = -0x7fffffff;
#pragma unroll
    for (int c = 0; c < KB; ++c)
        if (kvalid[c])
            wave_lim = std::max(wave_lim, kpos[c] + w);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        wave_lim = std::max(wave_lim, __shfl_xor(wave_lim, off));
    wave_lim = __builtin_amdgcn_readfirstlane(wave_lim);

    // ---- tiles in order, per query head (wave-uniform iterator; the issue
    // side runs AHEAD tiles ahead of the compute side)
    struct It {
        int head, sub, tile, count, cnt, start, owner;
    };
    auto it_next = [&](It &t, int &head, int &origin, int &valid, int &owner) {
        if (t.count == tiles_per_head) {  // next query head
            ++t.head;
            t.sub = -1;
            t.tile = 0;
            t.cnt = 0;
            t.count = 0;
        }
        ++t.count;
        head = kvh * p.ratio + t.head;
        while (t.tile * kKQueries >= t.cnt) {
            ++t.sub;
            t.tile = 0;
            t.cnt = __builtin_amdgcn_readfirstlane(sub_count[t.sub]);
            t.start = __builtin_amdgcn_readfirstlane(sub_start[t.sub]);
            t.owner = __builtin_amdgcn_readfirstlane(sub_owner[t.sub]);
        }
        valid = std::min(kKQueries, t.cnt - t.tile * kKQueries);
        origin = t.start + t.tile * kKQueries;
        owner = t.owner;
        ++t.tile;
    };
    It it_issue{0, -1, 0, 0, 0, 0, 0}, it_comp{0, -1, 0, 0, 0, 0, 0};

    // ---- staging: Q and dO tiles by LDS-DMA (all waves); per query the
    // position (wave 0), log2-domain log-sum-exp (wave 1), D (wave 2) and
    // group bits (wave 3) by 4-byte DMA
    Dma dma;
    dma.init(wave, lane);
    constexpr int per_tile = 2 * Dma::LOADS + 1;  // each wave's loads per tile
    constexpr int AHEAD = kDkvStages - 1;
    auto issue = [&](int S) {
        int head, origin, valid, owner;
        it_next(it_issue, head, origin, valid, owner);
        const int64_t r0 = (int64_t)head * rows + origin;
        dma.issue(p.q + r0 * D, valid, stage_lds(stg, S, offsetof(Stage, q)), wave);
        dma.issue(p.dout + r0 * D, valid, stage_lds(stg, S, offsetof(Stage, d)), wave);
        const uint32_t lo = (uint32_t)std::min(lane, valid - 1) * 4u;
        if (wave == 0)
            dma4(tok + origin, lo, stage_lds(stg, S, offsetof(Stage, pos)));
        else if (wave == 1)
            dma4(p.l2 + r0, lo, stage_lds(stg, S, offsetof(Stage, l2)));
        else if (wave == 2)
            dma4(p.drow + r0, lo, stage_lds(stg, S, offsetof(Stage, dd)));
        else
            dma4(egm + origin, lo, stage_lds(stg, S, offsetof(Stage, gm)));
    };

    // dK^T and dV^T of both key blocks, in AGPRs, cleared by zero products
    f32x16 dk_acc[KB][DB], dv_acc[KB][DB];
    {
        bf16x8 z;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            z[e] = (__bf16)0.f;
#pragma unroll
        for (int c = 0; c < KB; ++c)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                mfma_agpr_zero(dk_acc[c][db], z);
                mfma_agpr_zero(dv_acc[c][db], z);
            }
    }

    const uint32_t low = (1u << g) - 1u;

    // One query tile in stage S: S = Q K^T for both key blocks (each Q
    // fragment read once, streamed two steps ahead); the query masks; dP =
    // dO V^T with P formed between the products; dv^T += dO^T P and
    // dk^T += Q^T dS, each transpose fragment read once (two ahead) for both
    // blocks, dS formed between the dV products; then the DMA of tile
    // u + AHEAD and the end-of-tile barrier.
    auto body = [&](int S, int u) {
        int head_c, origin, valid, owner;
        it_next(it_comp, head_c, origin, valid, owner);
        (void)head_c;
        (void)origin;
        const char *ql = stg[S].q;
        const char *dl = stg[S].d;
        const int qfirst = stg[S].pos[0];

        f32x16 s[KB], dp[KB];
#pragma unroll
        for (int c = 0; c < KB; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[c][r] = dp[c][r] = 0.f;
        // fragments streamed two steps ahead: Q then dO, and with each Q
        // fragment the two key blocks' K fragments of the same k-step
        bf16x8 fr[3], kfr[3][KB];
        auto stream_at = [&](int n2) {
            fr[n2 % 3] = lds16(n2 < KS ? ql : dl, qoff(n2 % KS));
            if (n2 < KS) {
#pragma unroll
                for (int c = 0; c < KB; ++c)
                    kfr[n2 % 3][c] = lds16(kl, (uint32_t)(32 * c * RB) + qoff(n2));
            }
        };
        stream_at(0);
        stream_at(1);
        auto stream = [&](int i) {
            if (i + 2 < 2 * KS)
                stream_at(i + 2);
        };
#pragma unroll
        for (int i = 0; i < KS; ++i) {
            stream(i);
#pragma unroll
            for (int c = 0; c < KB; ++c)
                s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % 3], kfr[i % 3][c], s[c], 0,
                                                               0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }

        // Queries each of this lane's keys sees, as a bit mask over the tile:
        // the far ones (qpos >= kpos + w) are a suffix, since the queries
        // ascend; in owner tiles also without a lower shared group.
        const uint32_t vmask = valid == kKQueries ? 0xffffffffu : ((1u << valid) - 1u);
        uint32_t qmask[KB];
        bool need = false;
#pragma unroll
        for (int c = 0; c < KB; ++c) {
            int qlo = 0;
            if (__builtin_amdgcn_readfirstlane(qfirst) < wave_lim && kvalid[c]) {
                const int lim = kpos[c] + w;
                if (qfirst < lim) {
                    int lo = 0, hi = valid;
                    while (lo < hi) {
                        const int mid = (lo + hi) >> 1;
                        if (stg[S].pos[mid] < lim)
                            lo = mid + 1;
                        else
                            hi = mid;
                    }
                    qlo = lo;
                }
            }
            qmask[c] = kvalid[c] && qlo < kKQueries ? (vmask & (0xffffffffu << qlo)) : 0u;
            if (owner) {
                for (int qi = 0; qi < valid; ++qi)
                    if ((stg[S].gm[qi] & kgm[c] & low) != 0u)
                        qmask[c] &= ~(1u << qi);
            }
            need |= kvalid[c] && qmask[c] != 0xffffffffu;
        }
        // this lane's 16 queries are 16h .. 16h + 15; a wave whose valid keys
        // all see the whole tile skips the mask (the columns of keys past the
        // tile's end are never stored)
        const bool full = __builtin_amdgcn_ballot_w64(need) == 0;
        uint32_t mh[KB];
#pragma unroll
        for (int c = 0; c < KB; ++c)
            mh[c] = qmask[c] >> (16 * h);
        __builtin_amdgcn_sched_barrier(0);

        // dP chain for both blocks; P of registers NP i .. NP i + NP - 1
        // after step i (the log-sum-exp of those queries read alongside)
        auto dp_chain = [&](auto masked) {
#pragma unroll
            for (int i = 0; i < KS; ++i) {
                stream(KS + i);
                float l[NP];
                lds_floats<NP>(stg[S].l2 + 16 * h + NP * i, l);
#pragma unroll
                for (int c = 0; c < KB; ++c)
                    dp[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[(KS + i) % 3], vf[c][i],
                                                                    dp[c], 0, 0, 0);
#pragma unroll
                for (int c = 0; c < KB; ++c)
#pragma unroll
                    for (int e = 0; e < NP; ++e) {
                        const int r = NP * i + e;
                        const float pr = __builtin_amdgcn_exp2f(s[c][r] * p.c - l[e]);
                        if constexpr (decltype(masked)::value) {
                            const int keep = __builtin_amdgcn_sbfe((int)mh[c], r, 1);  // 0 or -1
                            s[c][r] = __int_as_float(__float_as_int(pr) & keep);
                        } else {
                            s[c][r] = pr;
                        }
                    }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if (full)
            dp_chain(std::false_type{});
        else
            dp_chain(std::true_type{});

        // transpose fragments j = 0 .. NTR - 1: dO^T (db, t) for the dV
        // products, then Q^T for the dK products; a ring of three, two ahead
        bf16x8 trf[3];
        auto tr_load = [&](int j) {
            const int jj = j % (2 * DB);
            const int db = jj / 2, t = jj % 2;
            const uint32_t step = (uint32_t)(8 * t * RB);
            trf[j % 3] = tr_frag(j < 2 * DB ? dl : ql, tro(db, 0) + step, tro(db, 1) + step);
        };
        tr_load(0);
        tr_load(1);
        bf16x8 pf[KB][2];
#pragma unroll
        for (int c = 0; c < KB; ++c) {
            pf[c][0] = pack8(s[c], 0);
            pf[c][1] = pack8(s[c], 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        // dv^T += dO^T P; dS of registers NS i .. NS i + NS - 1 after step i
#pragma unroll
        for (int i = 0; i < 2 * DB; ++i) {
            const int db = i / 2, t = i % 2;
            if (i + 2 < NTR)
                tr_load(i + 2);
            float dd[NS];
            lds_floats<NS>(stg[S].dd + 16 * h + NS * i, dd);
#pragma unroll
            for (int c = 0; c < KB; ++c)
                mfma_agpr(dv_acc[c][db], trf[i % 3], pf[c][t]);
#pragma unroll
            for (int c = 0; c < KB; ++c)
#pragma unroll
                for (int e = 0; e < NS; ++e) {
                    const int r = NS * i + e;
                    dp[c][r] = s[c][r] * (dp[c][r] - dd[e]);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 dsf[KB][2];
#pragma unroll
        for (int c = 0; c < KB; ++c) {
            dsf[c][0] = pack8(dp[c], 0);
            dsf[c][1] = pack8(dp[c], 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        // dk^T += Q^T dS
#pragma unroll
        for (int i = 0; i < 2 * DB; ++i) {
            const int j = 2 * DB + i;
            const int db = i / 2, t = i % 2;
            if (j + 2 < NTR)
                tr_load(j + 2);
#pragma unroll
            for (int c = 0; c < KB; ++c)
                mfma_agpr(dk_acc[c][db], trf[j % 3], dsf[c][t]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // tile u + AHEAD into the stage tile u - 1 left (every wave passed
        // the barrier after it), then: tile u + 1 landed (the tiles after it
        // may still fly) and every wave done with this stage
        if (u + AHEAD < T)
            issue(S == 0 ? kDkvStages - 1 : S - 1);
        if (u + 1 < T) {
            if (u + AHEAD < T)
                __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((AHEAD - 1) * per_tile));
            else
                wait_vm_n((T - 2 - u) * per_tile);
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
    };

    // the loads above have landed before any DMA is issued (the compiler's
    // own wait tracking then has nothing outstanding in the loop)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    asm volatile("" ::: "memory");
    for (int i = 0; i < AHEAD && i < T; ++i)
        issue(i);
    wait_vm_n((std::min(T, AHEAD) - 1) * per_tile);
    __syncthreads();
    for (int u = 0, S = 0; u < T; ++u, S = S == kDkvStages - 1 ? 0 : S + 1)
        body(S, u);

    // the last products land before the accumulators are read
    agpr_settle();
#pragma unroll
    for (int c = 0; c < KB; ++c)
#pragma unroll
        for (int db = 0; db < DB; ++db)
            asm volatile("" : "+a"(dk_acc[c][db]), "+a"(dv_acc[c][db]));
#pragma unroll
    for (int c = 0; c < KB; ++c) {
        if (!kvalid[c])
            continue;
        const int kr = wave * 32 * KB + 32 * c + m;
        float *dk = p.dk + ((int64_t)kvh * rows + row0 + kr) * D;
        float *dv = p.dv + ((int64_t)kvh * rows + row0 + kr) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = db * 32 + 8 * j + 4 * h;
                *reinterpret_cast<float4 *>(dk + d) = make_float4(
                    dk_acc[c][db][4 * j] * p.scale, dk_acc[c][db][4 * j + 1] * p.scale,
                    dk_acc[c][db][4 * j + 2] * p.scale, dk_acc[c][db][4 * j + 3] * p.scale);
                *reinterpret_cast<float4 *>(dv + d) =
                    make_float4(dv_acc[c][db][4 * j], dv_acc[c][db][4 * j + 1],
                                dv_acc[c][db][4 * j + 2], dv_acc[c][db][4 * j + 3]);
            }
    }
}

// ---------------------------------------------------------------------------
// row statistics, plan and the bucket-order copies

// D_i = dO_i . O_i in fp32, one wavefront per row, and the row's
// log-sum-exp in the log2 domain (L_i log2 e) for the exp2 of the passes.
template <int D>
__global__ __launch_bounds__(256) void bwd_drow_kernel(const __bf16 *__restrict__ out,
                                                       const __bf16 *__restrict__ dout,
                                                       const float *__restrict__ lse,
                                                       int64_t rows, float *__restrict__ drow,
                                                       float *__restrict__ l2)
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
    if (lane == 0) {
        drow[r] = s;
        l2[r] = lse[r] * kLog2e;
    }
}

// Tiles of up to ROWS entries inside each sub-bucket, one block per head.
template <int ROWS>
__global__ __launch_bounds__(256) void bwd_plan_kernel(const int32_t *__restrict__ offsets,
                                                       int K, int topk, int max_tiles,
                                                       int4 *__restrict__ tiles,
                                                       int32_t *__restrict__ ntiles)
{
    __shared__ int base[kMaxSubbuckets + 1];
    const int nsb = num_subbuckets(K, topk);
    const int h = blockIdx.x;
    const int32_t *off = offsets + (int64_t)h * (nsb + 1);
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int sb = 0; sb < nsb; ++sb) {
            base[sb] = acc;
            acc += (off[sb + 1] - off[sb] + ROWS - 1) / ROWS;
        }
        base[nsb] = acc;
        ntiles[h] = acc;
    }
    __syncthreads();
    for (int sb = threadIdx.x; sb < nsb; sb += blockDim.x) {
        const int lo = off[sb], cnt = off[sb + 1] - lo;
        int g = 0;
        while (g + 1 < K && group_base(g + 1, code_members(K, topk)) <= sb)
            ++g;
        for (int t = 0; t * ROWS < cnt; ++t) {
            const int slot = base[sb] + t;
            if (slot < max_tiles)
                tiles[(int64_t)h * max_tiles + slot] =
                    make_int4(sb, lo + t * ROWS, std::min(ROWS, cnt - t * ROWS), g);
        }
    }
}

// Bucket-order copies for the group passes: row e of head h of each
// destination is row tokens[h / ratio][e] of head h of its source (whole
// rows, 16 bytes per lane).
template <int D>
__global__ __launch_bounds__(256) void bwd_gather_rows_kernel(
    const __bf16 *__restrict__ a, const __bf16 *__restrict__ b,
    const int32_t *__restrict__ tokens, int ratio, int64_t n, int64_t E, int64_t total,
    __bf16 *__restrict__ da, __bf16 *__restrict__ db)
{
    constexpr int KCH = D / 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t r = idx / KCH;
    if (r >= total)
        return;
    const int c = (int)(idx % KCH);
    const int64_t h = r / E, e = r % E;
    const int64_t src = (h * n + tokens[(h / ratio) * E + e]) * D + c * 8;
    reinterpret_cast<uint4 *>(da + r * D)[c] = *reinterpret_cast<const uint4 *>(a + src);
    reinterpret_cast<uint4 *>(db + r * D)[c] = *reinterpret_cast<const uint4 *>(b + src);
}

// The per-row scalars of the same copies: log2-domain log-sum-exp and D per (query
// head, entry), group bits per (key/value head, entry).
__global__ __launch_bounds__(256) void bwd_gather_scalars_kernel(
    const float *__restrict__ l2, const float *__restrict__ drow,
    const uint32_t *__restrict__ gmask, const int32_t *__restrict__ tokens, int hq, int hkv,
    int ratio, int64_t n, int64_t E, float *__restrict__ gl2, float *__restrict__ gd,
    uint32_t *__restrict__ egm)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx < (int64_t)hq * E) {
        const int64_t h = idx / E, e = idx % E;
        const int64_t src = h * n + tokens[(h / ratio) * E + e];
        gl2[idx] = l2[src];
        gd[idx] = drow[src];
    }
    if (idx < (int64_t)hkv * E)
        egm[idx] = gmask[(idx / E) * n + tokens[idx]];
}

struct BwdLayout {
    size_t drow, l2, dq_grp, dk_grp, dv_grp, tiles, ntiles;
    size_t tiles_w, ntiles_w;
    size_t kg, vg, qg, dog, gl2, gd, egm, total;
    int max_tiles, max_tiles_w;
};

BwdLayout bwd_layout(const AttnShape &sh)
{
    BwdLayout L{};
    const int64_t n = sh.n, E = n * sh.topk;
    const int nsb = num_subbuckets(sh.K, sh.topk);
    L.max_tiles = (int)((E + kBwdRows - 1) / kBwdRows + nsb);
    L.max_tiles_w = (int)((E + kWideKeys - 1) / kWideKeys + nsb);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes, 256);
        return o;
    };
    L.drow = take(sizeof(float) * sh.hq * n);
    L.l2 = take(sizeof(float) * sh.hq * n);
    L.dq_grp = take(sizeof(float) * sh.hq * E * sh.d);
    L.dk_grp = take(sizeof(float) * sh.hkv * E * sh.d);
    L.dv_grp = take(sizeof(float) * sh.hkv * E * sh.d);
    L.tiles = take(sizeof(int4) * sh.hkv * (size_t)L.max_tiles);
    L.ntiles = take(sizeof(int32_t) * sh.hkv);
    L.tiles_w = take(sizeof(int4) * sh.hkv * (size_t)L.max_tiles_w);
    L.ntiles_w = take(sizeof(int32_t) * sh.hkv);
    // bucket-order copies read by the group passes
    L.kg = take(sizeof(__bf16) * sh.hkv * E * sh.d);
    L.vg = take(sizeof(__bf16) * sh.hkv * E * sh.d);
    L.qg = take(sizeof(__bf16) * sh.hq * E * sh.d);
    L.dog = take(sizeof(__bf16) * sh.hq * E * sh.d);
    L.gl2 = take(sizeof(float) * sh.hq * E);
    L.gd = take(sizeof(float) * sh.hq * E);
    L.egm = take(sizeof(uint32_t) * sh.hkv * E);
    L.total = off;
    return L;
}

// grid length rounded up to a whole number of blocks per XCD
inline unsigned xcd_grid(int64_t blocks)
{
    return (unsigned)((blocks + kXcds - 1) / kXcds * kXcds);
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
    p.l2 = reinterpret_cast<float *>(base + L.l2);
    p.drow = reinterpret_cast<float *>(base + L.drow);
    p.tokens = tokens;
    p.offsets = offsets;
    p.egm = nullptr;
    p.tiles = reinterpret_cast<const int4 *>(base + L.tiles);
    p.ntiles = reinterpret_cast<const int32_t *>(base + L.ntiles);
    p.max_tiles = L.max_tiles;
    p.tiles_w = reinterpret_cast<const int4 *>(base + L.tiles_w);
    p.ntiles_w = reinterpret_cast<const int32_t *>(base + L.ntiles_w);
    p.max_tiles_w = L.max_tiles_w;
    p.row_tiles = (int)((n + kBwdRows - 1) / kBwdRows);

    const int64_t qrows = (int64_t)sh.hq * n;
    hipLaunchKernelGGL(bwd_drow_kernel<D>, dim3((unsigned)((qrows + 3) / 4)), dim3(256), 0, s,
                       static_cast<const __bf16 *>(out), p.dout, lse, qrows,
                       reinterpret_cast<float *>(base + L.drow),
                       reinterpret_cast<float *>(base + L.l2));
    hipLaunchKernelGGL(bwd_plan_kernel<kBwdRows>, dim3(sh.hkv), dim3(256), 0, s, offsets, sh.K,
                       sh.topk, L.max_tiles, reinterpret_cast<int4 *>(base + L.tiles),
                       reinterpret_cast<int32_t *>(base + L.ntiles));
    hipLaunchKernelGGL(bwd_plan_kernel<kWideKeys>, dim3(sh.hkv), dim3(256), 0, s, offsets, sh.K,
                       sh.topk, L.max_tiles_w, reinterpret_cast<int4 *>(base + L.tiles_w),
                       reinterpret_cast<int32_t *>(base + L.ntiles_w));

    // group pass first (rows gathered into bucket order), then the window
    // pass, which adds each row's group partials and writes the results
    if (E > 0) {
        __bf16 *kg = reinterpret_cast<__bf16 *>(base + L.kg);
        __bf16 *vg = reinterpret_cast<__bf16 *>(base + L.vg);
        __bf16 *qg = reinterpret_cast<__bf16 *>(base + L.qg);
        __bf16 *dog = reinterpret_cast<__bf16 *>(base + L.dog);
        float *gl2 = reinterpret_cast<float *>(base + L.gl2);
        float *gd = reinterpret_cast<float *>(base + L.gd);
        uint32_t *egm = reinterpret_cast<uint32_t *>(base + L.egm);
        const int64_t krows = (int64_t)sh.hkv * E, qrows_g = (int64_t)sh.hq * E;
        hipLaunchKernelGGL(bwd_gather_rows_kernel<D>,
                           dim3((unsigned)((krows * (D / 8) + 255) / 256)), dim3(256), 0, s,
                           p.k, p.v, tokens, 1, n, E, krows, kg, vg);
        hipLaunchKernelGGL(bwd_gather_rows_kernel<D>,
                           dim3((unsigned)((qrows_g * (D / 8) + 255) / 256)), dim3(256), 0, s,
                           p.q, p.dout, tokens, p.ratio, n, E, qrows_g, qg, dog);
        hipLaunchKernelGGL(bwd_gather_scalars_kernel, dim3((unsigned)((qrows_g + 255) / 256)),
                           dim3(256), 0, s, p.l2, p.drow, gmask, tokens, sh.hq, sh.hkv, p.ratio,
                           n, E, gl2, gd, egm);
        BwdParams pg = p;
        pg.q = qg;
        pg.k = kg;
        pg.v = vg;
        pg.dout = dog;
        pg.l2 = gl2;
        pg.drow = gd;
        pg.egm = egm;
        pg.dq = reinterpret_cast<float *>(base + L.dq_grp);
        pg.dk = reinterpret_cast<float *>(base + L.dk_grp);
        pg.dv = reinterpret_cast<float *>(base + L.dv_grp);
        hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3(xcd_grid(sh.hq * L.max_tiles)),
                           dim3(kDqThreads), 0, s, pg);
        hipLaunchKernelGGL(bwd_dkv_wide_kernel<D>, dim3(xcd_grid(sh.hkv * L.max_tiles_w)),
                           dim3(kBwdThreads), 0, s, pg);
    }
    p.grp_dq = reinterpret_cast<const float *>(base + L.dq_grp);
    p.grp_dk = reinterpret_cast<const float *>(base + L.dk_grp);
    p.grp_dv = reinterpret_cast<const float *>(base + L.dv_grp);
    p.slot_entry = slot_entry;
    p.out_dq = static_cast<__bf16 *>(dq);
    p.out_dk = static_cast<__bf16 *>(dk);
    p.out_dv = static_cast<__bf16 *>(dv);
    hipLaunchKernelGGL((bwd_dq_kernel<D, false>), dim3(xcd_grid(sh.hq * p.row_tiles)),
                       dim3(kDqThreads), 0, s, p);
    hipLaunchKernelGGL(bwd_dkv_window_kernel<D>, dim3(xcd_grid(sh.hkv * p.row_tiles)),
                       dim3(kBwdThreads), 0, s, p);
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
