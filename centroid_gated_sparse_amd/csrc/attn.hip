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
//   * 512 threads = 8 wavefronts, two per SIMD; each wavefront owns 32
//     query rows and holds Q in registers for the whole key loop.  The
//     softmax's vector work is spread over both wavefronts of a SIMD: one
//     wavefront alone issues vector instructions at about half the SIMD's
//     rate.
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16 (fp32 inputs:
//     v_mfma_f32_32x32x2f32).  Computing the transposes puts one query per
//     lane column, so row max / row sum need one cross-half exchange per tile
//     and the P tile feeds the second product straight from registers.
//   * Key rows inside a 32-key block are permuted (sigma) so that lane half h,
//     register r of the S^T accumulator is key h*16 + r: the P fragment for
//     one 32x32x16 step is then 8 consecutive keys, matching one 16-byte read
//     of the V^T tile.
//   * K and V^T tiles of 64 keys are staged through LDS (XOR-swizzled), loaded
//     straight into LDS two tiles ahead over four stages (bf16; the fp32 path
//     double-buffers through registers); one barrier per tile.  Keys and
//     values are first gathered into bucket order (and V transposed) by a
//     prepare pass, so every tile load in the hot loop is contiguous.
//   * bf16: the two wavefronts of a SIMD run staggered roles (see the key
//     loop), so one wavefront's vector work overlaps the other's MFMAs.
//   * Grouped-query heads sharing a key/value head are packed into one block
//     (up to 4 heads x 64 rows), sharing every K/V tile and mask.
//   * Online softmax in the exp2 domain with lazy rescaling: the running max
//     is only moved when a tile raises it by more than 2^8.
#include <algorithm>
#include <cstring>
#include <type_traits>

#include "attn_common.hpp"

namespace focus {
namespace {
using namespace attn;

#ifndef FOCUS_ATTN_WAVES
#define FOCUS_ATTN_WAVES 8
#endif
constexpr int kThreads = 64 * FOCUS_ATTN_WAVES;  // 32 query rows per wavefront
static_assert(kRowsPerBlock == 32 * FOCUS_ATTN_WAVES, "32 rows per wavefront");
constexpr int kBlocksPerCU = 8 / FOCUS_ATTN_WAVES;  // two wavefronts per SIMD
constexpr int kWavesPerRole = FOCUS_ATTN_WAVES / 2;  // ping-pong roles A and B
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
    static constexpr int LOADS = 2 * (K_BYTES / 16) / kThreads;  // per role-A lane, K and V each

    struct QFrag {
        bf16x8 v[KS];
    };
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
    // sum of squares of the query elements this lane holds (half of them)
    __device__ static float q_sq_half(const QFrag &qf)
    {
        float a = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                a = __builtin_fmaf((float)qf.v[ks][e], (float)qf.v[ks][e], a);
        return a;
    }

    // Start the loads of one key tile straight into LDS (issued by the four
    // role-A wavefronts only; role B, on the critical path, issues none):
    // K rows row0.. of kmat and V^T columns row0.. of vmat (both zero-padded
    // past their last row, so no load needs a clamp).  Each global_load_lds writes 64
    // consecutive 16-byte LDS slots (one per lane), so every lane fetches the
    // chunk that the swizzled layout keeps in its slot.  Addresses are a
    // block-uniform base (scalar registers) plus a fixed per-lane 32-bit
    // offset.  Completion is awaited by the caller (vmcnt) before a barrier.
    struct Staged {
        uint32_t koff[LOADS];
        uint32_t voff[LOADS];
    };
    __device__ static void init_staging(Staged &st, const Params &p)
    {
        const int lane = threadIdx.x % kWave;
        const int wave = threadIdx.x / kWave;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int P = ((wave % kWavesPerRole) * LOADS + i) * kWave + lane;
            const int row = P / KCH;
            const int c = (P % KCH) ^ kswz(row);
            st.koff[i] = (uint32_t)((row * D + c * 8) * 2);
            const int d = P / 8;
            const int vc = (P % 8) ^ vswz(d);
            st.voff[i] = (uint32_t)(((int64_t)d * p.vcols + vc * 8) * 2);
        }
    }
    __device__ static void prefetch(Staged &st, const Params &p, int kvh, int64_t row0, char *kl,
                                    char *vl)
    {
        const char *kb = static_cast<const char *>(p.kmat) + ((int64_t)kvh * p.krows + row0) * D * 2;
        const char *vb = static_cast<const char *>(p.vmat) + ((int64_t)kvh * D * p.vcols + row0) * 2;
        const int wave = threadIdx.x / kWave;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int inst = wave * LOADS + i;
            dma16(kb, st.koff[i], lds_address(kl) + inst * 1024);
            dma16(vb, st.voff[i], lds_address(vl) + inst * 1024);
        }
    }
    __device__ static void land(const Staged &, char *, char *) {}

    // Per-lane byte offsets of this lane's MFMA operand fragments inside a K
    // tile (one per 16-wide step over d) and a V^T tile (one per 8-key
    // column group); the 32-row blocks of the tile add fixed offsets.
    struct LdsOff {
        uint32_t k[KS];
        uint32_t v[4];
    };
    __device__ static void init_lds_off(LdsOff &o, int m, int h)
    {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            o.k[ks] = (uint32_t)kslot(sigma(m), ks * 2 + h) * 16u;
#pragma unroll
        for (int j = 0; j < 4; ++j)  // j = kb * 2 + kk
            o.v[j] = (uint32_t)vslot(m, (j >> 1) * 4 + h * 2 + (j & 1)) * 16u;
    }
    // Hide the offsets' values from the optimiser at the start of each
    // compute phase: it then adds each stage's (constant) LDS address in the
    // instruction's immediate field instead of keeping a precomputed address
    // per stage live across the loop.
    __device__ static void refresh(LdsOff &o)
    {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            asm volatile("" : "+v"(o.k[ks]));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            asm volatile("" : "+v"(o.v[j]));
    }

    // The LDS reads of both products run ahead of the MFMAs that consume
    // them (two k-steps for S^T, one 16-key step for O^T), the order pinned
    // by scheduling fences: left alone, the scheduler issues each read just
    // before its use and the LDS latency stalls the matrix core.
    // (fence mask: VALU 0x2, SALU 0x4 and transcendental 0x400
    // instructions may cross, so the softmax still interleaves with the
    // MFMAs; LDS reads and MFMAs keep their order)
    static constexpr int kQkAhead = 2;
    static constexpr int kFence = 0x406;
    // S^T[key][query] for the two 32-key blocks of the tile.
    __device__ static void qk(f32x16 (&s)[2], const QFrag &qf, const char *kl, const LdsOff &o)
    {
        constexpr int AHEAD = kQkAhead < KS ? kQkAhead : KS;
        s[0] = f32x16{};
        s[1] = f32x16{};
        bf16x8 f[AHEAD + 1][2];
        auto load = [&](bf16x8 (&g)[2], int ks) {
            g[0] = *reinterpret_cast<const bf16x8 *>(kl + o.k[ks]);
            g[1] = *reinterpret_cast<const bf16x8 *>(kl + o.k[ks] + 32 * D * 2);
        };
#pragma unroll
        for (int ks = 0; ks < AHEAD; ++ks)
            load(f[ks], ks);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + AHEAD < KS)
                load(f[(ks + AHEAD) % (AHEAD + 1)], ks + AHEAD);
            __builtin_amdgcn_sched_barrier(kFence);
            const bf16x8(&g)[2] = f[ks % (AHEAD + 1)];
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(g[0], qf.v[ks], s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(g[1], qf.v[ks], s[1], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(kFence);
        }
    }

    // O^T[d][query] += V^T P^T, one 16-key step j = kb * 2 + kk at a time.
    __device__ static void pv(f32x16 (&o)[DB], const PFrag &pf, const char *vl, const LdsOff &lo)
    {
        bf16x8 f[2][DB];
        auto load = [&](bf16x8 (&g)[DB], int j) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
                g[db] = *reinterpret_cast<const bf16x8 *>(vl + lo.v[j] + db * 32 * 64 * 2);
        };
        load(f[0], 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j + 1 < 4)
                load(f[(j + 1) % 2], j + 1);
            __builtin_amdgcn_sched_barrier(kFence);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[j % 2][db], pf.v[j >> 1][j & 1],
                                                                o[db], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(kFence);
        }
    }

    // Exponentials of one tile -> bf16 P fragments; returns their fp32 sum.
    // (The sum is taken before rounding: near-uniform rows round their
    // probabilities the same way, and a sum of the rounded values would bias
    // the log-sum-exp by up to ~1e-3.)
    // (PRE: s already holds the exponent c s - m)
    template <bool PRE = false>
    __device__ static float exp_tile(const f32x16 (&s)[2], float c, float negm, PFrag &pf)
    {
        auto arg = [&](float x) { return PRE ? x : __builtin_fmaf(x, c, negm); };
        float l0 = 0.f, l1 = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(arg(s[kb][kk * 8 + e]));
                    const float p1 = __builtin_amdgcn_exp2f(arg(s[kb][kk * 8 + e + 1]));
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
    __device__ static void init_staging(Staged &, const Params &) {}

    __device__ static void load_q(QFrag &qf, const T *q, int64_t row_off, int h)
    {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf.v[ks] = q[row_off + ks * 2 + h];
    }
    __device__ static float q_sq_half(const QFrag &qf)
    {
        float a = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            a = __builtin_fmaf(qf.v[ks], qf.v[ks], a);
        return a;
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

    struct LdsOff {
        int m, h;
    };
    __device__ static void init_lds_off(LdsOff &o, int m, int h)
    {
        o.m = m;
        o.h = h;
    }
    __device__ static void refresh(LdsOff &) {}

    __device__ static void qk(f32x16 (&s)[2], const QFrag &qf, const char *kl, const LdsOff &lo)
    {
        const int m = lo.m, h = lo.h;
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

    __device__ static void pv(f32x16 (&o)[DB], const PFrag &pf, const char *vl, const LdsOff &lo)
    {
        const int m = lo.m, h = lo.h;
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

    template <bool PRE = false>
    __device__ static float exp_tile(const f32x16 (&s)[2], float c, float negm, PFrag &pf)
    {
        static_assert(!PRE, "the fp32 path forms its exponents here");
        float l = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, negm));
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
    float m;     // running max in the scaled log2 domain (may be -inf)
    float negm;  // exponent offset of P: -m, or 0 while m is -inf
    float thr;   // (m + kLazyRescale) / c, in raw-logit units
    float l;     // this lane half's partial row sum

    __device__ void init()
    {
#pragma unroll
        for (int db = 0; db < TL::DB; ++db)
            o[db] = f32x16{};
        m = -INFINITY;
        negm = 0.f;
        thr = -INFINITY;
        l = 0.f;
    }

    // Fixed exponent offset: m is set once to a bound on every logit of the
    // wavefront's rows (see kFixedOffsetMax) and never moves.
    __device__ void init_fixed(float m_bound)
    {
        init();
        m = m_bound;
        negm = -m_bound;
    }

    // Fold one tile of raw logits into the state; P receives the
    // probabilities for the PV product.
    //
    // FIXED: the offset is a bound on the logits, so P <= 1 and nothing is
    // ever rescaled: the tile costs its exponentials, their sum and the bf16
    // conversion.
    //
    // Otherwise a lazy rescale: the running max only moves when a row's max
    // grew by more than 2^8, so P stays below 2^8 and O is rarely rescaled.
    // The test needs no exchange between the lane halves: the row max
    // exceeds the row's threshold exactly when one of its halves does, and
    // the wavefront takes the update when any lane's does.  Only the update
    // forms the row max; the threshold and the exponent offset are kept with
    // m, so a tile that leaves m alone costs the half maxima and one compare.
    // (c > 0: the entry points require a positive scale.)
    // PRE (with FIXED only): s already holds the exponents c s - m
    template <bool FIXED, bool PRE = false>
    __device__ void softmax(const f32x16 (&s)[2], float c, typename TL::PFrag &pf)
    {
        if constexpr (!FIXED) {
            float t = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    t = fmaxf(t, s[kb][r]);
            if (__builtin_amdgcn_ballot_w64(t > thr) != 0) {
                const float mx = swap_halves_max(t) * c;
                const float m_new = fmaxf(m, mx);
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m - m_use);
                m = m_new;
                negm = -m_use;
                thr = (m_new + kLazyRescale) / c;
                l *= alpha;
#pragma unroll
                for (int db = 0; db < TL::DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        o[db][r] *= alpha;
            }
        }
        static_assert(FIXED || !PRE, "exponents are formed early only at a fixed offset");
        l += TL::template exp_tile<PRE>(s, c, negm, pf);
    }
};

// ---------------------------------------------------------------------------
// the attention kernel: GROUP selects the gathered within-group pass

// GA != 0 (bf16 dense pass only): the training-mode gate of the far pairs
// (Technical Summary, Gated Attention: s_ij = q_i.k_j * sigmoid(lambda a_ij)).
// This pass takes the far keys j <= i - gate_w only and writes a normalised
// partial O and LSE per row; the plain window pass then merges the window
// keys in.  Each stage also holds the tile's keys' assignment rows (bf16,
// GA = 16 or 32 groups wide, LDS-DMA'd by wavefront 0); the affinity tile
// a^T = A_k A_q^T is GA / 16 more MFMAs per 32 keys, and every score is
// multiplied by sigmoid(lambda a) before the softmax.
template <int D, bool BF16, bool GROUP, int GA>
__global__ __launch_bounds__(kThreads, kBlocksPerCU) void attn_kernel(Params p)
{
    // GA: 0, or the gated pass's padded assignment width (16 or 32 groups)
    constexpr bool GATED = GA != 0;
    constexpr int GCH = GATED ? GA / 8 : 1;  // 16-byte chunks per assignment row
    static_assert(!GATED || (BF16 && !GROUP), "the gate is a bf16 dense-pass feature");
    using TL = Tile<D, BF16>;
    using T = typename TL::T;
    constexpr int DB = TL::DB;
    // A stage holds one key tile: K, V^T, and the keys' positions, group bits
    // and the tile's valid-key count and owner-test flag.  bf16 runs the
    // staggered two-role schedule over four stages (loads two tiles ahead),
    // fp32 the plain double-buffered one.  Each part of each stage is its own LDS array, so
    // the compiler can tell an LDS-DMA write into one stage from a read of
    // another, and the K stages sit low enough for one lane offset plus an
    // immediate to address all of them.
    constexpr int NSTAGE = BF16 ? 4 : 2;
    constexpr int KEYS = 2 * kKeyTile + 4;
    constexpr int KB3 = NSTAGE >= 3 ? TL::K_BYTES : 16, VB3 = NSTAGE >= 3 ? TL::V_BYTES : 16;
    constexpr int KB4 = NSTAGE >= 4 ? TL::K_BYTES : 16, VB4 = NSTAGE >= 4 ? TL::V_BYTES : 16;
    __shared__ __attribute__((aligned(16))) char k_lds0[TL::K_BYTES];
    __shared__ __attribute__((aligned(16))) char k_lds1[TL::K_BYTES];
    __shared__ __attribute__((aligned(16))) char k_lds2[KB3];
    __shared__ __attribute__((aligned(16))) char k_lds3[KB4];
    __shared__ __attribute__((aligned(16))) char v_lds0[TL::V_BYTES];
    __shared__ __attribute__((aligned(16))) char v_lds1[TL::V_BYTES];
    __shared__ __attribute__((aligned(16))) char v_lds2[VB3];
    __shared__ __attribute__((aligned(16))) char v_lds3[VB4];
    __shared__ __attribute__((aligned(16))) int key_lds0[KEYS];
    __shared__ __attribute__((aligned(16))) int key_lds1[KEYS];
    __shared__ __attribute__((aligned(16))) int key_lds2[KEYS];
    __shared__ __attribute__((aligned(16))) int key_lds3[KEYS];
    constexpr int AB = GATED ? kKeyTile * GA * 2 : 16;
    __shared__ __attribute__((aligned(16))) char a_lds0[AB];
    __shared__ __attribute__((aligned(16))) char a_lds1[AB];
    __shared__ __attribute__((aligned(16))) char a_lds2[GATED ? AB : 16];
    __shared__ __attribute__((aligned(16))) char a_lds3[GATED ? AB : 16];
    // Stage<I> names the arrays of stage I at compile time.
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    struct Stage {
        char *k;
        char *v;
        int *key;
        char *a;
    };
    auto stage = [&](auto I) -> Stage {
        if constexpr (decltype(I)::value == 0)
            return Stage{k_lds0, v_lds0, key_lds0, a_lds0};
        else if constexpr (decltype(I)::value == 1)
            return Stage{k_lds1, v_lds1, key_lds1, a_lds1};
        else if constexpr (decltype(I)::value == 2)
            return Stage{k_lds2, v_lds2, key_lds2, a_lds2};
        else
            return Stage{k_lds3, v_lds3, key_lds3, a_lds3};
    };
    // the key sub-buckets a group-pass query tile visits (at most the codes
    // of one group), and the number of key tiles they hold
    __shared__ int sub_start[GROUP ? kMaxCodes : 1];
    __shared__ int sub_count[GROUP ? kMaxCodes : 1];
    __shared__ int sub_owner[GROUP ? kMaxCodes : 1];
    __shared__ int sub_tiles;

    const int lane = threadIdx.x % kWave;
    // (the wave index, and so the head, in scalar registers: the vector
    // registers it frees keep the gated and fp32 passes free of spills)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int m = lane % 32;
    const int h = lane / 32;

    // ---- which work item this block owns
    const int b_lin = (GROUP && p.order != nullptr) ? p.order[blockIdx.x]
                                                    : xcd_remap(blockIdx.x, gridDim.x);
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
    int g = 0, sbq = 0, e_start = 0;
    int64_t p_start = 0;
    int tile_rows;
    if (GROUP) {
        const int4 t = p.tiles[(int64_t)kvh * p.max_tiles + slot];
        sbq = t.x;
        e_start = t.y;
        tile_rows = t.z;
        g = t.w;
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
    // The gated pass covers only the far keys (j <= i - gate_w), all of them
    // gated; a plain window pass merges the window keys in afterwards.  Its
    // key range is the causal range of the query shifted back by gate_w, so
    // the masks and the tile range below use positions shifted by qsh.
    const int qsh = GATED ? p.gate_w : 0;

    typename TL::QFrag qf;
    TL::load_q(qf, static_cast<const T *>(p.q), ((int64_t)hq * p.n + qpos) * D, h);
    // gated pass: this lane's query's assignment, scaled by -lambda log2(e)
    // (the second copy of the packed rows), as the B operand of the affinity
    // product (groups 16j + 8h .. 16j + 8h + 7 for k-step j)
    bf16x8 aq[GATED ? GA / 16 : 1];
    // and the byte offset of its affinity A fragment in a stage: row sigma(m)
    // of the tile's keys, 16-byte chunk 2j + h swizzled by row bit 4 (the
    // chunk of k-step j and key block kb sits kb * 32 * GCH + 2j chunks on)
    const uint32_t a_off =
        GATED ? (uint32_t)((sigma(m) * GCH + (h ^ ((sigma(m) >> 4) & 1))) * 16) : 0u;
    if constexpr (GATED) {
        const bf16x8 *arow = static_cast<const bf16x8 *>(p.apack) +
                             ((int64_t)(p.hkv + kvh) * p.krows + qpos) * GCH;
#pragma unroll
        for (int j = 0; j < GA / 16; ++j)
            aq[j] = arow[2 * j + h];
    }

    // |q_i . k_j| <= |q_i| kmax for every key of this key/value head (the
    // largest of the per-block maxima the prepare pass left); the margin
    // covers the rounding of the norms and of the products' fp32 sums.
    // Lanes without a query row take -inf: they never bound the wavefront.
    float kmax = p.kpart[(int64_t)kvh * kNormBlocks + lane % kNormBlocks];
#pragma unroll
    for (int o = kNormBlocks / 2; o >= 1; o >>= 1)
        kmax = fmaxf(kmax, __shfl_xor(kmax, o));
    float qbound = qvalid ? __builtin_sqrtf(swap_halves_sum(TL::q_sq_half(qf))) : 0.f;
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1)
        qbound = fmaxf(qbound, __shfl_xor(qbound, o));
    // every scaled logit of this wavefront lies in [-mb, mb] (log2 units)
    const float mb = __uint_as_float(__builtin_amdgcn_readfirstlane(
        __float_as_uint(p.c * qbound * kmax * (1.f + 1.f / 256.f))));
    // With mb <= kFixedOffsetMax the offset m = mb needs no running max:
    // every P = 2^(c s - mb) lies in [2^-2mb, 1], inside the normal range of
    // fp32 and bf16, and fp32 keeps its relative precision at any scale.
    // (the gate lies in (0, 1), so the bound holds for gated logits too)
    const bool fixed_offset = BF16 && mb <= kFixedOffsetMax;
    const float rcp_c = 1.f / p.c;
    Acc<TL> acc;
    if (fixed_offset)
        acc.init_fixed(mb);
    else
        acc.init();

    // ---- key tile schedule
    const int w = p.window;
    uint32_t qlow = 0u;
    int64_t j_first = 0;
    int n_tiles_total = 0;
    if (GROUP) {
        qlow = gmh[qpos] & ((1u << g) - 1u);
        // Key sub-buckets of group g: a pair belongs to a lower group exactly
        // when the two tokens' lower sets meet, so a key sub-bucket whose
        // kept lower groups meet the query tile's is skipped whole.  Where a
        // lower set can hold more groups than its code keeps, a per-key test
        // on the group bits remains for the sub-buckets that keep all m.
        // Wave 0 walks the group's codes, 64 at a time; each lane counts the
        // keys at or before (last query position - w) of one kept code, and
        // the kept codes with keys are packed in order into LDS.
        if (wave == 0) {
            const int cm = code_members(p.K, p.topk);
            const LowerSet qs = decode_lower(g, sbq - group_base(g, cm));
            const int ncode = codes_of_group(g, cm);
            const int base = group_base(g, cm);
            const int32_t *offh =
                p.offsets + (int64_t)kvh * (num_subbuckets(p.K, p.topk) + 1);
            const int64_t lim = (int64_t)bq_max - w;
            const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
            int kept = 0, tiles = 0;
            if (lane == 0)
                sub_count[0] = 0;  // read by the iterator even when nothing is kept
            for (int c0 = 0; c0 < ncode; c0 += kWave) {
                const int c = c0 + lane;
                int cnt = 0, lo0 = 0, owner = 0;
                if (c < ncode) {
                    const LowerSet ks = decode_lower(g, c);
                    const bool meets = lower_sets_meet(qs, ks);
                    lo0 = offh[base + c];
                    const int hi0 = offh[base + c + 1];
                    if (!meets && hi0 > lo0) {
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
                tiles += (cnt + kKeyTile - 1) / kKeyTile;
            }
#pragma unroll
            for (int o = kWave / 2; o >= 1; o >>= 1)
                tiles += __shfl_xor(tiles, o);
            if (lane == 0)
                sub_tiles = tiles;
        }
        __syncthreads();
        n_tiles_total = __builtin_amdgcn_readfirstlane(sub_tiles);
    } else {
        const int64_t lo = max<int64_t>(0, p_start - qsh - w + 1);
        j_first = (lo / kKeyTile) * kKeyTile;
        const int64_t j_last = p_start + tile_rows - 1 - qsh;
        n_tiles_total = (w > 0 && (!GATED || j_last >= 0))
                            ? (int)((j_last - j_first) / kKeyTile + 1)
                            : 0;
    }

    // iterator over key tiles: (sub-bucket, tile) for the group pass.  The
    // current sub-bucket's start, count and owner flag are block-uniform and
    // kept in scalar registers; LDS is read only when the iterator steps to
    // the next sub-bucket, so the common step issues no LDS read (and no
    // wait) ahead of a tile's loads.
    int it_sub = 0, it_tile = 0;
    auto uniform = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    int sb_count = 0, sb_start = 0, sb_owner = 0;
    if (GROUP) {
        sb_count = uniform(sub_count[0]);
        sb_start = uniform(sub_start[0]);
        sb_owner = uniform(sub_owner[0]);
    }
    auto tile_origin = [&](int &valid, int &owner) -> int64_t {
        if (GROUP) {
            while (it_tile * kKeyTile >= sb_count) {
                ++it_sub;
                it_tile = 0;
                sb_count = uniform(sub_count[it_sub]);
                sb_start = uniform(sub_start[it_sub]);
                sb_owner = uniform(sub_owner[it_sub]);
            }
            valid = min(kKeyTile, sb_count - it_tile * kKeyTile);
            owner = sb_owner;
            return (int64_t)sb_start + (int64_t)it_tile * kKeyTile;
        } else {
            valid = kKeyTile;
            owner = 0;
            return j_first + (int64_t)it_tile * kKeyTile;
        }
    };

    typename TL::Staged st;
    TL::init_staging(st, p);
    typename TL::LdsOff lo;
    TL::init_lds_off(lo, m, h);
    // Positions (and, where an owner test is needed, group bits) of a tile's
    // keys live next to its K and V^T data.  They are read from global
    // memory into registers when the tile's loads are issued and written to
    // LDS only after the current tile's compute: writing them at once would
    // make the wavefront wait for every load issued before them.
    const int32_t *etk = GROUP ? p.etok + (int64_t)kvh * p.estride : nullptr;
    const uint32_t *egh = GROUP ? p.egm + (int64_t)kvh * p.estride : nullptr;
    auto load_keys = [&](int64_t origin, int valid, int owner, int &pos, uint32_t &gm) {
        pos = 0;
        gm = 0u;
        if (threadIdx.x < kKeyTile) {
            const int i = threadIdx.x;
            if (GROUP) {
                pos = i < valid ? etk[origin + i] : 0x7fffffff;
                gm = (i < valid && owner) ? egh[origin + i] : 0u;
            } else {
                pos = (int)(origin + i);
            }
        }
    };
    auto store_keys = [&](auto I, int pos, uint32_t gm, int valid, int owner) {
        int *kpos = stage(I).key;
        uint32_t *kgm = reinterpret_cast<uint32_t *>(kpos + kKeyTile);
        if (threadIdx.x < kKeyTile) {
            kpos[threadIdx.x] = pos;
            kgm[threadIdx.x] = gm;
        }
        if (threadIdx.x == 0) {
            kpos[2 * kKeyTile] = valid;
            kpos[2 * kKeyTile + 1] = owner;
        }
    };
    int cur_valid = 0, cur_owner = 0;
    if constexpr (!BF16) {
        if (n_tiles_total > 0) {
            const int64_t origin = tile_origin(cur_valid, cur_owner);
            int pos;
            uint32_t gm;
            load_keys(origin, cur_valid, cur_owner, pos, gm);
            TL::prefetch(st, p, kvh, origin, stage(I0{}).k, stage(I0{}).v);
            TL::land(st, stage(I0{}).k, stage(I0{}).v);
            store_keys(I0{}, pos, gm, cur_valid, cur_owner);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // Raw logits of one tile for this wavefront, masked where a pair falls
    // outside the pass: QK^T on the tile's K rows, then (only on tiles that
    // need it) the window / causal / owner tests on key positions in LDS.
    // (FIXED, gated pass: the gate and the fixed offset are folded in here,
    // and s leaves as the exponent c s g - m itself; see the gate below)
    // (j0_tile: the tile's first key position, used by the gated pass in
    // place of the stage's position list, which it does not fill)
    auto scores = [&](f32x16 (&s)[2], auto I, int valid, int owner, int j0_tile, auto fixed_tag) {
        constexpr bool FIXED = decltype(fixed_tag)::value;
        const int *kpos = stage(I).key;
        const uint32_t *kgm = reinterpret_cast<const uint32_t *>(kpos + kKeyTile);
        // Does any pair of this tile x wavefront need a mask?  Decided from
        // the tile's edge position, read before the products: the LDS read
        // then completes under the MFMAs instead of after them.
        // (no short-circuit: a branch here would make the wavefront wait
        // for the read before the products start)
        bool masked;
        if (GROUP) {
            const int last_key = kpos[valid - 1];  // valid >= 1
            masked = (valid < kKeyTile) | (owner != 0) | (last_key > wq_min - w);
        } else {
            const int j0 = GATED ? j0_tile : kpos[0];
            masked = !((j0 + kKeyTile - 1 <= wq_min - qsh) && (j0 > wq_max - qsh - w));
        }
        TL::qk(s, qf, stage(I).k, lo);
        if constexpr (GATED) {
            // every key of the gated pass is far: each score takes the gate
            // 1 / (1 + 2^a), a = -lambda log2(e) a_ij from the affinity
            // product (keys past the causal bound are masked below).  The
            // fragment address is formed here, by one add the compiler cannot
            // hoist: hoisted, it would hold one address per stage for the
            // whole loop and spill them.
            const uint32_t a_at = lds_add(lds_address(stage(I).a), a_off);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x16 a;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    a[r] = 0.f;
#pragma unroll
                for (int j = 0; j < GA / 16; ++j)
                    a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        lds_read16(a_at + (kb * 32 * GCH + 2 * j) * 16), aq[j], a, 0, 0, 0);
                if constexpr (FIXED) {
                    // c g = 1 / ((1 + 2^a) / c): the softmax's exponent
                    // c s g - m in two fused multiply-adds and a reciprocal
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        s[kb][r] = __builtin_fmaf(
                            s[kb][r],
                            __builtin_amdgcn_rcpf(
                                __builtin_fmaf(__builtin_amdgcn_exp2f(a[r]), rcp_c, rcp_c)),
                            acc.negm);
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        s[kb][r] *= __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(a[r]));
                }
            }
        }
        if (masked) {
            // Register r of lane half h holds key index kb*32 + h*16 + r of
            // the tile; compare that against per-lane bounds shifted by h*16.
            const int hshift = h * 16;
            int lo, hi;  // kept key indices: lo <= index <= hi
            if (GROUP) {
                // positions ascend inside a sub-bucket, so keys inside the
                // causal / window bound are a prefix of the tile's first
                // `valid` keys: count them with a binary search
                const int lim = qpos - w;
                int cnt = 0;  // ends at min(count, 63); the last probe covers 64
#pragma unroll
                for (int step = kKeyTile / 2; step >= 1; step >>= 1)
                    if (cnt + step - 1 < valid && kpos[cnt + step - 1] <= lim)
                        cnt += step;
                if (cnt < valid && kpos[cnt] <= lim)
                    ++cnt;
                lo = 0;
                hi = cnt - 1;
            } else {
                // window pass: key index i is position j0 + i
                const int j0 = GATED ? j0_tile : kpos[0];
                lo = qpos - qsh - w + 1 - j0;
                hi = qpos - qsh - j0;
            }
            if (!qvalid)
                hi = lo - 1;
            // owner test (top-k >= 3 only): bit i of ok is set when key i
            // shares no group below g with this lane's query.  A compact loop
            // over broadcast reads keeps this rare path light on registers.
            uint64_t ok = ~0ull;
            if (GROUP && owner) {
                ok = 0ull;
#pragma unroll 1
                for (int c = 0; c < kKeyTile / 4; ++c) {
                    const uint4 kg = reinterpret_cast<const uint4 *>(kgm)[c];
                    const uint32_t bits = ((kg.x & qlow) == 0u ? 1u : 0u) |
                                          ((kg.y & qlow) == 0u ? 2u : 0u) |
                                          ((kg.z & qlow) == 0u ? 4u : 0u) |
                                          ((kg.w & qlow) == 0u ? 8u : 0u);
                    ok |= (uint64_t)bits << (4 * c);
                }
            }
            const uint32_t ok_lo = (uint32_t)(ok >> hshift);          // keys h*16 + 0..31
            const uint32_t ok_hi = (uint32_t)(ok >> (32 + hshift));   // keys 32 + h*16 + 0..31
            lo -= hshift;
            hi -= hshift;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const uint32_t okb = kb ? ok_hi : ok_lo;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int idx = kb * 32 + r;
                    const bool keep = idx >= lo && idx <= hi && ((okb >> r) & 1u);
                    s[kb][r] = keep ? s[kb][r] : -INFINITY;
                }
            }
        }
    };

    if constexpr (!BF16) {
        // Plain schedule: compute on `cur` while the next tile streams into
        // `nxt`; one barrier per tile.  The two LDS buffers are distinct
        // arrays and the loop is unrolled by two, so each LDS read names one
        // buffer and each LDS write the other.
        auto step = [&](int t, auto CUR, auto NXT, auto FIXED) {
            const int valid = cur_valid;
            const int owner = cur_owner;
            const bool has_next = t + 1 < n_tiles_total;
            int nx_pos = 0;
            uint32_t nx_gm = 0u;
            if (has_next) {
                ++it_tile;
                const int64_t origin = tile_origin(cur_valid, cur_owner);
                load_keys(origin, cur_valid, cur_owner, nx_pos, nx_gm);
                TL::prefetch(st, p, kvh, origin, stage(NXT).k, stage(NXT).v);
            }
            // Every wavefront computes, including one whose rows all lie past
            // a ragged tile's end (its rows are masked and never stored): a
            // branch here would split the accumulator's live range and cost
            // a register copy of O per tile.
            f32x16 s[2];
            TL::refresh(lo);
            scores(s, CUR, valid, owner, 0, FIXED);
            typename TL::PFrag pf;
            acc.template softmax<decltype(FIXED)::value>(s, p.c, pf);
            TL::pv(acc.o, pf, stage(CUR).v, lo);
            if (has_next) {
                TL::land(st, stage(NXT).k, stage(NXT).v);
                store_keys(NXT, nx_pos, nx_gm, cur_valid, cur_owner);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        };
        auto loop = [&](auto FIXED) {
            for (int t = 0; t < n_tiles_total; t += 2) {
                step(t, I0{}, I1{}, FIXED);
                if (t + 1 < n_tiles_total)
                    step(t + 1, I1{}, I0{}, FIXED);
            }
        };
        // (one loop, the lazy rescale, keeps the fp32 registers within bounds)
        loop(std::false_type{});
    } else {
        // Two-role (staggered) schedule.  Each SIMD runs one wavefront of
        // role A (waves 0-3) and one of role B (waves 4-7); one block barrier
        // closes each tile interval u:
        //     A: QK(u), softmax(u), PV(u)
        //     B: softmax(u-1), PV(u-1), QK(u)
        // so within an interval A starts on the matrix cores while B starts
        // on the vector ALUs, and the SIMD overlaps the two.  B finishes the
        // last tile in one extra interval.  Tile u lives in stage u % 4; its
        // loads (K, V^T, key positions and group bits, all LDS-DMA) are
        // issued during interval u - 2 (after each role's first phase) and
        // awaited at the end of interval u - 1.  Both roles pass exactly one
        // barrier per interval.
        const int T = n_tiles_total;
        // LDS-DMA loads each wavefront issues per tile (waited on by count)
        // Role B's chain (softmax, PV, QK back to back) sets each interval's
        // length while role A waits at the barrier, so role A issues all of a
        // tile's K / V^T loads and role B none.
        const bool role_a_wave = __builtin_amdgcn_readfirstlane(wave) < kWavesPerRole;
        constexpr int DMA_KV = 2 * TL::LOADS;  // per role-A wavefront
        const bool key_wave = GROUP && __builtin_amdgcn_readfirstlane(wave) == 0;
        // gated pass: wavefront 0 also loads the keys' assignment rows
        // (GA * 128 bytes per tile, one LDS-DMA load per KB).  LDS slot P
        // holds chunk (P % GCH) ^ ((row >> 4) & 1) of row P / GCH, so the MFMA
        // reads of rows sigma(m) fall in distinct banks.
        constexpr int DMA_A = GATED ? kKeyTile * GA * 2 / 1024 : 0;
        const bool a_wave = GATED && __builtin_amdgcn_readfirstlane(wave) == 0;
        // valid-key count and owner flag of the tile in each stage: set by
        // every wavefront when it issues the tile's loads (the iterator runs
        // in each wavefront), read when the tile is computed; stage indices
        // are compile-time, so the ring stays in scalar registers
        int ring_valid[NSTAGE] = {}, ring_owner[NSTAGE] = {}, ring_origin[NSTAGE] = {};
        // (is_a: this wavefront's role, a compile-time constant inside the
        // role loops, so that role B's copies carry no load code or branches;
        // the gated pass keeps the run-time test, with which its registers
        // fit the loop without reloads)
        auto issue = [&](auto I, bool is_a) {
            int nv, no;
            const int64_t origin = tile_origin(nv, no);
            if (is_a)
                TL::prefetch(st, p, kvh, origin, stage(I).k, stage(I).v);
            int *kp = stage(I).key;
            if (GROUP) {
                if (is_a && key_wave) {
                    dma4(etk + origin, (uint32_t)lane * 4u, lds_address(kp));
                    dma4(egh + origin, (uint32_t)lane * 4u, lds_address(kp) + kKeyTile * 4);
                }
            } else if (!GATED && is_a && threadIdx.x < kKeyTile) {
                kp[threadIdx.x] = (int)(origin + threadIdx.x);
            }
            if constexpr (GATED) {
                if (a_wave) {
                    const char *abase = static_cast<const char *>(p.apack) +
                                        ((int64_t)kvh * p.krows + origin) * GA * 2;
                    // slot P = 64i + lane takes byte (P ^ b) * 16 of the
                    // rows, b = bit 4 of its row P / GCH: lane bit 5 for
                    // 16-group rows, i odd for 32-group rows.  The 1 KB step
                    // goes to the scalar base, so the lane keeps one or two
                    // offsets, not one per load.
#pragma unroll
                    for (int i = 0; i < DMA_A; ++i) {
                        const uint32_t b = GCH == 2 ? ((uint32_t)lane >> 5) & 1u : (uint32_t)i & 1u;
                        dma16(abase + i * 1024, (16u * (uint32_t)lane) ^ (b << 4),
                              lds_address(stage(I).a) + i * 1024);
                    }
                }
            }
            ring_valid[decltype(I)::value] = nv;
            ring_owner[decltype(I)::value] = no;
            ring_origin[decltype(I)::value] = (int)origin;
        };
        // end of an interval: everything but the newest tile's loads landed,
        // this interval's LDS traffic done, then the block barrier
        // (s_waitcnt immediates on gfx950: vmcnt in bits 3:0, expcnt 6:4,
        // lgkmcnt 11:8; 0x70 | n = "vmcnt(n) lgkmcnt(0)", expcnt untouched.
        // The builtin, unlike inline asm, is visible to the compiler's own
        // wait tracking, so it adds no waits of its own for these loads.)
        auto close_interval = [&](bool newest_in_flight, bool is_a) {
            if (!newest_in_flight)
                __builtin_amdgcn_s_waitcnt(0x70);
            else if (is_a && key_wave)
                __builtin_amdgcn_s_waitcnt(0x70 | (DMA_KV + 2));
            else if (a_wave)
                __builtin_amdgcn_s_waitcnt(0x70 | (DMA_KV + DMA_A));
            else if (is_a)
                __builtin_amdgcn_s_waitcnt(0x70 | DMA_KV);
            else
                __builtin_amdgcn_s_waitcnt(0x70);
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        static_assert(!BF16 || TL::LOADS == 2 || TL::LOADS == 4, "vmcnt counts assume 2-4 loads");
        static_assert(DMA_KV + DMA_A <= 15, "vmcnt immediate holds 4 bits here");

        // prologue: tiles 0 and 1 (tile 0's iterator position is current)
        if (T > 0)
            issue(I0{}, role_a_wave);
        if (T > 1) {
            ++it_tile;
            issue(I1{}, role_a_wave);
        }
        __builtin_amdgcn_s_waitcnt(0x70);
        __syncthreads();

        auto run = [&](auto role_tag, auto fixed_tag) {
            constexpr bool ROLE_A = decltype(role_tag)::value;
            constexpr bool FIXED = decltype(fixed_tag)::value;
            f32x16 s[2];
            typename TL::PFrag pf;
            auto interval = [&](int u, auto PREV, auto CUR, auto AHEAD, auto FIRST) {
                // The loads of tile u + 2 go out after each role's first
                // phase, not at the interval's start: both wavefronts of a
                // SIMD leave the barrier together, and issuing then would
                // hold both off the matrix core at once.
                const bool ahead = u + 2 < T;
                auto issue_ahead = [&] {
                    if (ahead) {
                        ++it_tile;
                        issue(AHEAD, GATED ? role_a_wave : ROLE_A);
                    }
                };
                TL::refresh(lo);
                if (ROLE_A) {
                    if (u < T) {
                        scores(s, CUR, ring_valid[decltype(CUR)::value],
                               ring_owner[decltype(CUR)::value],
                               ring_origin[decltype(CUR)::value], fixed_tag);
                        issue_ahead();
                        acc.template softmax<FIXED, GATED && FIXED>(s, p.c, pf);
                        TL::pv(acc.o, pf, stage(CUR).v, lo);
                    }
                } else {
                    if constexpr (decltype(FIRST)::value) {
                        issue_ahead();
                    } else {
                        acc.template softmax<FIXED, GATED && FIXED>(s, p.c, pf);
                        issue_ahead();
                        TL::pv(acc.o, pf, stage(PREV).v, lo);
                    }
                    if (u < T) {
                        scores(s, CUR, ring_valid[decltype(CUR)::value],
                               ring_owner[decltype(CUR)::value],
                               ring_origin[decltype(CUR)::value], fixed_tag);
                    }
                }
                close_interval(ahead, GATED ? role_a_wave : ROLE_A);
            };
            // interval 0 (role B has no previous tile to finish) is peeled
            // off, so that every interval of the unrolled loop has one shape
            // (an alternative branch there splits the accumulators' live
            // ranges and spills them)
            interval(0, I3{}, I0{}, I2{}, std::true_type{});
            for (int u = 1; u <= T; u += 4) {
                interval(u, I0{}, I1{}, I3{}, std::false_type{});
                if (u + 1 <= T)
                    interval(u + 1, I1{}, I2{}, I0{}, std::false_type{});
                if (u + 2 <= T)
                    interval(u + 2, I2{}, I3{}, I1{}, std::false_type{});
                if (u + 3 <= T)
                    interval(u + 3, I3{}, I0{}, I2{}, std::false_type{});
            }
        };
        if (__builtin_amdgcn_readfirstlane(wave) < kWavesPerRole) {
            if (fixed_offset)
                run(std::true_type{}, std::true_type{});
            else
                run(std::true_type{}, std::false_type{});
        } else {
            if (fixed_offset)
                run(std::false_type{}, std::true_type{});
            else
                run(std::false_type{}, std::false_type{});
        }
    }

    if (!wave_active)
        return;

    // ---- epilogue
    const float l_tot = swap_halves_sum(acc.l);
    // log2-domain log-sum-exp of the scaled logits
    const float lse2 = (l_tot > 0.f) ? acc.m + __builtin_amdgcn_logf(l_tot) : -INFINITY;

    if (GROUP || GATED) {
        // normalised partial O (in the I/O dtype: bf16 for bf16 inputs, as
        // the merged output is) and natural-log LSE at the query's entry
        // (the gated pass: at its row, for the window pass to merge)
        if (!qvalid)
            return;
        const int64_t e = GROUP ? (int64_t)(e_start + qr) : (int64_t)qpos;
        const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
        T *po = static_cast<T *>(p.part_o) + ((int64_t)hq * p.E + e) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                T *dst = po + db * 32 + a * 8 + h * 4;
                if constexpr (BF16) {
                    bf16x4 v;
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        v[x] = (__bf16)(acc.o[db][a * 4 + x] * inv);
                    *reinterpret_cast<bf16x4 *>(dst) = v;
                } else {
                    float4 v;
                    v.x = acc.o[db][a * 4 + 0] * inv;
                    v.y = acc.o[db][a * 4 + 1] * inv;
                    v.z = acc.o[db][a * 4 + 2] * inv;
                    v.w = acc.o[db][a * 4 + 3] * inv;
                    *reinterpret_cast<float4 *>(dst) = v;
                }
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
        const T *po = static_cast<const T *>(p.part_o) + ((int64_t)hq * p.E + ent) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const T *src = po + db * 32 + a * 8 + h * 4;
                if constexpr (BF16) {
                    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(src);
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        res[db][a * 4 + x] += a_s * (float)v[x];
                } else {
                    const float4 v = *reinterpret_cast<const float4 *>(src);
                    res[db][a * 4 + 0] += a_s * v.x;
                    res[db][a * 4 + 1] += a_s * v.y;
                    res[db][a * 4 + 2] += a_s * v.z;
                    res[db][a * 4 + 3] += a_s * v.w;
                }
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

// Largest Euclidean norm of the rows of x [H][n][D] (the keys), as
// kNormBlocks partial maxima per head: kpart[h][b] covers rows b, b + B, ...
// of head h (B = rows per block pass times kNormBlocks).  Each row is read by
// CH consecutive lanes, 16 bytes each.
template <typename T, int D>
__global__ __launch_bounds__(256) void key_norm_kernel(const T *__restrict__ x, int64_t n,
                                                       float *__restrict__ kpart)
{
    constexpr int CH = D * (int)sizeof(T) / 16;  // 8, 16 or 32 lanes per row
    constexpr int RPB = 256 / CH;                // rows per block pass
    const int h = blockIdx.y;
    const int c = threadIdx.x % CH;
    float best = 0.f;
    for (int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / CH; r < n;
         r += (int64_t)gridDim.x * RPB) {
        const uint4 v = reinterpret_cast<const uint4 *>(x + ((int64_t)h * n + r) * D)[c];
        float ss = 0.f;
        if constexpr (sizeof(T) == 2) {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xffff0000u);
                ss = __builtin_fmaf(lo, lo, ss);
                ss = __builtin_fmaf(hi, hi, ss);
            }
        } else {
            const float f[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                                __uint_as_float(v.w)};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ss = __builtin_fmaf(f[i], f[i], ss);
        }
#pragma unroll
        for (int o = 1; o < CH; o <<= 1)  // the CH lanes of one row
            ss += __shfl_xor(ss, o);
        best = fmaxf(best, ss);
    }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1)
        best = fmaxf(best, __shfl_xor(best, o));
    __shared__ float wmax[256 / kWave];
    if (threadIdx.x % kWave == 0)
        wmax[threadIdx.x / kWave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = wmax[0];
        for (int i = 1; i < 256 / kWave; ++i)
            b = fmaxf(b, wmax[i]);
        kpart[(int64_t)h * kNormBlocks + blockIdx.x] = __builtin_sqrtf(b);
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

// Bucket-order copies padded to a whole extra key tile: etok[h][e] =
// tokens[h][e] and egm[h][e] = gmask[h][tokens[h][e]] (the group bits of every
// entry), with INT_MAX / 0 past the last entry, so a key tile's positions and
// group bits load as one contiguous block that never leaves the array.
__global__ __launch_bounds__(256) void gather_entries_kernel(const uint32_t *__restrict__ gmask,
                                                             const int32_t *__restrict__ tokens,
                                                             int64_t n, int64_t E, int64_t estride,
                                                             int H, int32_t *__restrict__ etok,
                                                             uint32_t *__restrict__ egm)
{
    const int64_t total = (int64_t)H * estride;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t h = i / estride;
        const int64_t e = i % estride;
        if (e < E) {
            const int32_t t = tokens[h * E + e];
            etok[i] = t;
            egm[i] = gmask[h * n + t];
        } else {
            etok[i] = 0x7fffffff;
            egm[i] = 0u;
        }
    }
}

// Tile list of the group pass: for routing head h, every sub-bucket cut into
// query tiles of `rows` entries, last tile (latest positions, most keys)
// first.  tiles[h][i] = {sub-bucket, first entry, entry count, group}.
//
// With `work` given, each tile also gets an estimate of its key work, in
// [0, 1]: (last query position - w) / n times the share of the head's
// entries in the key sub-buckets its block visits (those whose lower sets
// miss the tile's), which is the block's key count if keys spread evenly
// over positions.  order_kernel sorts blocks by it.
__global__ __launch_bounds__(256) void plan_kernel(const int32_t *__restrict__ offsets, int K,
                                                   int topk, int rows, int max_tiles,
                                                   int4 *__restrict__ tiles,
                                                   int32_t *__restrict__ ntiles,
                                                   const int32_t *__restrict__ tokens, int64_t n,
                                                   int64_t E, int window,
                                                   float *__restrict__ work)
{
    __shared__ int start[kMaxSubbuckets + 1];
    __shared__ int compat[kMaxSubbuckets];
    const int nsb = num_subbuckets(K, topk);
    const int cm = code_members(K, topk);
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
    if (work != nullptr) {
        // entries of the key sub-buckets a query sub-bucket's blocks visit
        for (int sb = threadIdx.x; sb < nsb; sb += blockDim.x) {
            int g = 0;
            while (g + 1 < K && group_base(g + 1, cm) <= sb)
                ++g;
            const int gb = group_base(g, cm);
            const LowerSet qs = decode_lower(g, sb - gb);
            int c = 0;
            for (int code = 0; code < codes_of_group(g, cm); ++code) {
                if (!lower_sets_meet(qs, decode_lower(g, code)))
                    c += off[gb + code + 1] - off[gb + code];
            }
            compat[sb] = c;
        }
    }
    __syncthreads();
    int4 *th = tiles + (int64_t)h * max_tiles;
    const int32_t *tok = tokens + (int64_t)h * E;
    int g = 0;
    for (int sb = 0; sb < nsb; ++sb) {
        while (g + 1 < K && group_base(g + 1, cm) <= sb)
            ++g;
        const int nt = start[sb + 1] - start[sb];
        const int cnt = off[sb + 1] - off[sb];
        for (int j = threadIdx.x; j < nt; j += blockDim.x) {
            const int jj = nt - 1 - j;
            const int first = off[sb] + jj * rows, count = min(rows, cnt - jj * rows);
            th[start[sb] + j] = make_int4(sb, first, count, g);
            if (work != nullptr) {
                const int64_t far = (int64_t)tok[first + count - 1] - window;
                work[(int64_t)h * max_tiles + start[sb] + j] =
                    far > 0 ? (float)far / (float)n * ((float)compat[sb] / (float)E) : 0.f;
            }
        }
    }
}

// Group-pass blocks in descending order of estimated work (a counting sort
// over kOrderBins bins), so that the longest blocks start first and the
// grid's tail is short; slots past a head's tile count go last, and the
// grid's padding gets `total` (those blocks exit at once).  Blocks are
// independent, so the order changes no result.  One block of 1024 threads.
constexpr int kOrderBins = 4096;
constexpr int kOrderMaxBlocks = 16384;  // larger grids keep the XCD-contiguous order
__global__ __launch_bounds__(1024) void order_kernel(const float *__restrict__ work,
                                                     const int32_t *__restrict__ ntiles, int nhg,
                                                     int max_tiles, int total, int grid,
                                                     int32_t *__restrict__ order)
{
    __shared__ int hist[kOrderBins + 1];  // last bin: empty slots
    __shared__ int part[1024];
    const int tid = threadIdx.x;
    for (int i = tid; i <= kOrderBins; i += 1024)
        hist[i] = 0;
    __syncthreads();
    auto bin_of = [&](int b) {
        const int slot = b % max_tiles;
        const int kvh = b / max_tiles / nhg;
        if (slot >= ntiles[kvh])
            return kOrderBins;
        const int q = (int)(work[(int64_t)kvh * max_tiles + slot] * (float)(kOrderBins - 1));
        return kOrderBins - 1 - max(0, min(kOrderBins - 1, q));  // heavier first
    };
    for (int b = tid; b < total; b += 1024)
        atomicAdd(&hist[bin_of(b)], 1);
    __syncthreads();
    // exclusive scan of the kOrderBins + 1 counts: 4 or 5 bins per thread,
    // then the threads' sums
    constexpr int PER = (kOrderBins + 1 + 1023) / 1024;
    int local = 0;
    for (int i = 0; i < PER; ++i) {
        const int k = tid * PER + i;
        if (k <= kOrderBins)
            local += hist[k];
    }
    part[tid] = local;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
        const int v = tid >= o ? part[tid - o] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int acc = part[tid] - local;
    for (int i = 0; i < PER; ++i) {
        const int k = tid * PER + i;
        if (k <= kOrderBins) {
            const int c = hist[k];
            hist[k] = acc;
            acc += c;
        }
    }
    __syncthreads();
    for (int b = tid; b < total; b += 1024)
        order[atomicAdd(&hist[bin_of(b)], 1)] = b;
    for (int b = total + tid; b < grid; b += 1024)
        order[b] = total;
}

// ---------------------------------------------------------------------------
// host side

struct Layout {
    int hpb, nhg, rows_group, max_tiles;
    int64_t E, e_pad, n_pad;
    size_t kb, vb, kp, vt, etok, egm, po, pl, tiles, ntiles, kpart, work, order, total;
    int group_blocks;   // hkv x head groups x max_tiles
    bool ordered;       // group blocks sorted by estimated work (small grids)
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
    L.max_tiles = (int)((L.E + L.rows_group - 1) / L.rows_group) + num_subbuckets(sh.K, sh.topk);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    L.kb = take((size_t)sh.hkv * L.e_pad * sh.d * es);
    L.vb = take((size_t)sh.hkv * L.e_pad * sh.d * es);
    L.kp = take(sh.dt == FOCUS_BF16 ? (size_t)sh.hkv * L.n_pad * sh.d * 2 : 0);
    L.vt = take(sh.dt == FOCUS_BF16 ? (size_t)sh.hkv * sh.d * L.n_pad * 2 : 0);
    L.etok = take((size_t)sh.hkv * L.e_pad * 4);
    L.egm = take((size_t)sh.hkv * L.e_pad * 4);
    L.po = take((size_t)sh.hq * L.E * sh.d * es);  // partial O in the I/O dtype
    L.pl = take((size_t)sh.hq * L.E * 4);
    L.tiles = take((size_t)sh.hkv * L.max_tiles * sizeof(int4));
    L.ntiles = take((size_t)sh.hkv * sizeof(int32_t));
    L.kpart = take((size_t)sh.hkv * kNormBlocks * sizeof(float));
    L.group_blocks = sh.hkv * L.nhg * L.max_tiles;
    L.ordered = L.group_blocks <= kOrderMaxBlocks;
    L.work = take(L.ordered ? (size_t)sh.hkv * L.max_tiles * sizeof(float) : 0);
    L.order = take(L.ordered ? (size_t)(L.group_blocks + kXcds) * sizeof(int32_t) : 0);
    L.total = off;
    return L;
}

template <int D, bool BF16, bool GROUP, int GA = 0>
hipError_t launch_attn_kernel(const Params &p, hipStream_t s)
{
    const int grid = (p.total_blocks + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((attn_kernel<D, BF16, GROUP, GA>), dim3(grid), dim3(kThreads), 0, s, p);
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

hipError_t launch_key_norms(int d, bool bf16, const void *k, int64_t n, int H, float *kpart,
                            hipStream_t s)
{
    const dim3 grid(kNormBlocks, (unsigned)H);
    if (bf16) {
        auto K = static_cast<const __bf16 *>(k);
        if (d == 64)
            hipLaunchKernelGGL((key_norm_kernel<__bf16, 64>), grid, dim3(256), 0, s, K, n, kpart);
        else
            hipLaunchKernelGGL((key_norm_kernel<__bf16, 128>), grid, dim3(256), 0, s, K, n, kpart);
    } else {
        auto K = static_cast<const float *>(k);
        if (d == 64)
            hipLaunchKernelGGL((key_norm_kernel<float, 64>), grid, dim3(256), 0, s, K, n, kpart);
        else
            hipLaunchKernelGGL((key_norm_kernel<float, 128>), grid, dim3(256), 0, s, K, n, kpart);
    }
    return hipGetLastError();
}

// bytes of the key-norm partial maxima, at the end of the dense workspaces
size_t kpart_bytes(int hkv) { return align_up((size_t)hkv * kNormBlocks * sizeof(float), 256); }

}  // namespace

size_t attn_workspace_bytes(const AttnShape &sh) { return make_layout(sh).total; }

size_t dense_workspace_bytes(const AttnShape &sh)
{
    if (sh.dt != FOCUS_BF16)
        return kpart_bytes(sh.hkv);
    const int64_t n_pad = (sh.n + kKeyTile - 1) / kKeyTile * kKeyTile + kKeyTile;
    // transposed values, a zero-padded copy of the keys, the key norms
    return 2 * align_up((size_t)sh.hkv * sh.d * n_pad * 2, 256) + kpart_bytes(sh.hkv);
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
            if (e == hipSuccess)
                e = launch_gather(sh.d, K, (const int32_t *)nullptr, sh.n, sh.n, L.n_pad, sh.hkv,
                                  reinterpret_cast<__bf16 *>(w + L.kp), s);
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
            const int64_t total = (int64_t)sh.hkv * L.e_pad;
            const int blocks = (int)std::min<int64_t>((total + 255) / 256, 8192);
            hipLaunchKernelGGL(gather_entries_kernel, dim3(blocks), dim3(256), 0, s, gmask, tokens,
                               sh.n, L.E, L.e_pad, sh.hkv, reinterpret_cast<int32_t *>(w + L.etok),
                               reinterpret_cast<uint32_t *>(w + L.egm));
            e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
        hipLaunchKernelGGL(plan_kernel, dim3(sh.hkv), dim3(256), 0, s, offsets, sh.K, sh.topk,
                           L.rows_group, L.max_tiles, tiles, ntiles, tokens, sh.n, L.E,
                           (int)std::min<int64_t>(sh.window, sh.n),
                           L.ordered ? reinterpret_cast<float *>(w + L.work) : nullptr);
        if (L.ordered)
            hipLaunchKernelGGL(order_kernel, dim3(1), dim3(1024), 0, s,
                               reinterpret_cast<const float *>(w + L.work), ntiles, L.nhg,
                               L.max_tiles, L.group_blocks,
                               (L.group_blocks + kXcds - 1) / kXcds * kXcds,
                               reinterpret_cast<int32_t *>(w + L.order));
        e = hipGetLastError();
        if (e == hipSuccess)
            e = launch_key_norms(sh.d, bf16, k, sh.n, sh.hkv,
                                 reinterpret_cast<float *>(w + L.kpart), s);
        if (e != hipSuccess)
            return e;
    }

    Params p = base_params(sh, L);
    p.q = q;
    p.tokens = tokens;
    p.offsets = offsets;
    p.gmask = gmask;
    p.etok = reinterpret_cast<const int32_t *>(w + L.etok);
    p.egm = reinterpret_cast<const uint32_t *>(w + L.egm);
    p.estride = L.e_pad;
    p.part_o = w + L.po;
    p.part_lse = reinterpret_cast<float *>(w + L.pl);
    p.slot_entry = slot_entry;
    p.out = out;
    p.lse = lse;
    p.kpart = reinterpret_cast<const float *>(w + L.kpart);

    if (parts & FOCUS_PART_GROUP) {
        Params g = p;
        g.kmat = w + L.kb;
        g.vmat = w + L.vb;
        g.krows = L.e_pad;
        g.vcols = L.e_pad;
        g.tiles = tiles;
        g.ntiles = ntiles;
        g.max_tiles = L.max_tiles;
        g.total_blocks = L.group_blocks;
        g.order = L.ordered ? reinterpret_cast<const int32_t *>(w + L.order) : nullptr;
        e = dispatch_attn<true>(sh.d, bf16, g, s);
        if (e != hipSuccess)
            return e;
    }
    if (parts & FOCUS_PART_WINDOW) {
        Params wp = p;
        wp.kmat = bf16 ? (const void *)(w + L.kp) : k;
        wp.vmat = bf16 ? (const void *)(w + L.vt) : v;
        wp.krows = bf16 ? L.n_pad : sh.n;
        wp.vcols = L.n_pad;
        wp.merge = 1;
        wp.row_tiles = (int)((sh.n + (kRowsPerBlock / L.hpb) - 1) / (kRowsPerBlock / L.hpb));
        wp.total_blocks = sh.hkv * L.nhg * wp.row_tiles;
        e = dispatch_attn<false>(sh.d, bf16, wp, s);
    }
    return e;
}

namespace {
// The assignment padded to ga groups (16 or 32) and to n_pad zero rows per
// head, twice: [2][hkv][n_pad][ga] bf16.  The first copy holds A itself (the
// keys' side of the affinity product), the second -lambda log2(e) A (the
// queries' side), each rounded to bf16 once, so that the product lands
// directly in the exponent of the gate's 2^(-lambda log2(e) a).
__global__ __launch_bounds__(256) void gate_pack_kernel(const float *__restrict__ assign,
                                                        int64_t n, int64_t n_pad, int K, int ga,
                                                        int64_t total, float neg_lam2,
                                                        __bf16 *__restrict__ apack)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total)
        return;
    const int g = (int)(idx % ga);
    const int64_t ht = idx / ga;
    const int64_t h = ht / n_pad, t = ht % n_pad;
    const float x = (t < n && g < K) ? assign[(h * n + t) * K + g] : 0.f;
    apack[idx] = (__bf16)x;
    apack[total + idx] = (__bf16)(neg_lam2 * x);
}

// slot[h][i] = i: each row's one partial (the gated far pass's) sits at the
// row itself, for the window pass's merge
__global__ __launch_bounds__(256) void row_slots_kernel(int64_t n, int64_t total,
                                                        int32_t *__restrict__ slot)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx < total)
        slot[idx] = (int32_t)(idx % n);
}
}  // namespace

size_t gated_dense_workspace_bytes(const AttnShape &sh)
{
    const int64_t n_pad = (sh.n + kKeyTile - 1) / kKeyTile * kKeyTile + kKeyTile;
    return dense_workspace_bytes(sh) +
           align_up((size_t)2 * sh.hkv * n_pad * kGateGroups * 2, 256) +
           align_up((size_t)sh.hkv * sh.n * 4, 256);
}

namespace {
// the key norms sit at the end of a dense workspace of `bytes` bytes
float *dense_kpart(void *ws, size_t bytes, int hkv)
{
    return reinterpret_cast<float *>(static_cast<char *>(ws) + bytes - kpart_bytes(hkv));
}
}  // namespace

hipError_t launch_gated_dense(const AttnShape &sh, const void *q, const void *k, const void *v,
                              const float *assign, float lambda, void *out, float *lse, void *ws,
                              hipStream_t s)
{
    AttnShape d = sh;
    d.window = sh.n;
    d.K = 1;
    d.topk = 1;
    Layout L = make_layout(d);
    const int64_t n_pad = (sh.n + kKeyTile - 1) / kKeyTile * kKeyTile + kKeyTile;
    const size_t half = align_up((size_t)sh.hkv * sh.d * n_pad * 2, 256);
    __bf16 *vt = static_cast<__bf16 *>(ws);
    __bf16 *kp = reinterpret_cast<__bf16 *>(static_cast<char *>(ws) + half);
    __bf16 *apack = reinterpret_cast<__bf16 *>(static_cast<char *>(ws) + 2 * half);
    int32_t *slots = reinterpret_cast<int32_t *>(
        static_cast<char *>(ws) + 2 * half +
        align_up((size_t)2 * sh.hkv * n_pad * kGateGroups * 2, 256));
    hipError_t e = launch_transpose(sh.d, static_cast<const __bf16 *>(v), nullptr, sh.n, sh.n,
                                    n_pad, sh.hkv, vt, s);
    if (e == hipSuccess)
        e = launch_gather(sh.d, static_cast<const __bf16 *>(k), (const int32_t *)nullptr, sh.n,
                          sh.n, n_pad, sh.hkv, kp, s);
    if (e != hipSuccess)
        return e;
    const int ga = sh.K > 16 ? 32 : 16;
    const int64_t total = (int64_t)sh.hkv * n_pad * ga;
    hipLaunchKernelGGL(gate_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       assign, sh.n, n_pad, sh.K, ga, total, -lambda * kLog2e, apack);
    const int64_t nslots = (int64_t)sh.hkv * sh.n;
    if (nslots > 0)
        hipLaunchKernelGGL(row_slots_kernel, dim3((unsigned)((nslots + 255) / 256)), dim3(256), 0,
                           s, sh.n, nslots, slots);
    e = hipGetLastError();
    float *kpart = dense_kpart(ws, gated_dense_workspace_bytes(sh), sh.hkv);
    if (e == hipSuccess)
        e = launch_key_norms(sh.d, true, k, sh.n, sh.hkv, kpart, s);
    if (e != hipSuccess)
        return e;
    Params p = base_params(d, L);
    p.q = q;
    p.kmat = kp;
    p.vmat = vt;
    p.krows = n_pad;
    p.vcols = n_pad;
    p.merge = 0;
    p.out = out;
    p.lse = lse;
    p.row_tiles = (int)((sh.n + (kRowsPerBlock / L.hpb) - 1) / (kRowsPerBlock / L.hpb));
    p.total_blocks = sh.hkv * L.nhg * p.row_tiles;
    p.apack = apack;
    p.gate_w = (int)std::min<int64_t>(sh.window, sh.n);
    p.kpart = kpart;
    // far pass (gated scores): its normalised partial O and LSE go to out
    // and lse, which the window pass reads back and overwrites row by row
    p.part_o = out;
    p.part_lse = lse;
    if (ga == 16)
        e = sh.d == 64 ? launch_attn_kernel<64, true, false, 16>(p, s)
                       : launch_attn_kernel<128, true, false, 16>(p, s);
    else
        e = sh.d == 64 ? launch_attn_kernel<64, true, false, 32>(p, s)
                       : launch_attn_kernel<128, true, false, 32>(p, s);
    if (e != hipSuccess)
        return e;
    // window pass (plain scores over i - w < j <= i) with the merge
    Params pw = p;
    pw.window = p.gate_w;
    pw.merge = 1;
    pw.slot_entry = slots;
    pw.apack = nullptr;
    return sh.d == 64 ? launch_attn_kernel<64, true, false>(pw, s)
                      : launch_attn_kernel<128, true, false>(pw, s);
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
    const size_t half = align_up((size_t)sh.hkv * sh.d * n_pad * 2, 256);
    __bf16 *vt = static_cast<__bf16 *>(ws);
    __bf16 *kp = reinterpret_cast<__bf16 *>(static_cast<char *>(ws) + half);
    if (bf16) {
        e = launch_transpose(sh.d, static_cast<const __bf16 *>(v), nullptr, sh.n, sh.n, n_pad,
                             sh.hkv, vt, s);
        if (e == hipSuccess)
            e = launch_gather(sh.d, static_cast<const __bf16 *>(k), (const int32_t *)nullptr,
                              sh.n, sh.n, n_pad, sh.hkv, kp, s);
        if (e != hipSuccess)
            return e;
    }
    float *kpart = dense_kpart(ws, dense_workspace_bytes(sh), sh.hkv);
    e = launch_key_norms(sh.d, bf16, k, sh.n, sh.hkv, kpart, s);
    if (e != hipSuccess)
        return e;
    Params p = base_params(d, L);
    p.q = q;
    p.kpart = kpart;
    p.kmat = bf16 ? (const void *)kp : k;
    p.vmat = bf16 ? (const void *)vt : v;
    p.krows = bf16 ? n_pad : sh.n;
    p.vcols = n_pad;
    p.merge = 0;
    p.out = out;
    p.lse = lse;
    p.row_tiles = (int)((sh.n + (kRowsPerBlock / L.hpb) - 1) / (kRowsPerBlock / L.hpb));
    p.total_blocks = sh.hkv * L.nhg * p.row_tiles;
    return dispatch_attn<false>(sh.d, bf16, p, s);
}

}  // namespace focus
