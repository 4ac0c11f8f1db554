/*
 * Focus attention forward: plain CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the
 * GPU library.
 *
 * Source of the method: "Why Attend to Everything? Focus is the Key"
 * (arXiv 2604.03260), as summarised on the gist.science page, Technical
 * Summary section 2 "Methodology: Focus", bullets Learnable Centroids,
 * Token Grouping, Gated Attention (Local / Distant) and Inference
 * Efficiency (Top-k); and on the jindou-blog deep read, method bullets
 * (K centroids per layer, 16-dimensional routing, dot-product assignment,
 * exact softmax in the local window and inside groups).
 *
 * What is computed, written out from those passages:
 *   route : score(t, g) = <r_t, c_g> over the 16 routing dimensions; each
 *           token keeps its top-k groups G(t).
 *   attend: A(i) = { j <= i : i - j < w  or  G(i) and G(j) share a group }
 *           and the output is the exact softmax over A(i).
 *   bucket: the (token, group) entries sorted by group g, then by the
 *           token's lower set inside g (its groups below g: the lowest
 *           two or three of them, as a code), then by position.
 *   project: r_t = W x_t, the hidden state projected into the routing space
 *           by one 16 x d_model matrix per layer (Technical Summary, Core
 *           Architecture and Token Grouping; the thelatestinai.com Tables 2
 *           and 3 give its parameter count).
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *   - score arithmetic: fp32, products and sums in index order 0..d_g-1,
 *     no fused multiply-add (build with -ffp-contract=off);
 *   - projection arithmetic: the same rule, each sum starting at +0 and
 *     adding the rounded products in feature order 0..d_model-1;
 *   - ties in the top-k: the lower group index wins; -0.0 equals +0.0;
 *   - window: i - j < w (w keys including the query itself);
 *   - softmax scale is an argument (1/sqrt(d) in every workload);
 *   - attention sums are accumulated in double from the fp32 (or bf16
 *     widened) inputs, so the oracle's own error is far below the
 *     tolerances it is compared at.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEMORY 2

/* Score of one token against one centroid: fp32 products accumulated left to
 * right (Technical Summary, Token Grouping: the projected state is compared
 * with each centroid by a dot product). */
static float score_fixed_order(const float *r, const float *c, int dg)
{
    float s = r[0] * c[0];
    for (int e = 1; e < dg; ++e) {
        float p = r[e] * c[e];
        s = s + p;
    }
    return s;
}

/* Top-k routing (Technical Summary, Inference Efficiency (Top-k): each token
 * joins its k highest-scoring groups).  Selection sort: pass s picks the best
 * group not yet taken, scanning g upward and replacing only on a strictly
 * larger score, so equal scores resolve to the lower index. */
int oracle_route(const float *r, const float *centroids, int32_t H, int64_t n,
                 int32_t dg, int32_t K, int32_t topk, int32_t *groups,
                 uint32_t *gmask)
{
    if (!r || !centroids || !groups || H < 1 || n < 1 || dg < 1 || K < 1 ||
        K > 32 || topk < 1 || topk > K)
        return ORACLE_BAD_ARG;
#pragma omp parallel
    {
        float scores[32];
        int taken[32];
#pragma omp for schedule(static)
        for (int64_t ht = 0; ht < (int64_t)H * n; ++ht) {
            int64_t h = ht / n;
            const float *rt = r + ht * dg;
            for (int g = 0; g < K; ++g) {
                scores[g] = score_fixed_order(rt, centroids + ((int64_t)h * K + g) * dg, dg);
                taken[g] = 0;
            }
            uint32_t bits = 0;
            for (int s = 0; s < topk; ++s) {
                int best = -1;
                for (int g = 0; g < K; ++g) {
                    if (taken[g])
                        continue;
                    if (best < 0 || scores[g] > scores[best])
                        best = g;
                }
                taken[best] = 1;
                groups[ht * topk + s] = best;
                bits |= 1u << best;
            }
            if (gmask)
                gmask[ht] = bits;
        }
    }
    return ORACLE_OK;
}

/* One input element as fp32 (bf16 bit patterns widen exactly). */
static float load_as_f32(const void *base, int is_bf16, int64_t idx)
{
    if (is_bf16) {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return f;
    }
    return ((const float *)base)[idx];
}

/* Routing projection (Technical Summary, Core Architecture, Token Grouping:
 * a token's hidden state is projected into the 16-dimensional centroid
 * space before it is scored; the parameter counts of the thelatestinai.com
 * Tables 2 and 3, 148K on GPT-2 124M and 2.1M on a 7B model, match one
 * d_model x 16 matrix plus the centroids per layer):
 *     r[t][j] = sum over e = 0 .. dm-1 of W[j][e] * x[t][e]
 * fp32 products of W and x (bf16 x widened exactly), added in index order
 * starting from 0, no fused multiply-add: the same convention as the score,
 * so the projected vectors are bit-reproducible.  W is [16][dm], x [n][dm],
 * r [n][16]. */
int oracle_project(const void *x, int32_t is_bf16, int64_t n, int32_t dm,
                   const float *W, float *r)
{
    if (!x || !W || !r || n < 1 || dm < 1)
        return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        for (int j = 0; j < 16; ++j) {
            float s = 0.0f;
            for (int e = 0; e < dm; ++e) {
                float p = W[(int64_t)j * dm + e] * load_as_f32(x, is_bf16, t * dm + e);
                s = s + p;
            }
            r[t * 16 + j] = s;
        }
    }
    return ORACLE_OK;
}

/* How many of a token's lowest groups below g its code keeps: all of them
 * while top-k <= 3 (a lower set then has at most two), at top-k >= 4 the
 * lowest three when K <= 16 and the lowest two above that. */
static int kept_members(int K, int topk)
{
    if (topk <= 3)
        return topk - 1;
    return K <= 16 ? 3 : 2;
}

/* Binomial coefficient C(x, k) for small non-negative x, k (0 when k > x). */
static int binom(int x, int k)
{
    if (k < 0 || k > x)
        return 0;
    long long r = 1;
    for (int i = 1; i <= k; ++i)
        r = r * (x - k + i) / i;
    return (int)r;
}

/* Lower-set code of token t inside group g.  The token's groups below g,
 * ascending, are x_1 < x_2 < ...; the code keeps the lowest r of them
 * (r = min(their number, kept_members)) and numbers the kept set among all
 * subsets of {0, ..., g-1}: first by size, then in colexicographic order,
 * i.e. by the combinatorial number system,
 *     code = sum_{j < r} C(g, j) + sum_{i = 1..r} C(x_i, i).
 * Two tokens of group g share a group below g exactly when their full lower
 * sets meet; whenever a lower set has at most kept_members groups, the code
 * is the whole lower set. */
static int lower_code(const int32_t *gt, int topk, int g, int m)
{
    int low[32];
    int r = 0;
    for (int x = 0; x < g; ++x) { /* the groups below g, ascending */
        int in = 0;
        for (int s = 0; s < topk; ++s)
            in |= gt[s] == x;
        if (in && r < m)
            low[r++] = x;
    }
    int code = 0;
    for (int j = 0; j < r; ++j)
        code += binom(g, j);
    for (int i = 1; i <= r; ++i)
        code += binom(low[i - 1], i);
    return code;
}

/* Number of lower-set codes a token of group g can take: the subsets of
 * {0, ..., g-1} of at most m groups. */
static int codes_of_group(int g, int m)
{
    int total = 0;
    for (int j = 0; j <= m; ++j)
        total += binom(g, j);
    return total;
}

/* Sub-buckets per routing head: every (group, lower-set code). */
int oracle_num_subbuckets(int32_t K, int32_t topk)
{
    const int m = kept_members(K, topk);
    int total = 0;
    for (int g = 0; g < K; ++g)
        total += codes_of_group(g, m);
    return total;
}

/* Bucketing: the per-group token lists that within-group causal attention
 * runs over (Technical Summary, Key Contributions 5: the pattern splits into
 * a local-window call and a within-group causal call).  Entries are listed
 * group by group; inside a group, sub-bucket by lower-set code 0, 1, ...,
 * and inside a sub-bucket by ascending position.  offsets has one entry per
 * sub-bucket plus the total; slot_entry[t][s] is the entry that holds
 * (t, groups[t][s]). */
int oracle_bucket(const int32_t *groups, int32_t H, int64_t n, int32_t K,
                  int32_t topk, int32_t *offsets, int32_t *tokens,
                  int32_t *slot_entry)
{
    if (!groups || !offsets || !tokens || !slot_entry || H < 1 || n < 1 ||
        K < 1 || K > 32 || topk < 1 || topk > K || n * topk > INT32_MAX)
        return ORACLE_BAD_ARG;
    const int nsb = oracle_num_subbuckets(K, topk);
    const int m = kept_members(K, topk);
    int32_t *code = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
    int32_t *slot = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
    char *present = (char *)malloc((size_t)codes_of_group(K - 1, m));
    if (!code || !slot || !present) {
        free(code);
        free(slot);
        free(present);
        return ORACLE_NO_MEMORY;
    }
    for (int h = 0; h < H; ++h) {
        const int32_t *gh = groups + (int64_t)h * n * topk;
        int32_t *off = offsets + (int64_t)h * (nsb + 1);
        int32_t *tok = tokens + (int64_t)h * n * topk;
        int32_t *se = slot_entry + (int64_t)h * n * topk;
        int32_t cursor = 0;
        int base = 0; /* first sub-bucket of group g */
        for (int g = 0; g < K; ++g) {
            const int ncode = codes_of_group(g, m);
            memset(present, 0, (size_t)ncode);
            /* membership slot and lower-set code of every token for g */
            for (int64_t t = 0; t < n; ++t) {
                slot[t] = -1;
                for (int s = 0; s < topk; ++s)
                    if (gh[t * topk + s] == g)
                        slot[t] = s;
                code[t] = slot[t] >= 0 ? lower_code(gh + t * topk, topk, g, m) : -1;
                if (code[t] >= 0)
                    present[code[t]] = 1;
            }
            /* each code's tokens in position order (empty codes are skipped) */
            for (int c = 0; c < ncode; ++c) {
                off[base + c] = cursor;
                if (!present[c])
                    continue;
                for (int64_t t = 0; t < n; ++t) {
                    if (code[t] != c)
                        continue;
                    tok[cursor] = (int32_t)t;
                    se[t * topk + slot[t]] = cursor;
                    ++cursor;
                }
            }
            base += ncode;
        }
        off[nsb] = cursor;
    }
    free(code);
    free(slot);
    free(present);
    return ORACLE_OK;
}

static uint32_t group_bits(const int32_t *gt, int topk)
{
    uint32_t b = 0;
    for (int s = 0; s < topk; ++s)
        b |= 1u << gt[s];
    return b;
}

static double widen(const void *base, int is_bf16, int64_t idx)
{
    if (is_bf16) {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[idx];
}

/* Exact softmax over the attended set A(i) (Technical Summary, Gated
 * Attention: the local window w attends with exact softmax, distant tokens
 * only when they share a group; Inference Efficiency (Top-k): sharing at
 * least one of the top-k groups is enough).  Evaluates the listed (head, row)
 * pairs.  Query head h reads key/value head h / (Hq/Hkv) and the routing of
 * that key/value head.  q is [Hq, n, d], or [nrows, d] (the query of each
 * listed row) when q_per_row is set.  Outputs: o[row][d] (double), lse[row]
 * (natural log of the softmax denominator of the scaled scores),
 * count[row] = |A(i)|. */
int oracle_attn_rows(const void *q, int32_t q_per_row, const void *k, const void *v,
                     int32_t is_bf16, int32_t Hq, int32_t Hkv, int64_t n, int32_t d,
                     const int32_t *groups, int32_t K, int32_t topk, int64_t w,
                     double scale, const int32_t *row_head, const int64_t *row_pos,
                     int64_t nrows, double *o, double *lse, int64_t *count,
                     int32_t nthreads)
{
    if (!q || !k || !v || !groups || !row_head || !row_pos || Hq < 1 ||
        Hkv < 1 || Hq % Hkv || n < 1 || d < 1 || K < 1 || K > 32 ||
        topk < 1 || topk > K || w < 0 || nrows < 0)
        return ORACLE_BAD_ARG;
    for (int64_t r = 0; r < nrows; ++r)
        if (row_head[r] < 0 || row_head[r] >= Hq || row_pos[r] < 0 || row_pos[r] >= n)
            return ORACLE_BAD_ARG;
    uint32_t *bits = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(Hkv * n));
    if (!bits)
        return ORACLE_NO_MEMORY;
    for (int64_t ht = 0; ht < (int64_t)Hkv * n; ++ht)
        bits[ht] = group_bits(groups + ht * topk, topk);
    const int ratio = Hq / Hkv;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *sc = (double *)malloc(sizeof(double) * (size_t)n);
        double *qi = (double *)malloc(sizeof(double) * (size_t)d);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!sc || !qi || !acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            if (failed)
                continue;
            const int h = row_head[r];
            const int64_t i = row_pos[r];
            const int hk = h / ratio;
            const uint32_t *bk = bits + (int64_t)hk * n;
            const int64_t qb = q_per_row ? r * d : ((int64_t)h * n + i) * d;
            for (int e = 0; e < d; ++e)
                qi[e] = widen(q, is_bf16, qb + e);
            /* pass 1: scores of the attended keys and their maximum */
            double mx = -INFINITY;
            int64_t cnt = 0;
            for (int64_t j = 0; j <= i; ++j) {
                int in_window = (i - j) < w;
                int shares = (bk[i] & bk[j]) != 0;
                if (!in_window && !shares) {
                    sc[j] = NAN;
                    continue;
                }
                double s = 0.0;
                const int64_t kb = ((int64_t)hk * n + j) * d;
                for (int e = 0; e < d; ++e)
                    s += qi[e] * widen(k, is_bf16, kb + e);
                s *= scale;
                sc[j] = s;
                if (s > mx)
                    mx = s;
                ++cnt;
            }
            /* pass 2: softmax weights and the weighted sum of values */
            double l = 0.0;
            for (int e = 0; e < d; ++e)
                acc[e] = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                if (isnan(sc[j]))
                    continue;
                double p = exp(sc[j] - mx);
                l += p;
                const int64_t vb = ((int64_t)hk * n + j) * d;
                for (int e = 0; e < d; ++e)
                    acc[e] += p * widen(v, is_bf16, vb + e);
            }
            for (int e = 0; e < d; ++e)
                o[r * d + e] = acc[e] / l;
            lse[r] = mx + log(l);
            count[r] = cnt;
        }
        free(sc);
        free(qi);
        free(acc);
    }
    free(bits);
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* |A(i)| for every row of every routing head, without touching q, k, v:
 * min(i+1, w) window keys plus the keys j <= i - w whose group set meets
 * G(i).  Walks i upward keeping, per distinct group set, how many keys at or
 * before i - w carry it (the distinct sets are at most C(K, k) and never more
 * than n). */
int oracle_pair_counts(const int32_t *groups, int32_t H, int64_t n, int32_t K,
                       int32_t topk, int64_t w, int64_t *count)
{
    if (!groups || !count || H < 1 || n < 1 || K < 1 || K > 32 || topk < 1 ||
        topk > K || w < 0)
        return ORACLE_BAD_ARG;
    uint32_t *bits = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)n);
    uint32_t *cls = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)n);
    int32_t *cls_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
    int64_t *cnt = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    if (!bits || !cls || !cls_of || !cnt) {
        free(bits);
        free(cls);
        free(cls_of);
        free(cnt);
        return ORACLE_NO_MEMORY;
    }
    for (int h = 0; h < H; ++h) {
        const int32_t *gh = groups + (int64_t)h * n * topk;
        int64_t ncls = 0;
        for (int64_t t = 0; t < n; ++t) {
            bits[t] = group_bits(gh + t * topk, topk);
            int64_t c = 0;
            while (c < ncls && cls[c] != bits[t])
                ++c;
            if (c == ncls) {
                cls[ncls] = bits[t];
                cnt[ncls] = 0;
                ++ncls;
            }
            cls_of[t] = (int32_t)c;
        }
        for (int64_t i = 0; i < n; ++i) {
            int64_t far_end = i - w; /* keys 0..far_end lie outside the window */
            if (far_end >= 0)
                cnt[cls_of[far_end]] += 1;
            int64_t c_win = i + 1 < w ? i + 1 : w;
            int64_t c_far = 0;
            for (int64_t c = 0; c < ncls; ++c)
                if (cls[c] & bits[i])
                    c_far += cnt[c];
            count[(int64_t)h * n + i] = c_win + c_far;
        }
    }
    free(bits);
    free(cls);
    free(cls_of);
    free(cnt);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * Backward of the exact softmax over A(i): the gradients of the forward
 * above with respect to q, k and v, for the hard set (no gradient reaches the
 * routing).  Needed to fine-tune or train through Focus attention
 * (thelatestinai.com Table 5, all parameters fine-tuned; Technical Summary,
 * results: from-scratch training at 124M and 7B).  With
 *     s_ij = scale * q_i.k_j,   P_ij = exp(s_ij - L_i) on A(i),
 *     O_i = sum_j P_ij v_j,     D_i = dO_i . O_i,
 *     dP_ij = dO_i . v_j,       dS_ij = P_ij (dP_ij - D_i),
 * the chain rule gives
 *     dq_i = scale sum_{j in A(i)} dS_ij k_j
 *     dk_j = scale sum_{(h,i): j in A(i)} dS_ij q_i
 *     dv_j = sum_{(h,i): j in A(i)} P_ij dO_i
 * where the sums for dk and dv run over every query head h that reads the
 * key/value head of j.  All arithmetic is in double from the widened inputs;
 * O and L are the oracle's own (not a GPU result).
 * ------------------------------------------------------------------------ */

/* Softmax statistics of one row: L_i, and D_i = dO_i . O_i.  sc must hold n
 * doubles; qi is the widened query.  Returns |A(i)|. */
static int64_t row_stats(const double *qi, const void *k, const void *v, const void *dout,
                         int is_bf16, const uint32_t *bk, int64_t n, int d, int64_t w,
                         double scale, int64_t hk, int64_t dob, int64_t i, double *sc,
                         double *acc, double *L, double *D)
{
    double mx = -INFINITY;
    int64_t cnt = 0;
    for (int64_t j = 0; j <= i; ++j) {
        if (!((i - j) < w || (bk[i] & bk[j]) != 0)) {
            sc[j] = NAN;
            continue;
        }
        double s = 0.0;
        const int64_t kb = (hk * n + j) * d;
        for (int e = 0; e < d; ++e)
            s += qi[e] * widen(k, is_bf16, kb + e);
        sc[j] = s * scale;
        if (sc[j] > mx)
            mx = sc[j];
        ++cnt;
    }
    double l = 0.0;
    for (int e = 0; e < d; ++e)
        acc[e] = 0.0;
    for (int64_t j = 0; j <= i; ++j) {
        if (isnan(sc[j]))
            continue;
        double p = exp(sc[j] - mx);
        l += p;
        const int64_t vb = (hk * n + j) * d;
        for (int e = 0; e < d; ++e)
            acc[e] += p * widen(v, is_bf16, vb + e);
    }
    double dd = 0.0;
    for (int e = 0; e < d; ++e)
        dd += widen(dout, is_bf16, dob + e) * (acc[e] / l);
    *L = mx + log(l);
    *D = dd;
    return cnt;
}

/* dq of the listed (query head, position) rows: each row needs only its own
 * attended set.  dq is [nrows][d] (double). */
int oracle_attn_bwd_rows(const void *q, const void *k, const void *v, const void *dout,
                         int32_t is_bf16, int32_t Hq, int32_t Hkv, int64_t n, int32_t d,
                         const int32_t *groups, int32_t K, int32_t topk, int64_t w,
                         double scale, const int32_t *row_head, const int64_t *row_pos,
                         int64_t nrows, double *dq, int32_t nthreads)
{
    if (!q || !k || !v || !dout || !groups || !row_head || !row_pos || !dq || Hq < 1 ||
        Hkv < 1 || Hq % Hkv || n < 1 || d < 1 || K < 1 || K > 32 || topk < 1 ||
        topk > K || w < 0 || nrows < 0)
        return ORACLE_BAD_ARG;
    for (int64_t r = 0; r < nrows; ++r)
        if (row_head[r] < 0 || row_head[r] >= Hq || row_pos[r] < 0 || row_pos[r] >= n)
            return ORACLE_BAD_ARG;
    uint32_t *bits = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(Hkv * n));
    if (!bits)
        return ORACLE_NO_MEMORY;
    for (int64_t ht = 0; ht < (int64_t)Hkv * n; ++ht)
        bits[ht] = group_bits(groups + ht * topk, topk);
    const int ratio = Hq / Hkv;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *sc = (double *)malloc(sizeof(double) * (size_t)n);
        double *qi = (double *)malloc(sizeof(double) * (size_t)d);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!sc || !qi || !acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            if (failed)
                continue;
            const int h = row_head[r];
            const int64_t i = row_pos[r];
            const int64_t hk = h / ratio;
            const uint32_t *bk = bits + hk * n;
            const int64_t rowb = ((int64_t)h * n + i) * d;
            for (int e = 0; e < d; ++e)
                qi[e] = widen(q, is_bf16, rowb + e);
            double L, D;
            row_stats(qi, k, v, dout, is_bf16, bk, n, d, w, scale, hk, rowb, i, sc, acc, &L,
                      &D);
            for (int e = 0; e < d; ++e)
                acc[e] = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                if (isnan(sc[j]))
                    continue;
                const double p = exp(sc[j] - L);
                double dp = 0.0;
                const int64_t vb = (hk * n + j) * d;
                for (int e = 0; e < d; ++e)
                    dp += widen(dout, is_bf16, rowb + e) * widen(v, is_bf16, vb + e);
                const double ds = p * (dp - D);
                const int64_t kb = (hk * n + j) * d;
                for (int e = 0; e < d; ++e)
                    acc[e] += ds * widen(k, is_bf16, kb + e);
            }
            for (int e = 0; e < d; ++e)
                dq[r * d + e] = scale * acc[e];
        }
        free(sc);
        free(qi);
        free(acc);
    }
    free(bits);
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* Full gradients.  dq [Hq, n, d], dk and dv [Hkv, n, d], all double.  The
 * first sweep takes every query row (its L_i, D_i and dq_i); the second takes
 * every key row j of every key/value head and sums over the queries that
 * attend to it, so no two threads write the same output. */
int oracle_attn_bwd(const void *q, const void *k, const void *v, const void *dout,
                    int32_t is_bf16, int32_t Hq, int32_t Hkv, int64_t n, int32_t d,
                    const int32_t *groups, int32_t K, int32_t topk, int64_t w,
                    double scale, double *dq, double *dk, double *dv, int32_t nthreads)
{
    if (!q || !k || !v || !dout || !groups || !dq || !dk || !dv || Hq < 1 || Hkv < 1 ||
        Hq % Hkv || n < 1 || d < 1 || K < 1 || K > 32 || topk < 1 || topk > K || w < 0)
        return ORACLE_BAD_ARG;
    const int64_t rows = (int64_t)Hq * n;
    int32_t *rh = (int32_t *)malloc(sizeof(int32_t) * (size_t)rows);
    int64_t *rp = (int64_t *)malloc(sizeof(int64_t) * (size_t)rows);
    double *Ls = (double *)malloc(sizeof(double) * (size_t)rows);
    double *Ds = (double *)malloc(sizeof(double) * (size_t)rows);
    uint32_t *bits = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(Hkv * n));
    if (!rh || !rp || !Ls || !Ds || !bits) {
        free(rh);
        free(rp);
        free(Ls);
        free(Ds);
        free(bits);
        return ORACLE_NO_MEMORY;
    }
    for (int64_t r = 0; r < rows; ++r) {
        rh[r] = (int32_t)(r / n);
        rp[r] = r % n;
    }
    int rc = oracle_attn_bwd_rows(q, k, v, dout, is_bf16, Hq, Hkv, n, d, groups, K, topk, w,
                                  scale, rh, rp, rows, dq, nthreads);
    if (rc != ORACLE_OK)
        goto done;
    for (int64_t ht = 0; ht < (int64_t)Hkv * n; ++ht)
        bits[ht] = group_bits(groups + ht * topk, topk);
    const int ratio = Hq / Hkv;
    int failed = 0;
#pragma omp parallel
    {
        double *sc = (double *)malloc(sizeof(double) * (size_t)n);
        double *qi = (double *)malloc(sizeof(double) * (size_t)d);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!sc || !qi || !acc) {
#pragma omp atomic write
            failed = 1;
        }
        /* softmax statistics of every row */
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < rows; ++r) {
            if (failed)
                continue;
            const int h = (int)(r / n);
            const int64_t i = r % n;
            const int64_t hk = h / ratio;
            const int64_t rowb = r * d;
            for (int e = 0; e < d; ++e)
                qi[e] = widen(q, is_bf16, rowb + e);
            row_stats(qi, k, v, dout, is_bf16, bits + hk * n, n, d, w, scale, hk, rowb, i,
                      sc, acc, &Ls[r], &Ds[r]);
        }
        /* key rows: sum over the queries that attend to each key */
#pragma omp for schedule(dynamic, 16)
        for (int64_t kr = 0; kr < (int64_t)Hkv * n; ++kr) {
            if (failed)
                continue;
            const int64_t hk = kr / n;
            const int64_t j = kr % n;
            const uint32_t *bk = bits + hk * n;
            double *dkj = dk + kr * d;
            double *dvj = dv + kr * d;
            for (int e = 0; e < d; ++e)
                dkj[e] = dvj[e] = 0.0;
            for (int h = (int)hk * ratio; h < (int)(hk + 1) * ratio; ++h) {
                for (int64_t i = j; i < n; ++i) {
                    if (!((i - j) < w || (bk[i] & bk[j]) != 0))
                        continue;
                    const int64_t rowb = ((int64_t)h * n + i) * d;
                    double s = 0.0, dp = 0.0;
                    for (int e = 0; e < d; ++e) {
                        s += widen(q, is_bf16, rowb + e) * widen(k, is_bf16, kr * d + e);
                        dp += widen(dout, is_bf16, rowb + e) * widen(v, is_bf16, kr * d + e);
                    }
                    const double p = exp(s * scale - Ls[(int64_t)h * n + i]);
                    const double ds = p * (dp - Ds[(int64_t)h * n + i]);
                    for (int e = 0; e < d; ++e) {
                        dkj[e] += scale * ds * widen(q, is_bf16, rowb + e);
                        dvj[e] += p * widen(dout, is_bf16, rowb + e);
                    }
                }
            }
        }
        free(sc);
        free(qi);
        free(acc);
    }
    if (failed)
        rc = ORACLE_NO_MEMORY;
done:
    free(rh);
    free(rp);
    free(Ls);
    free(Ds);
    free(bits);
    return rc;
}

/* ------------------------------------------------------------------------
 * Training-mode forward (Technical Summary, Core Architecture: soft
 * assignment of each projected token to the groups; Gated Attention: the
 * distant pairs pass a learned gate s_ij = q_i.k_j * sigmoid(lambda a_ij)
 * with a_ij the group affinity; Key Technical Innovation: Sinkhorn
 * normalisation replaces softmax so that group sizes stay balanced, a
 * doubly-stochastic assignment; Significance: training still computes all
 * O(n^2) pairs because of the soft gate).  Readings where the pages are
 * silent:
 *   - the assignment starts from exp(score - max over the token's groups),
 *     score as in the routing above;
 *   - one Sinkhorn iteration scales every group column to total n/K, then
 *     every token row to total 1; `iters` iterations, so rows end summing
 *     to 1 exactly and columns approach n/K;
 *   - a_ij = sum_g A_ig A_jg, the chance that independent draws from the
 *     two tokens' assignments pick the same group;
 *   - lambda is a real scalar; the gate multiplies the score of the far
 *     pairs (i - j >= w) only; window pairs keep the plain score; every
 *     j <= i is attended (dense causal).
 * ------------------------------------------------------------------------ */

/* Sinkhorn assignment of every routing head: A [H, n, K] (double). */
int oracle_sinkhorn(const float *r, const float *centroids, int32_t H, int64_t n,
                    int32_t dg, int32_t K, int32_t iters, double *A)
{
    if (!r || !centroids || !A || H < 1 || n < 1 || dg < 1 || K < 1 || K > 32 || iters < 0)
        return ORACLE_BAD_ARG;
    double *col = (double *)malloc(sizeof(double) * (size_t)K);
    if (!col)
        return ORACLE_NO_MEMORY;
    for (int h = 0; h < H; ++h) {
        double *Ah = A + (int64_t)h * n * K;
        for (int64_t t = 0; t < n; ++t) {
            const float *rt = r + ((int64_t)h * n + t) * dg;
            double mx = -INFINITY;
            for (int g = 0; g < K; ++g) {
                double s = (double)score_fixed_order(rt, centroids + ((int64_t)h * K + g) * dg,
                                                     dg);
                Ah[t * K + g] = s;
                if (s > mx)
                    mx = s;
            }
            for (int g = 0; g < K; ++g)
                Ah[t * K + g] = exp(Ah[t * K + g] - mx);
        }
        for (int it = 0; it < iters; ++it) {
            /* columns to n / K */
            for (int g = 0; g < K; ++g)
                col[g] = 0.0;
            for (int64_t t = 0; t < n; ++t)
                for (int g = 0; g < K; ++g)
                    col[g] += Ah[t * K + g];
            for (int64_t t = 0; t < n; ++t)
                for (int g = 0; g < K; ++g)
                    Ah[t * K + g] *= ((double)n / K) / col[g];
            /* rows to 1 */
            for (int64_t t = 0; t < n; ++t) {
                double rs = 0.0;
                for (int g = 0; g < K; ++g)
                    rs += Ah[t * K + g];
                for (int g = 0; g < K; ++g)
                    Ah[t * K + g] /= rs;
            }
        }
    }
    free(col);
    return ORACLE_OK;
}

/* Gated dense causal attention for the listed (query head, row) pairs:
 * logit_ij = scale * q_i.k_j * (i - j < w ? 1 : sigmoid(lambda a_ij)),
 * softmax over every j <= i.  A is [Hkv, n, K] (double).  Outputs as in
 * oracle_attn_rows (o, natural-log lse). */
int oracle_gated_attn_rows(const void *q, const void *k, const void *v, int32_t is_bf16,
                           int32_t Hq, int32_t Hkv, int64_t n, int32_t d, const double *A,
                           int32_t K, int64_t w, double lambda, double scale,
                           const int32_t *row_head, const int64_t *row_pos, int64_t nrows,
                           double *o, double *lse, int32_t nthreads)
{
    if (!q || !k || !v || !A || !row_head || !row_pos || !o || !lse || Hq < 1 || Hkv < 1 ||
        Hq % Hkv || n < 1 || d < 1 || K < 1 || w < 0 || nrows < 0)
        return ORACLE_BAD_ARG;
    for (int64_t rr = 0; rr < nrows; ++rr)
        if (row_head[rr] < 0 || row_head[rr] >= Hq || row_pos[rr] < 0 || row_pos[rr] >= n)
            return ORACLE_BAD_ARG;
    const int ratio = Hq / Hkv;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *sc = (double *)malloc(sizeof(double) * (size_t)n);
        double *qi = (double *)malloc(sizeof(double) * (size_t)d);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!sc || !qi || !acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t rr = 0; rr < nrows; ++rr) {
            if (failed)
                continue;
            const int h = row_head[rr];
            const int64_t i = row_pos[rr];
            const int64_t hk = h / ratio;
            const double *Ai = A + (hk * n + i) * K;
            for (int e = 0; e < d; ++e)
                qi[e] = widen(q, is_bf16, ((int64_t)h * n + i) * d + e);
            double mx = -INFINITY;
            for (int64_t j = 0; j <= i; ++j) {
                double s = 0.0;
                const int64_t kb = (hk * n + j) * d;
                for (int e = 0; e < d; ++e)
                    s += qi[e] * widen(k, is_bf16, kb + e);
                double gate = 1.0;
                if (i - j >= w) {
                    const double *Aj = A + (hk * n + j) * K;
                    double a = 0.0;
                    for (int g = 0; g < K; ++g)
                        a += Ai[g] * Aj[g];
                    gate = 1.0 / (1.0 + exp(-lambda * a));
                }
                sc[j] = scale * s * gate;
                if (sc[j] > mx)
                    mx = sc[j];
            }
            double l = 0.0;
            for (int e = 0; e < d; ++e)
                acc[e] = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                const double p = exp(sc[j] - mx);
                l += p;
                const int64_t vb = (hk * n + j) * d;
                for (int e = 0; e < d; ++e)
                    acc[e] += p * widen(v, is_bf16, vb + e);
            }
            for (int e = 0; e < d; ++e)
                o[rr * d + e] = acc[e] / l;
            lse[rr] = mx + log(l);
        }
        free(sc);
        free(qi);
        free(acc);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}
