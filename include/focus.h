/*
 * focus.h — C ABI of the Focus attention forward path on AMD Instinct MI355X
 * (gfx950).
 *
 * Focus ("Why Attend to Everything? Focus is the Key", arXiv 2604.03260):
 * each token is routed to the top-k of K learnable centroids by dot products
 * of a 16-dimensional routing vector (gist.science Technical Summary,
 * section 2, Learnable Centroids / Token Grouping / Inference Efficiency
 * (Top-k); jindou-blog method bullets).  Query i then attends with exact
 * softmax to the set
 *     A(i) = { j <= i : i - j < w  or  G(i) and G(j) share a group }
 * (Technical Summary, Gated Attention: Local Attention and Distant
 * Attention).  The pages compute this with two library attention calls (a
 * local-window call and a within-group causal call; Technical Summary,
 * Key Contributions 5); this library computes the same set with its own
 * kernels: route, bucket, gathered group attention, window attention and a
 * log-sum-exp merge.
 *
 * Conventions for every call:
 *  - Pointers are device pointers owned by the caller, contiguous, at least
 *    16-byte aligned.  The library keeps no pointer after a call returns and
 *    allocates no device memory; scratch space is a caller-provided
 *    workspace whose size the *_workspace_bytes queries return.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    legacy default stream).  Arguments are validated on the host before
 *    anything is enqueued; on any error nothing is launched.  A fault inside
 *    a kernel is reported by the caller's next synchronisation.
 *  - Batch folds into heads: every head is an independent sequence.
 *  - Routing is per key/value head (H_r == Hkv); query head h uses
 *    key/value head h / (Hq / Hkv) and that head's routing.
 *  - No C++ exception crosses this boundary.
 */
#ifndef FOCUS_H
#define FOCUS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FOCUS_OK = 0,
    FOCUS_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size or range */
    FOCUS_ERR_UNSUPPORTED = 2,      /* d not in {64,128}, d_g != 16, K > 32     */
    FOCUS_ERR_WORKSPACE = 3,        /* workspace null or smaller than required  */
    FOCUS_ERR_HIP = 4               /* a launch or runtime call failed          */
} focus_status;

typedef enum { FOCUS_F32 = 0, FOCUS_BF16 = 1 } focus_dtype;

typedef void *focus_stream; /* hipStream_t */

/* Parts of focus_attn_fwd, for callers that time or schedule them apart. */
typedef enum {
    FOCUS_PART_PREPARE = 1, /* gather keys/values into bucket order, plan tiles */
    FOCUS_PART_GROUP = 2,   /* gathered within-group causal attention -> partials */
    FOCUS_PART_WINDOW = 4,  /* sliding-window attention + log-sum-exp merge -> out */
    FOCUS_PART_ALL = 7
} focus_part;

/* Human-readable name of a status; never NULL. */
const char *focus_status_string(focus_status s);

/* Text of the last error raised on the calling thread ("" if none). */
const char *focus_last_error(void);

/* ABI revision of this header (incremented on any incompatible change). */
int32_t focus_abi_version(void);

/*
 * focus_route — centroid scores and top-k group membership.
 * Technical Summary, Token Grouping (projected state compared with each
 * centroid) and Inference Efficiency (Top-k) (each token joins its k
 * highest-scoring groups); jindou-blog: K centroids per layer, 16-d routing,
 * dot-product assignment.
 *
 *   r          fp32 [H, n, d_g]   routing vectors (d_g must be 16)
 *   centroids  fp32 [H, K, d_g]   centroids of each routing head
 *   groups     int32 [H, n, topk] out: group ids, by score descending and,
 *                                 on equal scores, by ascending index
 *   gmask      uint32 [H, n]      out: bit g set iff g is among the groups
 * Scores are fp32 products accumulated in index order 0..15 with no fused
 * multiply-add, so the result is bit-reproducible on any IEEE machine.
 * Errors: INVALID_ARGUMENT for n < 1, H < 1, K < 1, topk not in [1, K];
 * UNSUPPORTED for d_g != 16 or K > 32.
 */
focus_status focus_route(const float *r, const float *centroids, int32_t H, int64_t n,
                         int32_t d_g, int32_t K, int32_t topk, int32_t *groups,
                         uint32_t *gmask, focus_stream stream);

/*
 * focus_route_project — the routing projection fused with focus_route.
 * Technical Summary, Core Architecture and Token Grouping (each hidden state
 * is projected into the 16-dimensional centroid space before it is compared
 * with the centroids); thelatestinai.com Tables 2 and 3 (one d_model x 16
 * projection per layer: 12 x 768 x 16 = 148K parameters for GPT-2,
 * 32 x 4096 x 16 = 2.1M for Mistral-7B), so every routing head of a layer
 * routes the same r_t against its own centroids.
 *
 *   x          [n, d_model] in xdt (FOCUS_BF16 or FOCUS_F32): hidden states
 *   Wt         fp32 [d_model, d_g]  the projection, one row of d_g weights
 *                                   per hidden feature:
 *                                   r_t[j] = sum_e Wt[e][j] * x_t[e]
 *                                   (a torch Linear(d_model, 16) weight,
 *                                   transposed)
 *   centroids  fp32 [H, K, d_g]
 *   groups     int32 [H, n, topk]   out, as focus_route
 *   gmask      uint32 [H, n]        out, as focus_route
 *   r          fp32 [n, d_g]        out, optional (NULL: not written)
 * Each r_t[j] starts at +0 and adds the fp32 products Wt[e][j] * x_t[e] for
 * e = 0, 1, ..., d_model - 1, each product rounded before its add (no fused
 * multiply-add); bf16 inputs widen exactly.  The scores and the top-k then
 * follow focus_route exactly, so focus_route on the returned r (broadcast to
 * the H heads) gives the same groups.  Any d_model >= 1 works; multiples of
 * 8 take the vectorised loads.
 * Errors: INVALID_ARGUMENT for null or misaligned pointers, n < 1, H < 1,
 * d_model < 1, K < 1, topk not in [1, K]; UNSUPPORTED for d_g != 16 or
 * K > 32.
 */
focus_status focus_route_project(const void *x, focus_dtype xdt, int64_t n, int32_t d_model,
                                 const float *Wt, const float *centroids, int32_t H,
                                 int32_t d_g, int32_t K, int32_t topk, int32_t *groups,
                                 uint32_t *gmask, float *r, focus_stream stream);

/*
 * focus_bucket — per-head bucketing of the n*topk (token, group) entries for
 * within-group causal attention (Technical Summary, Key Contributions 5:
 * the sparse pattern splits into a local-window call and a within-group
 * causal call; the pages leave the gathering itself open).
 *
 * A stable counting sort of the entries of each head by sub-bucket: group g,
 * then the token's lower set inside g (its groups below g), keyed by its m
 * lowest members as a code c, with m = topk - 1 for topk <= 3, m = 3 for
 * topk >= 4 when K <= 16 and m = 2 for topk >= 4 when K > 16:
 *     no group below g              c = 0
 *     only a below g                c = 1 + a
 *     a < b kept                    c = 1 + g + C(b, 2) + a
 *     a < b < c3 kept (m = 3)       c = 1 + g + C(g, 2) + C(c3, 3) + C(b, 2) + a
 * (sizes first, then colexicographic order).  Group g holds
 * codes_g = C(g, 0) + ... + C(g, m) sub-buckets, and sub-bucket
 * sb = (codes of the groups below g) + c.  Inside a sub-bucket positions
 * ascend.  Two tokens of g share a group below g exactly when their lower
 * sets meet, which the codes decide whole at topk <= 3, and at topk = 4 when
 * K <= 16; focus_num_subbuckets(K, topk) gives the count per head.
 *
 *   groups      int32 [H, n, topk]      from focus_route
 *   offsets     int32 [H, S + 1]        out, S = focus_num_subbuckets(K, topk):
 *                                        first entry of each sub-bucket;
 *                                        offsets[h][S] = n * topk.  Group g's
 *                                        entries are one run of whole
 *                                        sub-buckets: every token holding g,
 *                                        each once, ascending by position
 *                                        inside each sub-bucket (not across
 *                                        the whole group)
 *   tokens      int32 [H, n*topk]       out: position of each entry
 *   slot_entry  int32 [H, n, topk]      out: entry index of (t, groups[t][s])
 *   workspace   >= focus_bucket_workspace_bytes(...) bytes of device memory
 * Errors: INVALID_ARGUMENT for bad sizes or n*topk > INT32_MAX; UNSUPPORTED
 * for K > 32; WORKSPACE if the workspace is missing or short.  Group ids
 * outside [0, K) or repeated ids in a token's list are undefined input.
 */
int32_t focus_num_subbuckets(int32_t K, int32_t topk); /* 0 for K or topk out of range */
size_t focus_bucket_workspace_bytes(int32_t H, int64_t n, int32_t K, int32_t topk);
focus_status focus_bucket(const int32_t *groups, int32_t H, int64_t n, int32_t K,
                          int32_t topk, int32_t *offsets, int32_t *tokens,
                          int32_t *slot_entry, void *workspace, size_t workspace_bytes,
                          focus_stream stream);

/*
 * focus_bucket_noalloc — focus_bucket for callers that cannot allocate device
 * memory or pass a workspace (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, outputs and errors as
 * focus_bucket, minus the workspace: the per-chunk counts go to a fixed
 * scratch array inside the library, FOCUS_BUCKET_NOALLOC_SCRATCH_BYTES
 * (16 MiB) on each device it runs on, held until the process ends.  Shapes
 * whose focus_bucket_workspace_bytes(H, n, K, topk) exceeds that return
 * FOCUS_ERR_WORKSPACE with nothing launched (for example H = 8, n = 1M, K = 8,
 * topk = 2 needs 4.5 MiB and fits; K = 32 at that n does not).  The call
 * allocates nothing.  Every call on a device shares that device's scratch,
 * and each call rewrites every count it reads (nothing has to start at
 * zero); calls that overlap on one device (other streams or threads) race
 * and must be serialised by the caller.
 */
#define FOCUS_BUCKET_NOALLOC_SCRATCH_BYTES (16u << 20)
focus_status focus_bucket_noalloc(const int32_t *groups, int32_t H, int64_t n, int32_t K,
                                  int32_t topk, int32_t *offsets, int32_t *tokens,
                                  int32_t *slot_entry, focus_stream stream);

/*
 * focus_check_buckets — checks that a bucketing is the one focus_bucket builds
 * from the routing behind gmask, reading every array only inside its extent
 * (every value is range-tested before it serves as an index):
 *   offsets     start at 0, never decrease, end at n * topk;
 *   tokens      in [0, n), strictly ascending inside each sub-bucket;
 *   groups      each entry's group is a bit of its token's gmask, its
 *               sub-bucket's lower-set code is the token's inside that group,
 *               and every gmask holds exactly topk bits below K;
 *   slot_entry  slot_entry[t][s] is an entry of token t, and the groups of a
 *               token's topk entries are exactly its gmask bits.
 *   gmask, offsets, tokens, slot_entry   as passed to focus_attn_fwd
 *   workspace   >= FOCUS_CHECK_WORKSPACE_BYTES bytes of device memory
 * The call is synchronous: it waits for `stream` and returns FOCUS_OK, or
 * INVALID_ARGUMENT naming the failed checks in focus_last_error().  With
 * FOCUS_DEBUG=1 in the environment (read at every call), focus_attn_fwd (when
 * its parts include PREPARE) and focus_attn_bwd run this check on their own
 * workspace before launching anything that reads rows through the buckets,
 * and return its status; such calls then synchronise the stream and cannot be
 * captured into a graph.
 * (Technical Summary, Key Contributions 5: the within-group call needs the
 * tokens gathered by group; this validates that gathering.)
 */
#define FOCUS_CHECK_WORKSPACE_BYTES 256
focus_status focus_check_buckets(const uint32_t *gmask, const int32_t *offsets,
                                 const int32_t *tokens, const int32_t *slot_entry, int32_t H,
                                 int64_t n, int32_t K, int32_t topk, void *workspace,
                                 size_t workspace_bytes, focus_stream stream);

/*
 * focus_attn_fwd — exact softmax over A(i) for every query head and row
 * (Technical Summary, Gated Attention: local window with exact softmax;
 * distant tokens only when they share a group; Inference Efficiency
 * (Top-k): sharing any one of the top-k groups suffices).
 *
 * Each surviving pair is evaluated exactly once: pairs with i - j < w by the
 * window kernel, the others by the group kernel of the lowest group the two
 * tokens share; the parts are joined by a log-sum-exp merge.  When
 * 2 topk > K any two tokens share a group, A(i) is every j <= i, and the
 * window kernel takes every pair (as if w = n); focus_attn_bwd does the same.
 *
 *   q           [Hq, n, d]  in dt (FOCUS_BF16 or FOCUS_F32)
 *   k, v        [Hkv, n, d] in dt
 *   gmask       uint32 [Hkv, n]  from focus_route
 *   offsets, tokens, slot_entry  from focus_bucket (same groups)
 *   window      w >= 0; w = 0 keeps only group pairs (a token always shares
 *               its own groups, so every row keeps itself); w >= n is dense
 *               causal attention
 *   scale       logit scale (1/sqrt(d) for standard attention); must be
 *               positive and finite: the kernels keep a row's running max in
 *               raw-logit units and decide a lazy rescale there, which takes
 *               the order of scaled logits to be that of raw ones
 *   out         [Hq, n, d] in dt: softmax-weighted values, bf16 rounded to
 *               nearest even
 *   lse         fp32 [Hq, n]: natural log of sum_j exp(scale * q_i . k_j)
 *   workspace   >= focus_attn_fwd_workspace_bytes(...) bytes
 *               (focus_attn_workspace_bytes is the same query under its
 *               earlier name)
 * Errors: INVALID_ARGUMENT for null pointers, n < 1, Hq % Hkv != 0,
 * topk not in [1, K], window < 0, n*topk > INT32_MAX, scale <= 0; UNSUPPORTED
 * for d not in {64, 128} or K > 32; WORKSPACE if short.  Buckets that were not
 * built from the routing that produced gmask are undefined input, unless
 * FOCUS_DEBUG=1 (see focus_check_buckets), which turns them into
 * INVALID_ARGUMENT before anything is launched.
 *
 * focus_attn_fwd_part runs a subset of the same work (a focus_part bitmask);
 * the parts must run in the order PREPARE, GROUP, WINDOW on the same
 * workspace, and focus_attn_fwd equals focus_attn_fwd_part(..., FOCUS_PART_ALL).
 */
size_t focus_attn_fwd_workspace_bytes(focus_dtype dt, int32_t Hq, int32_t Hkv, int64_t n,
                                      int32_t d, int32_t K, int32_t topk);
size_t focus_attn_workspace_bytes(focus_dtype dt, int32_t Hq, int32_t Hkv, int64_t n,
                                  int32_t d, int32_t K, int32_t topk);
focus_status focus_attn_fwd(const void *q, const void *k, const void *v, focus_dtype dt,
                            int32_t Hq, int32_t Hkv, int64_t n, int32_t d,
                            const uint32_t *gmask, const int32_t *offsets,
                            const int32_t *tokens, const int32_t *slot_entry, int32_t K,
                            int32_t topk, int64_t window, float scale, void *out,
                            float *lse, void *workspace, size_t workspace_bytes,
                            focus_stream stream);
focus_status focus_attn_fwd_part(const void *q, const void *k, const void *v,
                                 focus_dtype dt, int32_t Hq, int32_t Hkv, int64_t n,
                                 int32_t d, const uint32_t *gmask, const int32_t *offsets,
                                 const int32_t *tokens, const int32_t *slot_entry,
                                 int32_t K, int32_t topk, int64_t window, float scale,
                                 void *out, float *lse, void *workspace,
                                 size_t workspace_bytes, int32_t parts,
                                 focus_stream stream);

/*
 * focus_attn_bwd — gradients of focus_attn_fwd with respect to q, k and v
 * for the hard attended set A(i) (the routing gets no gradient).  Needed to
 * fine-tune or train through Focus attention (thelatestinai.com Table 5,
 * all parameters fine-tuned; Technical Summary, from-scratch training).
 * With P_ij = exp(scale q_i.k_j - lse_i) on A(i), D_i = dO_i . O_i,
 * dP_ij = dO_i . v_j and dS_ij = P_ij (dP_ij - D_i):
 *     dq_i = scale sum_j dS_ij k_j
 *     dk_j = scale sum dS_ij q_i,  dv_j = sum P_ij dO_i
 * the last two summed over every (query head, row) that attends to j.  Each
 * pair is evaluated once, under the forward's partition (window pairs apart,
 * far pairs in the bucket of the lowest shared group).
 *
 *   q, out, dout  bf16 [Hq, n, d]  forward inputs, its output, and dL/dO
 *   k, v          bf16 [Hkv, n, d]
 *   lse           fp32 [Hq, n]     the forward's log-sum-exp
 *   gmask, offsets, tokens, slot_entry   the routing and buckets the
 *                 forward used; K, topk, window, scale as in the forward
 *   dq            bf16 [Hq, n, d]  out
 *   dk, dv        bf16 [Hkv, n, d] out
 *   workspace     >= focus_attn_bwd_workspace_bytes(...) bytes: fp32
 *                 partials of every bucket entry, the tile plans, and bf16
 *                 copies of q, dout, k and v (with the rows' statistics)
 *                 gathered into bucket order for the group passes (about
 *                 89 GiB at 1M tokens, 32/8 heads of 128, top-2)
 * Arithmetic: bf16 MFMA products with fp32 accumulation; P and dS are
 * rounded to bf16 as MFMA operands; outputs rounded to nearest even.
 * Deterministic (no atomics): two runs give the same bits.
 * Errors: INVALID_ARGUMENT as focus_attn_fwd (FOCUS_DEBUG=1 checks the
 * buckets first, as there); UNSUPPORTED for dt other than FOCUS_BF16, d not
 * in {64, 128} or K > 32; WORKSPACE if short.
 */
size_t focus_attn_bwd_workspace_bytes(focus_dtype dt, int32_t Hq, int32_t Hkv, int64_t n,
                                      int32_t d, int32_t K, int32_t topk);
focus_status focus_attn_bwd(const void *q, const void *k, const void *v, const void *out,
                            const float *lse, const void *dout, focus_dtype dt, int32_t Hq,
                            int32_t Hkv, int64_t n, int32_t d, const uint32_t *gmask,
                            const int32_t *offsets, const int32_t *tokens,
                            const int32_t *slot_entry, int32_t K, int32_t topk,
                            int64_t window, float scale, void *dq, void *dk, void *dv,
                            void *workspace, size_t workspace_bytes, focus_stream stream);

/*
 * Training-mode forward (Technical Summary, Core Architecture: soft
 * assignment of tokens to groups and the learned gate
 * s_ij = q_i.k_j * sigmoid(lambda a_ij) on distant pairs; Key Technical
 * Innovation: Sinkhorn normalisation instead of softmax, a doubly-stochastic
 * assignment with balanced group sizes; Significance: training evaluates
 * all O(n^2) pairs because of the soft gate).
 *
 * focus_sinkhorn — soft assignment of every token of every routing head.
 * Scores as focus_route; the assignment starts from exp(score - the token's
 * max score) and each of `iters` iterations scales every group column to
 * total n/K, then every token row to total 1 (rows end summing to 1,
 * columns approach n/K).
 *   r          fp32 [H, n, d_g]    routing vectors (d_g = 16)
 *   centroids  fp32 [H, K, d_g]
 *   assign     fp32 [H, n, K]      out
 *   workspace  >= focus_sinkhorn_workspace_bytes(H, n) bytes (fp64 sums)
 * Column sums are reduced in a fixed order: two calls give the same bits.
 * Errors: INVALID_ARGUMENT for bad sizes or iters outside [1, 1000];
 * UNSUPPORTED for d_g != 16 or K > 32; WORKSPACE if short.
 */
size_t focus_sinkhorn_workspace_bytes(int32_t H, int64_t n);
focus_status focus_sinkhorn(const float *r, const float *centroids, int32_t H, int64_t n,
                            int32_t d_g, int32_t K, int32_t iters, float *assign,
                            void *workspace, size_t workspace_bytes, focus_stream stream);

/*
 * focus_gated_attn_fwd — gated dense causal attention: for every j <= i the
 * logit is scale * q_i.k_j, times sigmoid(lambda a_ij) when i - j >= w, with
 * a_ij = sum_g assign[i][g] assign[j][g] (the key/value head's assignment);
 * exact softmax over all j <= i.
 *   q          bf16 [Hq, n, d];  k, v  bf16 [Hkv, n, d]
 *   assign     fp32 [Hkv, n, K]  from focus_sinkhorn (the keys' rows
 *                                rounded to bf16, the queries' rows scaled by
 *                                -lambda log2(e) and then rounded, for the
 *                                affinity product, a bf16 MFMA)
 *   lambda     any finite value; window w >= 0; scale > 0
 *   out        bf16 [Hq, n, d];  lse  fp32 [Hq, n] (natural log)
 *   workspace  >= focus_gated_attn_workspace_bytes(Hkv, n, d, K) bytes:
 *              padded copies of K and V^T, two bf16 copies of the
 *              assignment (plain and scaled) padded to 32 groups, and a
 *              row-to-partial map (Hkv x n int32)
 * Two passes: the far keys (i - j >= w, gated) first, written to out and
 * lse as a normalised partial; then the window keys, merged with that
 * partial by log-sum-exp, row by row in place.  out and lse must not
 * overlap q, k, v or the workspace.
 * Errors: INVALID_ARGUMENT as focus_attn_fwd (and a non-finite lambda);
 * UNSUPPORTED for dt other than FOCUS_BF16, d not in {64, 128}, K > 32;
 * WORKSPACE if short.
 */
size_t focus_gated_attn_workspace_bytes(int32_t Hkv, int64_t n, int32_t d, int32_t K);
focus_status focus_gated_attn_fwd(const void *q, const void *k, const void *v, focus_dtype dt,
                                  int32_t Hq, int32_t Hkv, int64_t n, int32_t d,
                                  const float *assign, int32_t K, int64_t window, float lambda,
                                  float scale, void *out, float *lse, void *workspace,
                                  size_t workspace_bytes, focus_stream stream);

/*
 * focus_dense_causal_fwd — plain causal attention (every j <= i) with the
 * same window kernel and layouts; the dense baseline that Focus is compared
 * against (thelatestinai.com Table 6 compares against full attention).
 * Not part of the method.  Arguments as in focus_attn_fwd; unlike a plain
 * attention call it takes a workspace (>= focus_dense_workspace_bytes(...)
 * bytes), where the keys are copied zero-padded and the values transposed,
 * the layouts the window kernel reads.
 */
size_t focus_dense_workspace_bytes(focus_dtype dt, int32_t Hkv, int64_t n, int32_t d);
focus_status focus_dense_causal_fwd(const void *q, const void *k, const void *v,
                                    focus_dtype dt, int32_t Hq, int32_t Hkv, int64_t n,
                                    int32_t d, float scale, void *out, float *lse,
                                    void *workspace, size_t workspace_bytes,
                                    focus_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* FOCUS_H */
