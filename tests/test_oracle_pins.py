"""Pins for the CPU oracle: each check compares it with something other than
itself — library softmax on the special cases where the Focus set reduces to
plain causal attention, closed-form set sizes, exact integer arithmetic,
hand-derived rounding cases and the statistics the pages print.

Pages: "Why Attend to Everything? Focus is the Key" — gist.science Technical
Summary section 2 (window, group gate, top-k), thelatestinai.com Table 7
(pairs retained by top-k at K=4).
"""
import json
import math
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
from centroid_gated_sparse_amd.workloads import Workload, routing_inputs

GOLDEN = Path(__file__).resolve().parent / "golden"


# ----------------------------------------------------------------------------
# helpers: library references (torch float64 on the CPU)

def _rand_qkv(rng, hq, hkv, n, d, std=1.0):
    q = (rng.standard_normal((hq, n, d)) * std).astype(np.float32)
    k = (rng.standard_normal((hkv, n, d)) * std).astype(np.float32)
    v = (rng.standard_normal((hkv, n, d)) * std).astype(np.float32)
    return q, k, v


def _expand_kv(x, hq):
    """Key/value head h // (Hq/Hkv) serves query head h (contiguous GQA)."""
    t = torch.from_numpy(x).double()
    return t.repeat_interleave(hq // x.shape[0], dim=0)


def _library_attention(q, k, v, scale, mask=None, causal=False):
    """torch scaled_dot_product_attention plus logsumexp, float64."""
    qt = torch.from_numpy(q).double()
    kt = _expand_kv(k, q.shape[0])
    vt = _expand_kv(v, q.shape[0])
    if causal:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                             scale=scale)
        n = q.shape[1]
        mask = torch.ones(n, n, dtype=torch.bool).tril()
    else:
        mask = torch.from_numpy(np.ascontiguousarray(mask))
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                             scale=scale)
    s = torch.matmul(qt, kt.transpose(-1, -2)) * scale
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


def _assert_close(o, lse, o_ref, lse_ref, tol=1e-9):
    np.testing.assert_allclose(o, o_ref, atol=tol, rtol=0)
    np.testing.assert_allclose(lse, lse_ref, atol=tol, rtol=0)


# ----------------------------------------------------------------------------
# routing

def test_route_integer_scores_exact():
    """Small integers make every fp32 product and sum exact, so the ranking
    equals numpy's stable sort of the exact integer dot products (ties to the
    lower index)."""
    rng = np.random.default_rng(1)
    H, n, K, dg = 3, 400, 8, 16
    r = rng.integers(-2, 3, (H, n, dg)).astype(np.float32)
    c = rng.integers(-2, 3, (H, K, dg)).astype(np.float32)
    exact = np.einsum("hnd,hkd->hnk", r.astype(np.int64), c.astype(np.int64))
    for topk in (1, 2, 3, 8):
        groups, gmask = oracle.route(r, c, topk)
        want = np.argsort(-exact, axis=-1, kind="stable")[..., :topk]
        np.testing.assert_array_equal(groups, want)
        bits = np.zeros((H, n), np.uint32)
        for s in range(topk):
            bits |= (np.uint32(1) << want[..., s].astype(np.uint32))
        np.testing.assert_array_equal(gmask, bits)
    # many ties must exist for the tie rule to be exercised
    assert (np.sort(exact, -1)[..., -1] == np.sort(exact, -1)[..., -2]).mean() > 0.03


def test_route_golden_rounding_cases():
    fx = json.loads((GOLDEN / "route_fixed_order.json").read_text())
    for case in fx["cases"]:
        r = np.array([[[float.fromhex(x) for x in case["r"]]]], np.float32)
        c = np.array([[[float.fromhex(x) for x in row] for row in case["centroids"]]],
                     np.float32)
        groups, _ = oracle.route(r, c, case["topk"])
        assert groups[0, 0].tolist() == case["expected_groups"], case["name"]


def test_route_closed_forms():
    rng = np.random.default_rng(2)
    H, n, K = 2, 64, 6
    c = rng.standard_normal((H, K, 16)).astype(np.float32)
    # r = 0: every score is +-0, so the first k indices in order
    g, _ = oracle.route(np.zeros((H, n, 16), np.float32), c, 3)
    assert (g == np.array([0, 1, 2])).all()
    # K = 1: the only group
    g, m = oracle.route(rng.standard_normal((H, n, 16)).astype(np.float32), c[:, :1], 1)
    assert (g == 0).all() and (m == 1).all()
    # k = K: every group, each exactly once
    g, m = oracle.route(rng.standard_normal((H, n, 16)).astype(np.float32), c, K)
    assert (np.sort(g, -1) == np.arange(K)).all() and (m == (1 << K) - 1).all()
    # duplicated centroids a < b: a is listed before b whenever both are kept
    cd = c.copy()
    cd[:, 4] = cd[:, 1]
    r = rng.standard_normal((H, n, 16)).astype(np.float32)
    g, _ = oracle.route(r, cd, K)
    pos1 = np.argmax(g == 1, axis=-1)
    pos4 = np.argmax(g == 4, axis=-1)
    assert (pos1 + 1 == pos4).all()


def test_route_recovers_cluster_labels():
    """Clustered routing vectors (noise 0.3 around unit centroids): the top-1
    group is the generating cluster for the large majority of tokens; a
    negated or transposed score would fail this."""
    wl = Workload("t", 4096, 2, 2, 64, 4, 1, 64, "f32")
    c, r, z = routing_inputs(wl, 7)
    g, _ = oracle.route(r, c, 1)
    assert (g[..., 0] == z).mean() > 0.9


# ----------------------------------------------------------------------------
# bucketing: properties that together determine the output uniquely

def _kept(K, topk):
    """How many of the lowest groups below g a sub-bucket's key keeps: the
    whole lower set at top-k <= 3, three at top-k >= 4 with K <= 16, else two."""
    return topk - 1 if topk <= 3 else (3 if K <= 16 else 2)


def _low(gt, g, m):
    """The token's groups below g, ascending, at most the m lowest: what a
    sub-bucket of group g holds in common."""
    return tuple(sorted(x for x in gt if x < g)[:m])


@pytest.mark.parametrize("K,topk,n", [(4, 1, 300), (4, 2, 500), (8, 3, 257), (5, 5, 64),
                                      (1, 1, 33), (8, 4, 400), (6, 3, 300), (3, 2, 40),
                                      (16, 6, 200), (20, 4, 200)])
def test_bucket_properties(K, topk, n):
    """The bucketing, pinned by properties that fix it uniquely: every group's
    run of sub-buckets holds exactly the tokens of that group (brute force),
    two tokens share a sub-bucket exactly when their m lowest groups below g
    agree, sub-buckets follow one another by the size of that set, then
    colexicographically (highest member first), positions ascend inside each,
    every token appears topk times, slot_entry inverts tokens, and the number
    of sub-buckets of group g is the number of sets it can hold,
    C(g, 0) + ... + C(g, m)."""
    rng = np.random.default_rng(K * 100 + topk)
    H = 3
    r = rng.standard_normal((H, n, 16)).astype(np.float32)
    c = rng.standard_normal((H, K, 16)).astype(np.float32)
    groups, _ = oracle.route(r, c, topk)
    offsets, tokens, slot_entry = oracle.bucket(groups, K)
    m = _kept(K, topk)
    per_group = [sum(math.comb(g, s) for s in range(m + 1)) for g in range(K)]
    nsb = sum(per_group)
    assert oracle.num_subbuckets(K, topk) == nsb == offsets.shape[1] - 1
    first = np.concatenate([[0], np.cumsum(per_group)])
    for h in range(H):
        off = offsets[h]
        assert off[0] == 0 and off[nsb] == n * topk
        assert (np.diff(off) >= 0).all()
        seen = np.zeros(n, np.int64)
        where = {}
        for g in range(K):
            members = [t for t in range(n) if g in groups[h, t].tolist()]
            run = tokens[h, off[first[g]]:off[first[g + 1]]]
            assert sorted(run.tolist()) == members
            order = []
            for sb in range(first[g], first[g + 1]):
                toks = tokens[h, off[sb]:off[sb + 1]]
                assert (np.diff(toks) > 0).all()          # ascending positions
                if toks.size == 0:
                    continue
                keys = {_low(groups[h, t].tolist(), g, m) for t in toks}
                assert len(keys) == 1                     # one lower set per sub-bucket
                key = keys.pop()
                assert key not in [k for k, _ in order]   # and one sub-bucket per lower set
                order.append((key, sb))
                for t in toks:
                    where[(int(t), g)] = sb
            ranks = [(len(k), tuple(reversed(k))) for k, _ in order]
            assert ranks == sorted(ranks)
            for _, sb in order:
                seen[tokens[h, off[sb]:off[sb + 1]]] += 1
        assert (seen == topk).all()                   # each token k times
        for t in range(n):
            for s_ in range(topk):
                e = slot_entry[h, t, s_]
                sb = where[(t, int(groups[h, t, s_]))]
                assert tokens[h, e] == t and off[sb] <= e < off[sb + 1]


# ----------------------------------------------------------------------------
# attention: special cases that reduce to textbook causal attention

def _random_groups(rng, H, n, K, topk):
    r = rng.standard_normal((H, n, 16)).astype(np.float32)
    c = rng.standard_normal((H, K, 16)).astype(np.float32)
    return oracle.route(r, c, topk)[0]


def _run(q, k, v, groups, K, w, scale):
    return oracle.attn_full(q, k, v, groups, K, w, scale)


DENSE_CASE_SEEDS = {"K1": 1101, "window_ge_n": 1102, "topk_majority": 1103, "same_sets": 1104}


@pytest.mark.parametrize("case", list(DENSE_CASE_SEEDS))
def test_attn_reduces_to_dense_causal(case):
    rng = np.random.default_rng(DENSE_CASE_SEEDS[case])
    hq, hkv, n, d = 4, 2, 150, 32
    q, k, v = _rand_qkv(rng, hq, hkv, n, d)
    scale = 1 / math.sqrt(d)
    if case == "K1":
        K, w, groups = 1, 7, np.zeros((hkv, n, 1), np.int32)
    elif case == "window_ge_n":
        K, w, groups = 4, n, _random_groups(rng, hkv, n, 4, 1)
    elif case == "topk_majority":       # two 3-subsets of 4 groups always meet
        K, w, groups = 4, 3, _random_groups(rng, hkv, n, 4, 3)
    else:                               # every token in {0, 1}
        K, w = 4, 5
        groups = np.tile(np.array([1, 0], np.int32), (hkv, n, 1))
    o, lse, cnt = _run(q, k, v, groups, K, w, scale)
    o_ref, lse_ref = _library_attention(q, k, v, scale, causal=True)
    _assert_close(o, lse, o_ref, lse_ref)
    assert (cnt == np.arange(1, n + 1)).all()


def test_attn_w1_top1_is_causal_within_each_group():
    """w = 1 and top-1: token i sees exactly the earlier tokens of its own
    group, i.e. textbook causal attention over that group's subsequence."""
    rng = np.random.default_rng(11)
    hq, hkv, n, d, K = 4, 2, 200, 16, 4
    q, k, v = _rand_qkv(rng, hq, hkv, n, d)
    groups = _random_groups(rng, hkv, n, K, 1)
    scale = 0.37
    o, lse, _ = _run(q, k, v, groups, K, 1, scale)
    for h in range(hq):
        hk = h // (hq // hkv)
        for g in range(K):
            idx = np.nonzero(groups[hk, :, 0] == g)[0]
            if idx.size == 0:
                continue
            o_ref, lse_ref = _library_attention(q[h:h + 1, idx], k[hk:hk + 1, idx],
                                                v[hk:hk + 1, idx], scale, causal=True)
            _assert_close(o[h, idx], lse[h, idx], o_ref[0], lse_ref[0])


def test_attn_brute_force_mask_small():
    """Random top-2 routing, small n: the oracle equals library softmax under
    an explicit n x n boolean mask of the attended set."""
    rng = np.random.default_rng(12)
    hq, hkv, n, d, K, w = 2, 1, 96, 16, 4, 5
    q, k, v = _rand_qkv(rng, hq, hkv, n, d)
    groups = _random_groups(rng, hkv, n, K, 2)
    gm = np.zeros((hkv, n), np.int64)
    for s in range(2):
        gm |= 1 << groups[..., s].astype(np.int64)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    mask = (j <= i) & (((i - j) < w) | ((gm[0][:, None] & gm[0][None, :]) != 0))
    o, lse, cnt = _run(q, k, v, groups, K, w, 0.25)
    o_ref, lse_ref = _library_attention(q, k, v, 0.25, mask=np.broadcast_to(mask, (hq, n, n)))
    _assert_close(o, lse, o_ref, lse_ref)
    assert (cnt[0] == mask.sum(1)).all()
    # some far pairs are dropped, so this is not dense attention
    assert mask.sum() < n * (n + 1) // 2


# ----------------------------------------------------------------------------
# closed-form set sizes (q = 0 makes every logit 0: exp(LSE) = |A(i)| and the
# output is the mean of v over A(i))

def _rr_far_count(i, w, K, residues):
    total = 0
    for rho in residues:
        x = i - w - ((i - rho) % K)
        total += max(0, x // K + 1)
    return total


@pytest.mark.parametrize("K,w,topk", [(4, 8, 1), (3, 1, 1), (4, 6, 2), (5, 3, 2), (4, 0, 1)])
def test_counts_round_robin_closed_form(K, w, topk):
    n, d = 300, 8
    t = np.arange(n)
    if topk == 1:
        groups = (t % K).astype(np.int32)[None, :, None]
        residues = [0]
    else:                       # {t mod K, t+1 mod K} meets {j mod K, ...} iff (i-j) mod K in {0, 1, K-1}
        groups = np.stack([t % K, (t + 1) % K], -1).astype(np.int32)[None]
        residues = sorted({0, 1, K - 1})
    want = np.array([min(i + 1, w) + _rr_far_count(i, w, K, residues) if w > 0
                     else _rr_far_count(i, 0, K, residues) for i in range(n)])
    np.testing.assert_array_equal(oracle.pair_counts(groups, K, w)[0], want)
    rng = np.random.default_rng(13)
    q = np.zeros((1, n, d), np.float32)
    k = rng.standard_normal((1, n, d)).astype(np.float32)
    v = rng.standard_normal((1, n, d)).astype(np.float32)
    o, lse, cnt = _run(q, k, v, groups, K, w, 0.5)
    np.testing.assert_array_equal(cnt[0], want)
    np.testing.assert_allclose(np.exp(lse[0]), want, rtol=1e-12)
    for i in (0, 1, w, w + 1, 97, n - 1):
        if i >= n:
            continue
        js = [j for j in range(i + 1) if i - j < w or (i - j) % K in residues]
        np.testing.assert_allclose(o[0, i], v[0, js].astype(np.float64).mean(0), atol=1e-12)


def test_pair_counts_brute_force_and_dense():
    rng = np.random.default_rng(14)
    H, n, K = 2, 180, 5
    for topk, w in ((1, 4), (2, 9), (3, 1), (2, 0)):
        groups = _random_groups(rng, H, n, K, topk)
        gm = np.zeros((H, n), np.int64)
        for s in range(topk):
            gm |= 1 << groups[..., s].astype(np.int64)
        got = oracle.pair_counts(groups, K, w)
        i = np.arange(n)[:, None]
        j = np.arange(n)[None, :]
        for h in range(H):
            mask = (j <= i) & (((i - j) < w) | ((gm[h][:, None] & gm[h][None, :]) != 0))
            np.testing.assert_array_equal(got[h], mask.sum(1))
    groups = _random_groups(rng, 1, n, K, 1)
    assert oracle.pair_counts(groups, K, n)[0].sum() == n * (n + 1) // 2


def test_far_pairs_retained_top1_balanced():
    """Table 7 (thelatestinai.com): top-1 of K=4 keeps about a quarter of the
    pairs (26% / 25%); with balanced clustered routing the far-pair share is
    about 1/K."""
    wl = Workload("t", 8192, 1, 1, 64, 4, 1, 128, "f32")
    c, r, _ = routing_inputs(wl, 21)
    groups, _ = oracle.route(r, c, 1)
    cnt = oracle.pair_counts(groups, wl.K, wl.window)[0].astype(np.float64)
    i = np.arange(wl.n)
    win = np.minimum(i + 1, wl.window)
    far_all = np.maximum(0, i - wl.window + 1)
    share = (cnt - win).sum() / far_all.sum()
    assert 0.22 < share < 0.29


def test_attn_rows_matches_full_rows():
    rng = np.random.default_rng(15)
    hq, hkv, n, d, K = 4, 2, 120, 16, 4
    q, k, v = _rand_qkv(rng, hq, hkv, n, d)
    groups = _random_groups(rng, hkv, n, K, 2)
    o, lse, cnt = _run(q, k, v, groups, K, 9, 0.3)
    rh = np.array([0, 3, 1, 2, 2], np.int32)
    rp = np.array([0, 119, 57, 8, 9], np.int64)
    o2, lse2, cnt2 = oracle.attn_rows(q, k, v, groups, K, 9, 0.3, rh, rp)
    np.testing.assert_array_equal(o2, o[rh, rp])
    np.testing.assert_array_equal(lse2, lse[rh, rp])
    np.testing.assert_array_equal(cnt2, cnt[rh, rp])


def test_attn_bf16_inputs_widen_exactly():
    """bf16 inputs given as bit patterns equal the same values given as fp32."""
    rng = np.random.default_rng(16)
    hq, hkv, n, d, K = 2, 2, 64, 16, 4
    q, k, v = _rand_qkv(rng, hq, hkv, n, d)
    tb = [torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v)]
    bits = [t.view(torch.int16).numpy().view(np.uint16) for t in tb]
    f32 = [t.float().numpy() for t in tb]
    groups = _random_groups(rng, hkv, n, K, 2)
    a = _run(*bits, groups, K, 4, 0.25)
    b = _run(*f32, groups, K, 4, 0.25)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# ----------------------------------------------------------------------------
# routing projection r = W x (Technical Summary, Token Grouping; one d_model x
# 16 matrix per layer, as the parameter counts of Tables 2 and 3 imply)

def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values that bf16 represents exactly -> their bf16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not representable in bf16"
    return (b >> 16).astype(np.uint16)


def test_project_integer_exact():
    # small integers: every product and partial sum is exact in fp32, so the
    # result must equal integer matrix arithmetic (a transposed or shifted W
    # index cannot pass)
    rng = np.random.default_rng(11)
    n, dm = 37, 96
    x = rng.integers(-8, 9, (n, dm)).astype(np.float32)
    W = rng.integers(-5, 6, (16, dm)).astype(np.float32)
    want = (x.astype(np.int64) @ W.T.astype(np.int64)).astype(np.float32)
    assert np.array_equal(oracle.project(x, W), want)
    assert np.array_equal(oracle.project(_bf16_bits(x), W), want)


def test_project_order_and_no_fma():
    # Hand-derived rounding cases that fix the arithmetic reading (fp32,
    # index order from 0, separate multiply and add).
    # (a) W0 = 1 + 2^-20, W1 = -W0, x = (1 + 2^-7, 1 + 2^-7): each product
    #     rounds to 1 + 2^-7 + 2^-20 (the 2^-27 term is below half an ulp), so
    #     the sum is exactly 0; a fused multiply-add would keep -2^-27.
    W = np.zeros((16, 2), np.float32)
    W[0] = [1 + 2.0**-20, -(1 + 2.0**-20)]
    x = np.array([[1 + 2.0**-7, 1 + 2.0**-7]], np.float32)
    r = oracle.project(_bf16_bits(x), W)
    assert r[0, 0] == 0.0
    # (b) x = (1, 2^-24 x 15), W = 1: in index order every 1 + 2^-24 rounds to
    #     even, back to 1; summing the small terms first would give 1 + 2^-20.
    x = np.array([[1.0] + [2.0**-24] * 15], np.float32)
    W = np.ones((16, 16), np.float32)
    r = oracle.project(_bf16_bits(x), W)
    assert np.all(r[0] == 1.0)


def test_route_project_identity_reduces_to_route():
    # W = [I_16 | 0]: the projected vector is the first 16 hidden components,
    # so the groups are the (pinned) routing of those components
    rng = np.random.default_rng(12)
    n, dm, H, K, topk = 300, 40, 3, 8, 2
    x = rng.standard_normal((n, dm)).astype(np.float32)
    W = np.zeros((16, dm), np.float32)
    W[:, :16] = np.eye(16, dtype=np.float32)
    c = rng.standard_normal((H, K, 16)).astype(np.float32)
    r, g, m = oracle.route_project(x, W, c, topk)
    assert np.array_equal(r, x[:, :16])
    g_ref, m_ref = oracle.route(np.ascontiguousarray(np.broadcast_to(x[:, :16], (H, n, 16))),
                                c, topk)
    assert np.array_equal(g, g_ref) and np.array_equal(m, m_ref)


# ----------------------------------------------------------------------------
# backward: gradients of the exact softmax over A(i) with respect to q, k, v

def _library_grads(q, k, v, dout, scale, mask):
    """torch autograd (float64, CPU) through a plain masked softmax attention
    with Hq/Hkv head sharing: the gradients of sum(dout * O)."""
    hq = q.shape[0]
    qt = torch.from_numpy(q).double().requires_grad_(True)
    kt = torch.from_numpy(k).double().requires_grad_(True)
    vt = torch.from_numpy(v).double().requires_grad_(True)
    ke = kt.repeat_interleave(hq // k.shape[0], dim=0)
    ve = vt.repeat_interleave(hq // v.shape[0], dim=0)
    s = torch.matmul(qt, ke.transpose(-1, -2)) * scale
    s = s.masked_fill(~torch.from_numpy(np.ascontiguousarray(mask)), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), ve)
    (o * torch.from_numpy(dout).double()).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def _set_mask(groups, w):
    """Boolean [Hkv, n, n] mask of A(i), from its definition."""
    hkv, n, topk = groups.shape
    gm = np.zeros((hkv, n), np.int64)
    for s in range(topk):
        gm |= 1 << groups[..., s].astype(np.int64)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return (j <= i)[None] & (((i - j) < w)[None] | ((gm[:, :, None] & gm[:, None, :]) != 0))


def _assert_grads(got, want, tol=1e-10):
    for g, r, name in zip(got, want, ("dq", "dk", "dv")):
        np.testing.assert_allclose(g, r, atol=tol, rtol=0, err_msg=name)


def test_attn_bwd_finite_differences():
    """The gradients equal central differences of the pinned forward:
    d/dx sum(dout * O) for sampled elements of q, k and v."""
    rng = np.random.default_rng(21)
    hq, hkv, n, d, K, w, scale = 2, 1, 48, 8, 3, 4, 0.5
    q, k, v = _rand_qkv(rng, hq, hkv, n, d)
    dout = rng.standard_normal((hq, n, d)).astype(np.float32)
    groups = _random_groups(rng, hkv, n, K, 2)
    grads = oracle.attn_bwd(q, k, v, dout, groups, K, w, scale)

    def loss(qq, kk, vv):
        o, _, _ = _run(qq, kk, vv, groups, K, w, scale)
        return float((o * dout.astype(np.float64)).sum())

    h = np.float32(2.0 ** -10)
    for which, arr in enumerate((q, k, v)):
        for _ in range(12):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[idx] = arr[idx] + h
            minus[idx] = arr[idx] - h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = plus, minus
            fd = (loss(*args_p) - loss(*args_m)) / (float(plus[idx]) - float(minus[idx]))
            an = grads[which][idx]
            assert abs(fd - an) <= 2e-5 + 1e-4 * abs(an), (which, idx, fd, an)


@pytest.mark.parametrize("case", ["K1", "window_ge_n"])
def test_attn_bwd_reduces_to_dense_causal(case):
    rng = np.random.default_rng(22 + len(case))
    hq, hkv, n, d = 4, 2, 90, 16
    q, k, v = _rand_qkv(rng, hq, hkv, n, d)
    dout = rng.standard_normal((hq, n, d)).astype(np.float32)
    if case == "K1":
        K, w, groups = 1, 5, np.zeros((hkv, n, 1), np.int32)
    else:
        K, w, groups = 4, n, _random_groups(rng, hkv, n, 4, 1)
    got = oracle.attn_bwd(q, k, v, dout, groups, K, w, 0.3)
    causal = np.broadcast_to(np.tril(np.ones((n, n), bool)), (hq, n, n))
    _assert_grads(got, _library_grads(q, k, v, dout, 0.3, causal))


def test_attn_bwd_w1_top1_is_causal_within_each_group():
    """w = 1, top-1: each group's subsequence is textbook causal attention,
    so its gradients are those of that attention alone."""
    rng = np.random.default_rng(23)
    hq, hkv, n, d, K = 2, 2, 120, 8, 4
    q, k, v = _rand_qkv(rng, hq, hkv, n, d)
    dout = rng.standard_normal((hq, n, d)).astype(np.float32)
    groups = _random_groups(rng, hkv, n, K, 1)
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, groups, K, 1, 0.4)
    for h in range(hq):
        for g in range(K):
            idx = np.nonzero(groups[h, :, 0] == g)[0]
            if idx.size == 0:
                continue
            m = idx.size
            causal = np.tril(np.ones((m, m), bool))[None]
            rq, rk, rv = _library_grads(q[h:h + 1, idx], k[h:h + 1, idx], v[h:h + 1, idx],
                                        dout[h:h + 1, idx], 0.4, causal)
            _assert_grads((dq[h, idx], dk[h, idx], dv[h, idx]), (rq[0], rk[0], rv[0]))


def test_attn_bwd_brute_force_mask_small():
    """Random top-2 routing with grouped-query heads: equal to autograd
    through a softmax under the explicit mask of A(i)."""
    rng = np.random.default_rng(24)
    hq, hkv, n, d, K, w = 4, 2, 80, 16, 4, 6
    q, k, v = _rand_qkv(rng, hq, hkv, n, d)
    dout = rng.standard_normal((hq, n, d)).astype(np.float32)
    groups = _random_groups(rng, hkv, n, K, 2)
    mask = np.repeat(_set_mask(groups, w), hq // hkv, axis=0)
    got = oracle.attn_bwd(q, k, v, dout, groups, K, w, 0.25)
    _assert_grads(got, _library_grads(q, k, v, dout, 0.25, mask))
    # rows-only dq agrees with the full computation
    rh = np.array([0, 1, 3, 2], np.int32)
    rp = np.array([0, 5, 79, 40], np.int64)
    dq_rows = oracle.attn_bwd_rows(q, k, v, dout, groups, K, w, 0.25, rh, rp)
    np.testing.assert_allclose(dq_rows, got[0][rh, rp], atol=1e-12, rtol=0)


def test_attn_bwd_column_identities():
    """Each row's softmax weights sum to one and its dS sums to zero, so
    sum_j dv_j equals the sum of dout over the query heads of the key/value
    head, and sum_j dk_j = 0."""
    rng = np.random.default_rng(25)
    hq, hkv, n, d, K, w = 4, 2, 100, 8, 3, 3
    q, k, v = _rand_qkv(rng, hq, hkv, n, d)
    dout = rng.standard_normal((hq, n, d)).astype(np.float32)
    groups = _random_groups(rng, hkv, n, K, 1)
    _, dk, dv = oracle.attn_bwd(q, k, v, dout, groups, K, w, 0.5)
    r = hq // hkv
    for hk in range(hkv):
        want = dout[hk * r:(hk + 1) * r].astype(np.float64).sum(axis=(0, 1))
        np.testing.assert_allclose(dv[hk].sum(0), want, atol=1e-9, rtol=0)
        np.testing.assert_allclose(dk[hk].sum(0), 0.0, atol=1e-9)


# ----------------------------------------------------------------------------
# training-mode forward: Sinkhorn assignment and gated dense attention

def _unit_scores_inputs(u, v):
    """Routing vectors (u_t, v_t, 0, ...) against centroids e_0, e_1: the fixed-
    order score of token t is exactly u_t for group 0 and v_t for group 1."""
    n = len(u)
    r = np.zeros((1, n, 16), np.float32)
    r[0, :, 0] = u
    r[0, :, 1] = v
    c = np.zeros((1, 2, 16), np.float32)
    c[0, 0, 0] = 1.0
    c[0, 1, 1] = 1.0
    return r, c


def test_sinkhorn_rows_and_columns():
    rng = np.random.default_rng(31)
    H, n, K = 2, 300, 5
    r = rng.standard_normal((H, n, 16)).astype(np.float32)
    c = rng.standard_normal((H, K, 16)).astype(np.float32)
    A1 = oracle.sinkhorn(r, c, 1)
    np.testing.assert_allclose(A1.sum(-1), 1.0, atol=1e-12)
    A = oracle.sinkhorn(r, c, 300)
    np.testing.assert_allclose(A.sum(-1), 1.0, atol=1e-12)
    np.testing.assert_allclose(A.sum(1), n / K, rtol=1e-8)
    assert (A > 0).all()


def test_sinkhorn_uniform_and_single_group():
    H, n = 1, 40
    r = np.zeros((H, n, 16), np.float32)
    c = np.random.default_rng(32).standard_normal((H, 4, 16)).astype(np.float32)
    np.testing.assert_allclose(oracle.sinkhorn(r, c, 3), 0.25, atol=1e-15)
    r1 = np.random.default_rng(33).standard_normal((H, n, 16)).astype(np.float32)
    np.testing.assert_allclose(oracle.sinkhorn(r1, c[:, :1], 3), 1.0, atol=1e-15)


def test_sinkhorn_two_by_two_closed_form():
    """n = 2, K = 2: the doubly-stochastic scaling of a positive 2x2 matrix M
    is [[x, 1-x], [1-x, x]] with x = sqrt(m00 m11) / (sqrt(m00 m11) +
    sqrt(m01 m10))."""
    u = np.array([0.5, -1.25], np.float32)
    v = np.array([-0.75, 1.0], np.float32)
    r, c = _unit_scores_inputs(u, v)
    A = oracle.sinkhorn(r, c, 200)[0]
    s = np.stack([u, v], 1).astype(np.float64)
    M = np.exp(s - s.max(1, keepdims=True))
    a, b = math.sqrt(M[0, 0] * M[1, 1]), math.sqrt(M[0, 1] * M[1, 0])
    x = a / (a + b)
    np.testing.assert_allclose(A, [[x, 1 - x], [1 - x, x]], atol=1e-12)


def test_sinkhorn_one_iteration_worked_example():
    """One iteration on n = 2 tokens, K = 2 groups, worked by hand: scale each
    column of M to total n/K = 1, then each row to total 1."""
    u = np.array([0.5, -1.25], np.float32)
    v = np.array([-0.75, 1.0], np.float32)
    r, c = _unit_scores_inputs(u, v)
    A = oracle.sinkhorn(r, c, 1)[0]
    m00, m01 = 1.0, math.exp(-0.75 - 0.5)      # token 0: max score 0.5 (group 0)
    m10, m11 = math.exp(-1.25 - 1.0), 1.0      # token 1: max score 1.0 (group 1)
    c0, c1 = m00 + m10, m01 + m11
    b = [[m00 / c0, m01 / c1], [m10 / c0, m11 / c1]]
    want = [[x / sum(row) for x in row] for row in b]
    np.testing.assert_allclose(A, want, atol=1e-14)


def test_sinkhorn_limit_is_a_diagonal_scaling():
    """The Sinkhorn-Knopp limit is diag(a) M diag(b): log(A / M) is a sum of a
    row term and a column term, so its double-centred residual vanishes."""
    rng = np.random.default_rng(34)
    n, K = 64, 4
    u = rng.standard_normal((1, n, 16)).astype(np.float32)
    cen = rng.standard_normal((1, K, 16)).astype(np.float32)
    A = oracle.sinkhorn(u, cen, 500)[0]
    s = np.array([[np.float32(0)] * K] * n, np.float64)
    for t in range(n):
        for g in range(K):
            acc = np.float32(u[0, t, 0]) * np.float32(cen[0, g, 0])
            for e in range(1, 16):
                acc = np.float32(acc + np.float32(u[0, t, e]) * np.float32(cen[0, g, e]))
            s[t, g] = acc
    L = np.log(A) - s
    resid = L - L.mean(1, keepdims=True) - L.mean(0, keepdims=True) + L.mean()
    assert np.abs(resid).max() < 1e-9
    np.testing.assert_allclose(A.sum(0), n / K, rtol=1e-9)


def _gated_library(q, k, v, mult, scale):
    """Library softmax (torch, float64) of scale * q.k * mult over j <= i."""
    hq, n, _ = q.shape
    kt = _expand_kv(k, hq)
    vt = _expand_kv(v, hq)
    s = torch.matmul(torch.from_numpy(q).double(), kt.transpose(-1, -2)) * scale
    s = s * torch.from_numpy(mult).double()
    causal = torch.ones(n, n, dtype=torch.bool).tril()
    s = s.masked_fill(~causal, float("-inf"))
    return (torch.matmul(torch.softmax(s, -1), vt).numpy(), torch.logsumexp(s, -1).numpy())


def _all_rows(hq, n):
    return (np.repeat(np.arange(hq, dtype=np.int32), n),
            np.tile(np.arange(n, dtype=np.int64), hq))


@pytest.mark.parametrize("case", ["lambda_large", "window_ge_n"])
def test_gated_attention_reduces_to_dense_causal(case):
    rng = np.random.default_rng(35 + len(case))
    hq, hkv, n, d, K = 4, 2, 70, 16, 3
    q, k, v = _rand_qkv(rng, hq, hkv, n, d)
    # mild scores keep every a_ij well above 0, so lambda a_ij is large
    A = oracle.sinkhorn((0.1 * rng.standard_normal((hkv, n, 16))).astype(np.float32),
                        rng.standard_normal((hkv, K, 16)).astype(np.float32), 3)
    assert np.einsum("hik,hjk->hij", A, A).min() > 0.05
    lam, w = (1e6, 4) if case == "lambda_large" else (-3.0, n)
    rh, rp = _all_rows(hq, n)
    o, lse = oracle.gated_attn_rows(q, k, v, A, w, lam, 0.3, rh, rp)
    o_ref, lse_ref = _library_attention(q, k, v, 0.3, causal=True)
    np.testing.assert_allclose(o.reshape(hq, n, d), o_ref, atol=1e-9)
    np.testing.assert_allclose(lse.reshape(hq, n), lse_ref, atol=1e-9)


def test_gated_attention_one_hot_assignment():
    """One-hot assignments make a_ij 1 for tokens of one group and 0 otherwise,
    so far pairs carry the factor sigmoid(lambda) or 1/2, window pairs 1."""
    rng = np.random.default_rng(37)
    hq, hkv, n, d, K, w, lam = 2, 1, 60, 8, 3, 5, 1.7
    q, k, v = _rand_qkv(rng, hq, hkv, n, d)
    z = rng.integers(0, K, n)
    A = np.zeros((hkv, n, K))
    A[0, np.arange(n), z] = 1.0
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    far_gate = np.where(z[:, None] == z[None, :], 1 / (1 + math.exp(-lam)), 0.5)
    mult = np.broadcast_to(np.where(i - j < w, 1.0, far_gate), (hq, n, n)).copy()
    rh, rp = _all_rows(hq, n)
    o, lse = oracle.gated_attn_rows(q, k, v, A, w, lam, 0.45, rh, rp)
    o_ref, lse_ref = _gated_library(q, k, v, mult, 0.45)
    np.testing.assert_allclose(o.reshape(hq, n, d), o_ref, atol=1e-9)
    np.testing.assert_allclose(lse.reshape(hq, n), lse_ref, atol=1e-9)
