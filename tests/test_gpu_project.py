"""GPU parity of the fused routing projection (focus_route_project) against
the CPU oracle on the same seeded inputs.

Bar: the routing vectors r, the group ids and the group masks are all
bit-exact — both sides add the rounded fp32 products in index order from +0
with no fused multiply-add, and select groups by the same rule.  The cases
reach every kernel variant: bf16 and fp32 hidden states, the 8-element
vector path and the element path (d_model not a multiple of 8), 1, 2 and 4
tokens per lane (chosen by n), an odd chunk count, ragged tails, K = 32 and
topk = K.  At the 1M-token 7B size the oracle checks sampled tokens, and
every token is checked against focus_route applied to the returned r.
"""
import numpy as np
import pytest
import torch

import oracle
from centroid_gated_sparse_amd import focus as F
from centroid_gated_sparse_amd.workloads import (PROJECTION_WORKLOADS, ProjectionWorkload,
                                                 projection_inputs, seed_for, to_bf16_bits)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(msg):
    print(msg, flush=True)


def host_view(x):
    if x.dtype == torch.bfloat16:
        return to_bf16_bits(x)
    return x.detach().cpu().contiguous().numpy()


def run_gpu(x, W, c, topk, want_r=True):
    Wt = torch.from_numpy(np.ascontiguousarray(W.T)).to(DEV)
    ct = torch.from_numpy(c).to(DEV)
    groups, gmask, r = F.focus_route_project(x, Wt, ct, topk, want_r=want_r)
    torch.cuda.synchronize()
    return groups, gmask, r


def assert_same(tag, got, want):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (tag, got.shape, want.shape)
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, f"{tag}: {bad.size} mismatches, first at flat index {bad[0]}"


CASES = [
    # name, n, d_model, heads, K, topk, dtype
    ProjectionWorkload("gpt2_dm768_n3000", 3000, 768, 12, 4, 2, "bf16"),
    ProjectionWorkload("q7b_dm4096_n1500", 1500, 4096, 8, 8, 2, "bf16"),
    ProjectionWorkload("f32_dm256_topk_eq_k", 5000, 256, 4, 16, 16, "f32"),
    ProjectionWorkload("bf16_dm8_one_chunk", 1000, 8, 2, 3, 1, "bf16"),
    ProjectionWorkload("bf16_dm24_odd_chunks", 2049, 24, 3, 6, 2, "bf16"),
    ProjectionWorkload("f32_dm100_element_path", 777, 100, 3, 5, 3, "f32"),
    ProjectionWorkload("bf16_dm52_k32", 333, 52, 2, 32, 4, "bf16"),
    ProjectionWorkload("single_token", 1, 64, 1, 1, 1, "bf16"),
    ProjectionWorkload("two_tokens_per_lane", 600001, 64, 2, 8, 2, "bf16"),
    ProjectionWorkload("four_tokens_per_lane_f32", 1048600, 24, 2, 8, 2, "f32"),
]


@pytest.mark.parametrize("pw", CASES, ids=lambda p: p.name)
def test_project_bitexact(pw):
    log(f"route_project {pw}")
    x, W, c = projection_inputs(pw, seed_for(pw.name), DEV)
    groups, gmask, r = run_gpu(x, W, c, pw.topk)
    r_ref, g_ref, m_ref = oracle.route_project(host_view(x), W, c, pw.topk)
    assert_same(f"{pw.name} r", r.cpu().numpy().view(np.uint32), r_ref.view(np.uint32))
    assert_same(f"{pw.name} groups", groups.cpu().numpy(), g_ref)
    assert_same(f"{pw.name} gmask", gmask.cpu().numpy().view(np.uint32), m_ref)
    # without r the same groups come out
    g2, m2, r2 = run_gpu(x, W, c, pw.topk, want_r=False)
    assert r2 is None
    assert torch.equal(g2, groups) and torch.equal(m2, gmask)


def test_project_gpt2_full_size():
    pw = PROJECTION_WORKLOADS["gpt2_proj_n64k"]
    log(f"route_project full {pw}")
    x, W, c = projection_inputs(pw, seed_for(pw.name), DEV)
    groups, gmask, r = run_gpu(x, W, c, pw.topk)
    r_ref, g_ref, m_ref = oracle.route_project(host_view(x), W, c, pw.topk)
    assert_same("r", r.cpu().numpy().view(np.uint32), r_ref.view(np.uint32))
    assert_same("groups", groups.cpu().numpy(), g_ref)
    assert_same("gmask", gmask.cpu().numpy().view(np.uint32), m_ref)


def test_project_7b_full_size_sampled():
    """1M tokens x 4096 features: the oracle on 4096 sampled tokens (edges,
    lane and wave boundaries, random), and every token through focus_route
    on the returned r."""
    pw = PROJECTION_WORKLOADS["gqa7b_proj_n1m_k8"]
    log(f"route_project full {pw}")
    x, W, c = projection_inputs(pw, seed_for(pw.name), DEV)
    groups, gmask, r = run_gpu(x, W, c, pw.topk)
    n = pw.n
    rng = np.random.default_rng(7)
    fixed = np.array([0, 1, 63, 64, 255, 256, 1023, 1024, n // 2, n - 257, n - 256, n - 2,
                      n - 1])
    idx = np.unique(np.concatenate([fixed, rng.choice(n, 4096 - fixed.size, replace=False)]))
    it = torch.from_numpy(idx).to(DEV)
    r_ref, g_ref, m_ref = oracle.route_project(host_view(x[it]), W, c, pw.topk)
    assert_same("r sampled", r[it].cpu().numpy().view(np.uint32), r_ref.view(np.uint32))
    assert_same("groups sampled", groups[:, it].cpu().numpy(), g_ref)
    assert_same("gmask sampled", gmask[:, it].cpu().numpy().view(np.uint32), m_ref)
    # every token: the fused routing equals focus_route on the returned r
    H = c.shape[0]
    rb = r.unsqueeze(0).expand(H, n, 16).contiguous()
    g2, m2 = F.focus_route(rb, torch.from_numpy(c).to(DEV), pw.topk)
    torch.cuda.synchronize()
    assert torch.equal(g2, groups) and torch.equal(m2, gmask)
    # a balanced-enough routing: every group is used by every head
    for h in range(H):
        assert torch.unique(groups[h]).numel() == pw.K
