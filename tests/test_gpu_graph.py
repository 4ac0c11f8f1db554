"""The Focus step (route -> bucket -> attention) replayed from a HIP graph.

The C ABI launches kernels only (no allocation, memset or synchronisation),
so a caller can capture a whole step once and replay it. Each replay must
give the bits of an eager step on the same buffers. Eager work and
synchronisations run between the replays, and the last replay follows an
in-place change of q.
"""
from __future__ import annotations

import math

import pytest
import torch

from centroid_gated_sparse_amd import focus as F
from centroid_gated_sparse_amd.workloads import Workload, qkv_inputs, routing_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _step(wl, q, k, v, rt, ct):
    H, n, K, topk = wl.hkv, wl.n, wl.K, wl.topk
    i32 = dict(dtype=torch.int32, device=DEV)
    b = {
        "groups": torch.empty((H, n, topk), **i32),
        "gmask": torch.empty((H, n), **i32),
        "offsets": torch.empty((H, F.focus_num_subbuckets(K, topk) + 1), **i32),
        "tokens": torch.empty((H, n * topk), **i32),
        "slot_entry": torch.empty((H, n, topk), **i32),
        "bws": torch.empty(max(F.focus_bucket_workspace_bytes(H, n, K, topk), 16),
                           dtype=torch.uint8, device=DEV),
        "aws": torch.empty(F.focus_attn_workspace_bytes(F.FOCUS_BF16, wl.hq, H, n, wl.d, K,
                                                        topk), dtype=torch.uint8, device=DEV),
        "out": torch.empty_like(q),
        "lse": torch.empty((wl.hq, n), dtype=torch.float32, device=DEV),
    }

    def step():
        F.focus_route(rt, ct, topk, b["groups"], b["gmask"])
        F.focus_bucket(b["groups"], K, b["offsets"], b["tokens"], b["slot_entry"], b["bws"])
        F.focus_attn_fwd(q, k, v, b["gmask"], b["offsets"], b["tokens"], b["slot_entry"], K,
                         wl.window, wl.scale, b["out"], b["lse"], b["aws"])

    return step, b


@pytest.mark.parametrize("topk", [2, 3])
def test_step_graph_replays_match_eager(topk):
    # top-2 takes the group pass; top-3 of K = 4 the all-pairs window path
    wl = Workload(f"graph_gqa_n3000_top{topk}", 3000, 8, 2, 128, 4, topk, 64, "bf16",
                  qkv_std=1.0 / math.sqrt(128))
    seed = 5150 + topk
    c, r, _ = routing_inputs(wl, seed)
    q, k, v = qkv_inputs(wl, seed, DEV)
    rt = torch.from_numpy(r).to(DEV)
    ct = torch.from_numpy(c).to(DEV)
    step, b = _step(wl, q, k, v, rt, ct)

    step()
    torch.cuda.synchronize()
    ref_out, ref_lse = b["out"].clone(), b["lse"].clone()
    assert torch.isfinite(ref_lse).all()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for i in range(3):
        # eager work between replays: clobber the outputs and the routing
        b["out"].zero_()
        b["lse"].fill_(float("nan"))
        b["groups"].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(b["out"], ref_out), f"replay {i}: out differs from the eager step"
        assert torch.equal(b["lse"], ref_lse), f"replay {i}: lse differs from the eager step"

    # the graph reads the same buffers: an in-place change of q shows up
    q.mul_(0.5)
    step()
    torch.cuda.synchronize()
    ref2_out, ref2_lse = b["out"].clone(), b["lse"].clone()
    assert not torch.equal(ref2_lse, ref_lse)
    b["out"].zero_()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(b["out"], ref2_out) and torch.equal(b["lse"], ref2_lse)
