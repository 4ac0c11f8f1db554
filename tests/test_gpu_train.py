"""GPU parity of the training-mode forward (focus_sinkhorn and
focus_gated_attn_fwd) against the CPU oracle on the same seeded inputs.

Bars:
  * Sinkhorn assignment: max |A_gpu - A_oracle| <= 2e-5 (fp32 on the GPU,
    double in the oracle; entries lie in [0, 1]).
  * gated attention: O max-abs <= 2e-2 (bf16 output), LSE <= 5e-3.  The
    affinity's exponent -lambda log2(e) a_ij is formed from the keys'
    assignment rows rounded to bf16 and the queries' rows scaled by
    -lambda log2(e) and then rounded (2^-9 relative each), so the gate moves
    by at most |lambda| / 4 * 2^-8 and a logit of size |x| by that fraction
    of |x|; at the inputs here that bounds the LSE change well below 5e-3.
The oracle uses its own Sinkhorn assignment; the GPU chain uses its own.
"""
import numpy as np
import pytest
import torch

import oracle
from centroid_gated_sparse_amd import focus as F
from centroid_gated_sparse_amd.workloads import (Workload, qkv_inputs, routing_inputs,
                                                 sample_rows, to_bf16_bits)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(msg):
    print(msg, flush=True)


SK_CASES = [
    # H, n, K, iters
    (2, 1000, 4, 3),
    (8, 4099, 8, 5),
    (1, 300, 1, 2),
    (2, 300, 32, 4),
    (3, 1, 5, 3),
]


@pytest.mark.parametrize("case", SK_CASES, ids=lambda c: "H{}_n{}_K{}_it{}".format(*c))
def test_sinkhorn_matches_oracle(case):
    H, n, K, iters = case
    wl = Workload("sk", n, H, H, 64, K, 1, 1, "f32")
    c, r, _ = routing_inputs(wl, 4000 + n + K)
    A = F.focus_sinkhorn(torch.from_numpy(r).to(DEV), torch.from_numpy(c).to(DEV), iters)
    A2 = F.focus_sinkhorn(torch.from_numpy(r).to(DEV), torch.from_numpy(c).to(DEV), iters)
    torch.cuda.synchronize()
    assert torch.equal(A, A2)
    ref = oracle.sinkhorn(r, c, iters)
    err = np.abs(A.cpu().double().numpy() - ref).max()
    log(f"sinkhorn {case}: max |dA| = {err:.2e}")
    assert err <= 2e-5


def test_sinkhorn_full_size():
    """8 routing heads, 1M tokens, K = 8: every entry against the oracle."""
    wl = Workload("sk_1m", 1 << 20, 8, 8, 128, 8, 2, 1, "bf16")
    c, r, _ = routing_inputs(wl, 4100)
    A = F.focus_sinkhorn(torch.from_numpy(r).to(DEV), torch.from_numpy(c).to(DEV), 3)
    torch.cuda.synchronize()
    ref = oracle.sinkhorn(r, c, 3)
    err = np.abs(A.cpu().double().numpy() - ref).max()
    cols = A.double().sum(1).cpu().numpy() / (wl.n / wl.K)
    log(f"sinkhorn 1M: max |dA| = {err:.2e}, column totals / (n/K) in "
        f"[{cols.min():.4f}, {cols.max():.4f}]")
    assert err <= 2e-5


W = Workload
GATED = [
    # name, n, Hq, Hkv, d, K, topk (unused), w, dtype; lambda and Sinkhorn iterations
    (W("g_gqa_d128", 700, 4, 2, 128, 4, 1, 32, "bf16", qkv_std=0.5), 2.0, 3),
    (W("g_mha_d64_w0", 513, 2, 2, 64, 8, 1, 0, "bf16", qkv_std=0.7), -1.5, 2),
    (W("g_d128_k20", 300, 2, 1, 128, 20, 1, 16, "bf16", qkv_std=0.5), 3.0, 3),
    (W("g_d64_w_ge_n", 257, 2, 1, 64, 4, 1, 257, "bf16", qkv_std=1.0), 5.0, 1),
    (W("g_single", 1, 2, 1, 128, 3, 1, 4, "bf16", qkv_std=1.0), 1.0, 2),
    (W("g_gqa4_d128_n1100", 1100, 8, 2, 128, 8, 1, 64, "bf16", qkv_std=0.4), 0.8, 3),
    # w = 1: the window pass takes only j = i, the gated far pass the rest
    (W("g_d128_w1", 333, 2, 1, 128, 6, 1, 1, "bf16", qkv_std=0.5), 1.2, 2),
    # w = n - 1 with 32-group rows: one far pair per head, (n - 1, 0)
    (W("g_d64_k24_wn1", 300, 4, 2, 64, 24, 1, 299, "bf16", qkv_std=0.6), -0.7, 3),
]


def run_gated(wl, lam, iters, seed):
    c, r, _ = routing_inputs(wl, seed)
    q, k, v = qkv_inputs(wl, seed, DEV)
    A = F.focus_sinkhorn(torch.from_numpy(r).to(DEV), torch.from_numpy(c).to(DEV), iters)
    out, lse = F.focus_gated_attn_fwd(q, k, v, A, wl.window, lam, wl.scale)
    torch.cuda.synchronize()
    return c, r, q, k, v, out, lse


def compare(tag, out, lse, q, k, v, A_ref, wl, lam, rh, rp, scale=None):
    scale = wl.scale if scale is None else scale
    o_ref, lse_ref = oracle.gated_attn_rows(to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v),
                                            A_ref, wl.window, lam, scale, rh, rp)
    ih = torch.from_numpy(rh).long().to(DEV)
    ip = torch.from_numpy(rp).long().to(DEV)
    o = out[ih, ip].float().cpu().double().numpy()
    l = lse[ih, ip].cpu().double().numpy()
    eo, el = np.abs(o - o_ref).max(), np.abs(l - lse_ref).max()
    log(f"[{tag}] rows={len(rh)} max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert np.isfinite(o).all() and np.isfinite(l).all()
    assert eo <= 2e-2 and el <= 5e-3


@pytest.mark.parametrize("case", GATED, ids=lambda c: c[0].name)
def test_gated_attention_all_rows(case):
    wl, lam, iters = case
    seed = 4200 + GATED.index(case)
    c, r, q, k, v, out, lse = run_gated(wl, lam, iters, seed)
    A_ref = oracle.sinkhorn(r, c, iters)
    rh = np.repeat(np.arange(wl.hq, dtype=np.int32), wl.n)
    rp = np.tile(np.arange(wl.n, dtype=np.int64), wl.hq)
    compare(wl.name, out, lse, q, k, v, A_ref, wl, lam, rh, rp)


def test_gated_attention_7b_shape_sampled_rows():
    """32/8 heads of 128 at 32K tokens, K = 8: 512 sampled rows."""
    wl = W("g_gqa7b_n32k", 32768, 32, 8, 128, 8, 1, 1024, "bf16", qkv_std=128 ** -0.5)
    lam, iters = 4.0, 3
    c, r, q, k, v, out, lse = run_gated(wl, lam, iters, 4300)
    A_ref = oracle.sinkhorn(r, c, iters)
    rh, rp = sample_rows(wl, 4300, 512)
    compare(wl.name, out, lse, q, k, v, A_ref, wl, lam, rh, rp)


def test_gated_attention_running_max_path():
    """Logits past the fixed-offset bound: with scale 1 every row's bound
    |q_i| max|k| scale log2(e) exceeds 60 log2 units, so every wavefront of
    the gated pass takes the running-max softmax (the cases above all fit
    the fixed offset).  Every row; lambda small, so that the gate's bf16
    rounding (at most |lambda| / 4 * 2^-8 of a logit) stays inside the LSE
    bar at these larger logits."""
    wl = W("g_lazy_d128", 600, 4, 2, 128, 8, 1, 48, "bf16", qkv_std=0.7)
    lam, iters, scale = 0.05, 3, 1.0
    c, r, _ = routing_inputs(wl, 4400)
    q, k, v = qkv_inputs(wl, 4400, DEV)
    qn = q.float().norm(dim=-1)
    kmax = k.float().norm(dim=-1).amax(dim=-1)
    ratio = wl.hq // wl.hkv
    bound = qn * kmax.repeat_interleave(ratio)[:, None] * scale * 1.4426950408889634
    assert float(bound.min()) > 64.0
    A = F.focus_sinkhorn(torch.from_numpy(r).to(DEV), torch.from_numpy(c).to(DEV), iters)
    out, lse = F.focus_gated_attn_fwd(q, k, v, A, wl.window, lam, scale)
    torch.cuda.synchronize()
    A_ref = oracle.sinkhorn(r, c, iters)
    rh = np.repeat(np.arange(wl.hq, dtype=np.int32), wl.n)
    rp = np.tile(np.arange(wl.n, dtype=np.int64), wl.hq)
    compare(wl.name, out, lse, q, k, v, A_ref, wl, lam, rh, rp, scale=scale)
