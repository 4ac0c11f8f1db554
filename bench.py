"""Benchmark of the Focus attention forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = the whole path over one synthetic batch: focus_route ->
focus_bucket -> focus_attn_fwd (prepare, gathered group attention,
window attention + merge), inputs already resident in HBM.  Prints one JSON
line: tokens/s of the whole step, the group kernel's MFMA roofline (FLOPs
over the surviving far pairs it evaluates, timed with HIP events on the
launch stream), and the CPU oracle timed on a bounded sample of rows.

Default workload: a 7B-style grouped-query layer at 1M tokens (32 query /
8 key-value heads of 128, K=8 centroids, top-2, window 2048) — the context
length of the pages' headline speedup.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

import numpy as np

METRIC = "Focus attn fwd tokens/s + % bf16 MFMA peak at 128K–1M tokens, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3


ROOT = Path(__file__).resolve().parent
# sources of the attention kernels (their hash keys the recorded counters)
ATTN_SOURCES = ("attn.hip", "attn_common.hpp", "common.hpp")


def recorded_traffic(workload: str):
    """HBM bytes per group-kernel launch from the committed rocprofv3 counter
    summary of this workload (FETCH_SIZE and WRITE_SIZE, copy-calibrated),
    or None when there is none or the kernel source changed since."""
    path = ROOT / "profiles" / f"attn_{workload}.md"
    if not path.exists():
        return None
    text = path.read_text()
    m_hash = re.search(r"sha256: `([0-9a-f]{64})`", text)
    m_bytes = re.search(r"group_kernel_traffic_bytes_per_launch: ([0-9.eE+]+)", text)
    if not m_hash or not m_bytes:
        return None
    h = hashlib.sha256()
    for name in ATTN_SOURCES:
        h.update((ROOT / "centroid_gated_sparse_amd" / "csrc" / name).read_bytes())
    return float(m_bytes.group(1)) if h.hexdigest() == m_hash.group(1) else None


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def window_pairs(n: int, w: int) -> int:
    """sum_i min(i + 1, w): keys inside the window, per query head."""
    w = min(w, n)
    return w * (w + 1) // 2 + (n - w) * w


def _far_pairs_by_subsets(g: np.ndarray, w: int) -> int:
    """Pairs (i, j), j <= i - w, whose group sets meet, for one routing head
    (g: [n, topk] distinct groups per token), by inclusion-exclusion over the
    shared subsets: sum over nonempty T of (-1)^(|T|+1) times the pairs
    whose sets both contain T.  Memory is O(n * 2^topk), whatever K is."""
    from itertools import combinations

    n, topk = g.shape
    pos = np.arange(n, dtype=np.int64)
    one = np.int64(1)
    assert n < (1 << 31)
    total = 0
    for size in range(1, topk + 1):
        masks = np.concatenate([
            np.bitwise_or.reduce(one << g[:, list(c)].astype(np.int64), axis=1)
            for c in combinations(range(topk), size)])
        # (subset, position) keys, sorted: masks < 2^32 and positions < 2^31
        keys = np.sort((masks << np.int64(31)) + np.tile(pos, masks.size // n))
        # first entry of each key's subset, and the entries of that subset at
        # positions <= position - w (a query below the subset's first entry
        # counts nothing)
        idx = np.arange(keys.size, dtype=np.int64)
        new_subset = np.ones(keys.size, bool)
        new_subset[1:] = (keys[1:] >> 31) != (keys[:-1] >> 31)
        start = np.maximum.accumulate(np.where(new_subset, idx, 0))
        cnt = np.searchsorted(keys, keys - w, side="right") - start
        total += (1 if size % 2 else -1) * int(np.clip(cnt, 0, None).sum())
    return total


def surviving_pairs(groups: np.ndarray, K: int, w: int) -> np.ndarray:
    """|A(i)| summed over rows, per routing head (host-side count from the GPU
    routing: window keys plus earlier keys j <= i - w sharing a group)."""
    H, n, topk = groups.shape
    out = np.zeros(H, np.int64)
    for h in range(H):
        out[h] = _far_pairs_by_subsets(groups[h], w) + window_pairs(n, w)
    return out


def cpu_baseline(wl, seed, q, k, v, groups_np, r, c, budget_s: float):
    """The oracle as it stands on the host cores: full routing and bucketing,
    attention on seeded sampled rows until about budget_s of attention time,
    extrapolated to the whole layer by exact surviving-pair counts."""
    import torch

    import oracle
    from centroid_gated_sparse_amd.workloads import sample_rows, to_bf16_bits

    # the OpenMP threads the oracle's row loop runs on, passed explicitly
    cores = int(os.environ.get("OMP_NUM_THREADS") or 0) or len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    g_ref, _ = oracle.route(r, c, wl.topk)
    oracle.bucket(g_ref, wl.K)
    t_route_bucket = time.perf_counter() - t0
    counts = oracle.pair_counts(g_ref, wl.K, wl.window)          # [Hkv, n]
    kb = to_bf16_bits(k) if wl.dtype == "bf16" else k.cpu().numpy()
    vb = to_bf16_bits(v) if wl.dtype == "bf16" else v.cpu().numpy()
    heads, pos = sample_rows(wl, seed, 4096)
    done_rows, t_attn, pairs_done = 0, 0.0, 0
    chunk = 64
    while done_rows < len(pos) and t_attn < budget_s:
        rh = heads[done_rows:done_rows + chunk]
        rp = pos[done_rows:done_rows + chunk]
        qrows = q[torch.from_numpy(rh).long().to(q.device),
                  torch.from_numpy(rp).long().to(q.device)]
        qn = to_bf16_bits(qrows) if wl.dtype == "bf16" else qrows.cpu().numpy()
        t1 = time.perf_counter()
        _, _, cnt = oracle.attn_rows(qn, kb, vb, g_ref, wl.K, wl.window, wl.scale, rh, rp,
                                     nthreads=cores, num_q_heads=wl.hq)
        t_attn += time.perf_counter() - t1
        pairs_done += int(cnt.sum())
        done_rows += len(rh)
    ratio = wl.hq // wl.hkv
    total_pairs = float(counts.sum()) * ratio
    t_full = t_route_bucket + t_attn * total_pairs / max(pairs_done, 1)
    return {
        "value": wl.n / t_full,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{done_rows} seeded query rows (one random query head each; "
                   f"{pairs_done} attended pairs, {t_attn:.1f} s) of the same layer, "
                   f"extrapolated by exact surviving-pair count {total_pairs:.4g}; "
                   f"routing+bucketing timed in full ({t_route_bucket:.2f} s); fp64 "
                   f"accumulation, OpenMP over rows"),
    }


def make_step(F, wl, q, k, v, rt, ct):
    """Buffers of one workload and its step: route -> bucket -> attention
    (prepare, group, window + merge), each part bracketed by optional
    events."""
    import torch

    dev = q.device
    H, n, K, topk = wl.hkv, wl.n, wl.K, wl.topk
    i32 = dict(dtype=torch.int32, device=dev)
    b = {
        "groups": torch.empty((H, n, topk), **i32),
        "gmask": torch.empty((H, n), **i32),
        "offsets": torch.empty((H, F.focus_num_subbuckets(K, topk) + 1), **i32),
        "tokens": torch.empty((H, n * topk), **i32),
        "slot_entry": torch.empty((H, n, topk), **i32),
        "bws": torch.empty(max(F.focus_bucket_workspace_bytes(H, n, K, topk), 16),
                           dtype=torch.uint8, device=dev),
        "out": torch.empty_like(q),
        "lse": torch.empty((wl.hq, n), dtype=torch.float32, device=dev),
    }
    dt_code = F.FOCUS_BF16 if wl.dtype == "bf16" else F.FOCUS_F32
    b["aws"] = torch.empty(F.focus_attn_workspace_bytes(dt_code, wl.hq, H, n, wl.d, K, topk),
                           dtype=torch.uint8, device=dev)

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        F.focus_route(rt, ct, topk, b["groups"], b["gmask"])
        mark(1)
        F.focus_bucket(b["groups"], K, b["offsets"], b["tokens"], b["slot_entry"], b["bws"])
        mark(2)
        args_ = (q, k, v, b["gmask"], b["offsets"], b["tokens"], b["slot_entry"], K, wl.window,
                 wl.scale, b["out"], b["lse"], b["aws"])
        F.focus_attn_fwd_part(*args_, parts=F.PART_PREPARE)
        mark(3)
        F.focus_attn_fwd_part(*args_, parts=F.PART_GROUP)
        mark(4)
        F.focus_attn_fwd_part(*args_, parts=F.PART_WINDOW)
        mark(5)

    return step, b


def timed_ms(fn, warmup: int, steps: int) -> float:
    """Median time of fn() over `steps` runs after `warmup`, by events on
    the current stream."""
    import torch

    for _ in range(warmup):
        fn()
    ts = []
    for i in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
        if ts[-1] > 5000.0:  # long steps report as they finish
            log(f"timed step {i + 1}/{steps}: {ts[-1]:.0f} ms")
    return float(np.median(ts))


def graph_of(fn):
    """fn() captured once into a HIP graph (torch's CUDAGraph on ROCm, on a
    side stream of default priority); returns the graph, whose replay()
    launches the same kernels on the same buffers."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # the first launches happen outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


# Speed against full attention that the pages report in Table 6 (H100,
# FlashAttention on both sides; shape and window not stated): context
# only, printed next to this sweep's own ratio.
TABLE6_PAGES = {4: (0.2, 0.5, 1.5, 2.2, 3.0, 4.0, 4.1), 8: (0.2, 0.6, 1.8, 3.1, 4.7, 7.6, 8.6)}


def run_sweep(steps: int, warmup: int) -> int:
    """Focus step against our dense causal kernel over the Table 6 context
    lengths and group counts (top-1, 7B-style GQA layer, w = 1024); one
    JSON object with a row per (K, n)."""
    import torch

    from centroid_gated_sparse_amd import focus as F
    from centroid_gated_sparse_amd.workloads import (TABLE6_CONTEXTS, TABLE6_GROUPS,
                                                     qkv_inputs, routing_inputs, seed_for,
                                                     table6_workload)

    F.lib()
    rows = []
    for i, n in enumerate(TABLE6_CONTEXTS):
        base = table6_workload(n, TABLE6_GROUPS[0])
        q, k, v = qkv_inputs(base, seed_for(base.name), "cuda")
        dws = torch.empty(max(F.focus_dense_workspace_bytes(F.FOCUS_BF16, base.hkv, n, base.d),
                              16), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(q)
        lse = torch.empty((base.hq, n), dtype=torch.float32, device="cuda")
        dense_fn = lambda: F.focus_dense_causal_fwd(q, k, v, base.scale, out, lse, dws)  # noqa: E731
        dense_ms = timed_ms(dense_fn, 1, max(1, min(steps, 2) if n > 300000 else steps))
        # launch-bound short contexts: the same work replayed from a HIP graph
        dense_graph_ms = None
        if n <= 65536:
            dg = graph_of(dense_fn)
            dense_graph_ms = timed_ms(dg.replay, 1, steps)
            del dg
        del dws, out, lse
        for K in TABLE6_GROUPS:
            wl = table6_workload(n, K)
            c, r, _ = routing_inputs(wl, seed_for(wl.name))
            rt = torch.from_numpy(r).cuda()
            ct = torch.from_numpy(c).cuda()
            step, b = make_step(F, wl, q, k, v, rt, ct)
            focus_ms = timed_ms(step, warmup, steps)
            focus_graph_ms = None
            if dense_graph_ms is not None:
                fg = graph_of(step)
                focus_graph_ms = timed_ms(fg.replay, warmup, steps)
                del fg
            surv = int(surviving_pairs(b["groups"].cpu().numpy(), K, wl.window).sum()) * (
                wl.hq // wl.hkv)
            dense_pairs = wl.hq * n * (n + 1) // 2
            rows.append({
                "n": n, "K": K, "topk": wl.topk, "window": wl.window,
                "focus_ms": focus_ms, "dense_ms": dense_ms,
                "speedup_vs_dense": dense_ms / focus_ms,
                "focus_graph_ms": focus_graph_ms, "dense_graph_ms": dense_graph_ms,
                "speedup_vs_dense_graph": (dense_graph_ms / focus_graph_ms
                                           if focus_graph_ms else None),
                "focus_tokens_per_s": n / (focus_ms / 1e3),
                "pairs_kept_vs_dense": surv / dense_pairs,
                "focus_tflops_surviving": 4.0 * wl.d * surv / (focus_ms / 1e3) / 1e12,
                "dense_tflops": 4.0 * wl.d * dense_pairs / (dense_ms / 1e3) / 1e12,
                "pages_table6_speedup_h100": TABLE6_PAGES[K][i],
            })
            log(f"sweep: n={n} K={K} focus {focus_ms:.2f} ms dense {dense_ms:.2f} ms "
                f"-> {dense_ms / focus_ms:.2f}x" + (
                    f"; graphs {focus_graph_ms:.3f} / {dense_graph_ms:.3f} ms -> "
                    f"{dense_graph_ms / focus_graph_ms:.2f}x" if focus_graph_ms else ""))
            del step, b, rt, ct
        del q, k, v
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": "table6_contexts", "model": "gqa7b 32/8 heads d128 bf16",
                      "rows": rows}), flush=True)
    return 0


# thelatestinai.com Table 7 (K = 4, PG-19; hardware and context unstated):
# speed-up and pairs retained per top-k, GPT-2 124M and Mistral 7B
TABLE7_PAGES = {1: {"speedup": 4.0, "pairs_gpt2": 0.26, "pairs_mistral": 0.25},
                2: {"speedup": 2.0, "pairs_gpt2": 0.60, "pairs_mistral": 0.73},
                3: {"speedup": 1.3, "pairs_gpt2": 1.00, "pairs_mistral": None},
                4: {"speedup": 1.0, "pairs_gpt2": 1.00, "pairs_mistral": None}}


def run_topk_sweep(n: int, K: int, steps: int, warmup: int) -> int:
    """The top-k trade-off (Table 7 uses K = 4): the Focus step for
    top-k = 1..4 against our dense causal kernel on the 7B-style GQA layer
    (w = 1024), with the fraction of causal pairs each keeps; one JSON
    object, a row per top-k.  The routing vectors are one draw shared by
    every top-k."""
    import torch

    from centroid_gated_sparse_amd import focus as F
    from centroid_gated_sparse_amd.workloads import (TABLE7_TOPK, qkv_inputs, routing_inputs,
                                                     seed_for, table7_workload)

    F.lib()
    base = table7_workload(n, 1, K)
    seed = seed_for(base.name)
    q, k, v = qkv_inputs(base, seed, "cuda")
    c, r, _ = routing_inputs(base, seed)
    rt = torch.from_numpy(r).cuda()
    ct = torch.from_numpy(c).cuda()
    dws = torch.empty(max(F.focus_dense_workspace_bytes(F.FOCUS_BF16, base.hkv, n, base.d), 16),
                      dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((base.hq, n), dtype=torch.float32, device="cuda")
    dense_ms = timed_ms(lambda: F.focus_dense_causal_fwd(q, k, v, base.scale, out, lse, dws),
                        1, steps)
    del dws, out, lse
    dense_pairs = base.hq * n * (n + 1) // 2
    rows = []
    for topk in TABLE7_TOPK:
        wl = table7_workload(n, topk, K)
        step, b = make_step(F, wl, q, k, v, rt, ct)
        focus_ms = timed_ms(step, warmup, steps)
        surv = int(surviving_pairs(b["groups"].cpu().numpy(), wl.K, wl.window).sum()) * (
            wl.hq // wl.hkv)
        rows.append({
            "topk": topk, "K": wl.K, "n": n, "window": wl.window,
            "focus_ms": focus_ms, "dense_ms": dense_ms,
            "speedup_vs_dense": dense_ms / focus_ms,
            "pairs_kept_vs_dense": surv / dense_pairs,
            "focus_tflops_surviving": 4.0 * wl.d * surv / (focus_ms / 1e3) / 1e12,
            "pages_table7": TABLE7_PAGES[topk] if K == 4 else None,
        })
        log(f"topk sweep: n={n} top-{topk} focus {focus_ms:.2f} ms dense {dense_ms:.2f} ms "
            f"-> {dense_ms / focus_ms:.2f}x, pairs kept {surv / dense_pairs:.3f}")
        del step, b
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": "table7_topk", "K": K, "model": "gqa7b 32/8 heads d128 bf16",
                      "rows": rows}), flush=True)
    return 0


# fp32 vector rate of one MI355X without packed or fused forms: 256 CUs x
# 4 SIMDs x 16 lanes, one operation per lane per clock at 2.4 GHz.
PEAK_F32_VALU_TFLOPS = 256 * 4 * 16 * 2.4e9 / 1e12
PEAK_HBM_GBS = 8000.0


def run_project(steps: int, warmup: int) -> int:
    """The fused routing projection (focus_route_project) at each projection
    workload: one JSON object with a row per workload, each with its vector
    ALU roofline (a separate multiply and add per weight, 32 * d_model
    operations per token, plus 31 per centroid score)."""
    import torch

    from centroid_gated_sparse_amd import focus as F
    from centroid_gated_sparse_amd.workloads import (PROJECTION_WORKLOADS, projection_inputs,
                                                     seed_for)

    F.lib()
    rows = []
    for pw in PROJECTION_WORKLOADS.values():
        x, W, c = projection_inputs(pw, seed_for(pw.name), "cuda")
        Wt = torch.from_numpy(np.ascontiguousarray(W.T)).cuda()
        ct = torch.from_numpy(c).cuda()
        groups = torch.empty((pw.heads, pw.n, pw.topk), dtype=torch.int32, device="cuda")
        gmask = torch.empty((pw.heads, pw.n), dtype=torch.int32, device="cuda")
        ms = timed_ms(lambda: F.focus_route_project(x, Wt, ct, pw.topk, groups, gmask),
                      warmup, steps)
        ops = pw.n * (32.0 * pw.d_model + 31.0 * pw.heads * pw.K)
        hbm = pw.n * (pw.d_model * x.element_size() + pw.heads * 4 * (pw.topk + 1))
        achieved = ops / (ms / 1e3) / 1e12
        rows.append({
            "workload": pw.name, "n": pw.n, "d_model": pw.d_model, "heads": pw.heads,
            "centroids": pw.K, "topk": pw.topk, "dtype": pw.dtype, "ms": ms,
            "tokens_per_s": pw.n / (ms / 1e3),
            "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_F32_VALU_TFLOPS,
                         "unit": "TFLOP/s", "frac": achieved / PEAK_F32_VALU_TFLOPS},
            "hbm_gbs": hbm / (ms / 1e3) / 1e9,
            "hbm_frac": hbm / (ms / 1e3) / 1e9 / PEAK_HBM_GBS,
        })
        log(f"project: {pw.name} {ms:.3f} ms, {achieved:.2f} TFLOP/s "
            f"({achieved / PEAK_F32_VALU_TFLOPS:.1%} of the vector ALU rate)")
        del x, Wt, ct, groups, gmask
        torch.cuda.empty_cache()
    print(json.dumps({"bench": "route_project", "rows": rows}), flush=True)
    return 0


def run_backward(workload: str, steps: int, warmup: int) -> int:
    """focus_attn_bwd after one forward at a workload: one JSON object with the
    backward's time, tokens/s and MFMA roofline.  Algorithmic work: 10 d FLOPs
    per surviving pair (S, dP, dV, dK, dQ at 2 d each); the kernels execute
    14 d (the dq pass recomputes S and dP)."""
    import torch

    from centroid_gated_sparse_amd import focus as F
    from centroid_gated_sparse_amd.workloads import (WORKLOADS, dout_input, qkv_inputs,
                                                     routing_inputs, seed_for)

    F.lib()
    wl = WORKLOADS[workload]
    seed = seed_for(wl.name)
    c, r, _ = routing_inputs(wl, seed)
    rt = torch.from_numpy(r).cuda()
    ct = torch.from_numpy(c).cuda()
    q, k, v = qkv_inputs(wl, seed, "cuda")
    dout = dout_input(wl, seed, "cuda")
    step, b = make_step(F, wl, q, k, v, rt, ct)
    step()
    del b["aws"]
    torch.cuda.empty_cache()
    H, n, K, topk = wl.hkv, wl.n, wl.K, wl.topk
    need = F.focus_attn_bwd_workspace_bytes(F.FOCUS_BF16, wl.hq, H, n, wl.d, K, topk)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    log(f"backward: workload {wl.name}, workspace {need / 2**30:.2f} GiB")

    def bwd():
        F.focus_attn_bwd(q, k, v, b["out"], b["lse"], dout, b["gmask"], b["offsets"],
                         b["tokens"], b["slot_entry"], K, wl.window, wl.scale, dq, dk, dv, ws)

    ms = timed_ms(bwd, warmup, steps)
    surv = int(surviving_pairs(b["groups"].cpu().numpy(), K, wl.window).sum()) * (wl.hq // H)
    achieved = 10.0 * wl.d * surv / (ms / 1e3) / 1e12
    out = {
        "bench": "backward", "workload": wl.name, "n": n, "q_heads": wl.hq, "kv_heads": H,
        "head_dim": wl.d, "centroids": K, "topk": topk, "window": wl.window,
        "dtype": "bf16", "ms": ms, "tokens_per_s": n / (ms / 1e3),
        "surviving_pairs": surv,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "flops_per_pair": 10 * wl.d, "executed_flops_per_pair": 14 * wl.d},
    }
    log(f"backward: {ms:.1f} ms, {achieved:.0f} TFLOP/s algorithmic")
    print(json.dumps(out), flush=True)
    return 0


def run_train_forward(workload: str, steps: int, warmup: int, lam: float = 2.0,
                      iters: int = 3) -> int:
    """Training-mode forward at a workload: focus_sinkhorn + focus_gated_attn_fwd
    (dense causal, every j <= i).  One JSON object; MFMA roofline of the
    gated attention kernel on 4 d FLOPs per causal pair (QK^T and PV; the
    affinity product adds 2 * 16 or 2 * 32 more per pair, not counted)."""
    import torch

    from centroid_gated_sparse_amd import focus as F
    from centroid_gated_sparse_amd.workloads import (WORKLOADS, qkv_inputs, routing_inputs,
                                                     seed_for)

    F.lib()
    wl = WORKLOADS[workload]
    seed = seed_for(wl.name)
    c, r, _ = routing_inputs(wl, seed)
    rt = torch.from_numpy(r).cuda()
    ct = torch.from_numpy(c).cuda()
    q, k, v = qkv_inputs(wl, seed, "cuda")
    A = torch.empty((wl.hkv, wl.n, wl.K), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(int(F.lib().focus_sinkhorn_workspace_bytes(wl.hkv, wl.n)), 16),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((wl.hq, wl.n), dtype=torch.float32, device="cuda")
    sk_ms = timed_ms(lambda: F.focus_sinkhorn(rt, ct, iters, A, ws), warmup, steps)
    gws = torch.empty(max(int(F.lib().focus_gated_attn_workspace_bytes(wl.hkv, wl.n, wl.d,
                                                                         wl.K)), 16),
                      dtype=torch.uint8, device="cuda")
    at_ms = timed_ms(lambda: F.focus_gated_attn_fwd(q, k, v, A, wl.window, lam, wl.scale,
                                                    out, lse, gws), warmup, steps)
    pairs = wl.hq * wl.n * (wl.n + 1) // 2
    achieved = 4.0 * wl.d * pairs / (at_ms / 1e3) / 1e12
    res = {
        "bench": "train_forward", "workload": wl.name, "n": wl.n, "q_heads": wl.hq,
        "kv_heads": wl.hkv, "head_dim": wl.d, "centroids": wl.K, "window": wl.window,
        "lambda": lam, "sinkhorn_iters": iters, "dtype": "bf16",
        "sinkhorn_ms": sk_ms, "gated_attn_ms": at_ms,
        "tokens_per_s": wl.n / ((sk_ms + at_ms) / 1e3),
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "kernel": "focus_gated_attn_fwd: gated far pass + window pass "
                               "(4 d FLOPs per causal pair)"},
    }
    log(f"train forward: sinkhorn {sk_ms:.3f} ms, gated attention {at_ms:.1f} ms, "
        f"{achieved:.0f} TFLOP/s")
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="gqa7b_n1m_k8")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle attention time for the CPU baseline")
    ap.add_argument("--cpu-budget-other", type=float, default=3.0,
                    help="seconds of oracle attention time for each other workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="time only --workload (no per-workload blocks for the others)")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--topk-sweep", type=int, default=0, metavar="N",
                    help="the top-k trade-off (top-1..4) on an N-token layer")
    ap.add_argument("--topk-K", type=int, default=4, help="centroids for --topk-sweep")
    ap.add_argument("--sweep", action="store_true",
                    help="only run the Table 6 context sweep (Focus vs our dense kernel)")
    ap.add_argument("--train-forward", action="store_true",
                    help="only time the training-mode forward (Sinkhorn + gated dense "
                         "attention) at --workload")
    ap.add_argument("--backward", action="store_true",
                    help="only time focus_attn_bwd at --workload")
    ap.add_argument("--project", action="store_true",
                    help="only time the fused routing projection (focus_route_project)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes three "
                         "times (scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        src = torch.ones(args.copy_calibration // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "launches": 3}))
        return 0

    if args.sweep:
        return run_sweep(args.steps, args.warmup)
    if args.topk_sweep:
        return run_topk_sweep(args.topk_sweep, args.topk_K, args.steps, args.warmup)
    if args.project:
        return run_project(max(args.steps, 5), args.warmup)
    if args.backward:
        return run_backward(args.workload, args.steps, args.warmup)
    if args.train_forward:
        return run_train_forward(args.workload, args.steps, args.warmup)

    from centroid_gated_sparse_amd import focus as F
    from centroid_gated_sparse_amd.workloads import WORKLOADS, WORKLOAD_ORDER

    F.lib()  # fail loudly before anything else if the HIP library is missing
    wl = WORKLOADS[args.workload]
    res = measure_workload(F, wl, args.steps, args.warmup, dense=not args.no_dense,
                           dense_reps=3, cpu_budget=None if args.no_cpu_baseline
                           else args.cpu_budget, headline=True)
    result = res.pop("headline")
    # every other workload of the set, each timed the same way (the 1M-token
    # layer's buffers are gone by now), as blocks of the same JSON line
    if not args.no_other_workloads:
        blocks = {}
        for name in WORKLOAD_ORDER:
            if name == wl.name:
                continue
            blocks[name] = measure_workload(
                F, WORKLOADS[name], max(args.steps, 10), max(args.warmup, 2),
                dense=not args.no_dense, dense_reps=5,
                cpu_budget=None if args.no_cpu_baseline else args.cpu_budget_other)
        result["detail"]["workloads"] = blocks
    print(json.dumps(result), flush=True)
    return 0


def measure_workload(F, wl, steps: int, warmup: int, dense: bool, dense_reps: int,
                     cpu_budget, headline: bool = False) -> dict:
    """Times `steps` whole Focus steps of one workload (after `warmup`), with
    per-part HIP events on the launch stream, then our dense causal kernel
    (median of `dense_reps` launches) and the CPU oracle on sampled rows.
    Returns the workload's block; with headline=True also the bench's JSON
    result under "headline".  Frees every device buffer it made."""
    import torch

    from centroid_gated_sparse_amd.workloads import qkv_inputs, routing_inputs, seed_for

    seed = seed_for(wl.name)
    dev = "cuda"
    log(f"bench: workload {wl}")
    c, r, _ = routing_inputs(wl, seed)
    rt = torch.from_numpy(r).to(dev)
    ct = torch.from_numpy(c).to(dev)
    q, k, v = qkv_inputs(wl, seed, dev)
    step, bufs = make_step(F, wl, q, k, v, rt, ct)
    H, n, K, topk = wl.hkv, wl.n, wl.K, wl.topk
    dt_code = F.FOCUS_BF16 if wl.dtype == "bf16" else F.FOCUS_F32
    log(f"bench: workspace {bufs['aws'].numel() / 2**30:.2f} GiB")
    names = ["route", "bucket", "prepare", "group", "window"]

    for i in range(warmup):
        step()
        torch.cuda.synchronize()
        if headline:
            log(f"bench: warmup {i + 1}/{warmup} done")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"bench: {wl.name}: {steps} steps in {wall:.3f} s")
    part_ms = {nm: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in events]))
               for j, nm in enumerate(names)}
    groups_np = bufs["groups"].cpu().numpy()

    # algorithmic work: 4*d FLOPs (QK^T and PV) per surviving pair
    pairs_h = surviving_pairs(groups_np, K, wl.window)     # per routing head
    ratio = wl.hq // H
    surv = int(pairs_h.sum()) * ratio
    win = window_pairs(n, wl.window) * wl.hq
    far = surv - win
    flops_group = 4.0 * wl.d * far
    flops_all = 4.0 * wl.d * surv
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    group_tflops = flops_group / (part_ms["group"] / 1e3) / 1e12
    attn_ms = part_ms["group"] + part_ms["window"]
    attn_tflops = flops_all / (attn_ms / 1e3) / 1e12
    ms_per_step = wall / steps * 1e3
    # HBM bytes the method must move: routing reads r and writes groups and
    # gmask; bucketing reads the group ids twice and writes tokens and slots
    route_bytes = H * n * (16 * 4 + 4 * topk + 4)
    bucket_bytes = H * n * topk * 16
    block = {
        "n": n, "q_heads": wl.hq, "kv_heads": H, "head_dim": wl.d, "centroids": K,
        "topk": topk, "window": wl.window, "dtype": wl.dtype, "steps": steps,
        "ms_per_step": ms_per_step,
        "tokens_per_s": n / (wall / steps),
        "part_ms": part_ms,
        "window_merge_ms": part_ms["window"],
        "group_kernel": {"tflops": group_tflops, "frac": group_tflops / peak, "peak": peak,
                         "far_pairs": far},
        "group_plus_window": {"tflops": attn_tflops, "frac": attn_tflops / peak,
                              "surviving_pairs": surv},
        "step_tflops_surviving": flops_all / (ms_per_step / 1e3) / 1e12,
        "pairs_kept_vs_dense": surv / (wl.hq * n * (n + 1) / 2),
        "route_gbs": route_bytes / (part_ms["route"] / 1e3) / 1e9,
        "bucket_gbs": bucket_bytes / (part_ms["bucket"] / 1e3) / 1e9,
    }
    log(f"bench: {wl.name}: {ms_per_step:.3f} ms/step, group {group_tflops:.0f} TFLOP/s "
        f"({group_tflops / peak:.1%}), group+window {attn_tflops / peak:.1%}")

    headline_result = None
    if headline:
        headline_result = {
            "metric": METRIC,
            "value": n / (wall / steps),
            "unit": "tokens/s",
            "n_gpus": 1,
            "steps": steps,
            "warmup": warmup,
            "ms_per_step": ms_per_step,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": wl.dtype,
            "data": "synthetic",
            "config": {"workload": wl.name, "n": n, "q_heads": wl.hq, "kv_heads": H,
                       "head_dim": wl.d, "centroids": K, "topk": topk, "window": wl.window,
                       "batch": 1, "parallelism": "single-gpu"},
            "roofline": {"bound": "mfma", "achieved": group_tflops, "peak": peak,
                         "unit": "TFLOP/s", "frac": group_tflops / peak,
                         "traffic": recorded_traffic(wl.name),
                         "kernel": "attn_kernel group pass (focus_attn_fwd part GROUP): "
                                   "4 d FLOPs per surviving far pair over its event time",
                         "group_plus_window_frac": attn_tflops / peak},
            "detail": {
                "part_ms": part_ms,
                "surviving_pairs": surv,
                "far_pairs": far,
                "window_pairs": win,
                "pairs_kept_vs_dense": block["pairs_kept_vs_dense"],
                "attn_tflops_surviving": attn_tflops,
                "step_tflops_surviving": block["step_tflops_surviving"],
                "route_gbs": block["route_gbs"],
                "bucket_gbs": block["bucket_gbs"],
            },
        }

    # free the Focus buffers (the 1M-token workspace is 44 GiB) before the
    # dense baseline and the oracle
    del step, bufs
    torch.cuda.empty_cache()
    if dense:
        dws = torch.empty(max(F.focus_dense_workspace_bytes(dt_code, H, n, wl.d), 16),
                          dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)
        lse = torch.empty((wl.hq, n), dtype=torch.float32, device=dev)
        dense_ms = timed_ms(lambda: F.focus_dense_causal_fwd(q, k, v, wl.scale, out, lse, dws),
                            1, dense_reps)
        dense_flops = 4.0 * wl.d * wl.hq * n * (n + 1) / 2
        dense_block = {
            "ms": dense_ms,
            "launches": dense_reps,
            "timing": f"median of {dense_reps} launches after one warm-up",
            "tflops": dense_flops / (dense_ms / 1e3) / 1e12,
            "frac": dense_flops / (dense_ms / 1e3) / 1e12 / peak,
            "focus_step_speedup": dense_ms / ms_per_step,
        }
        block["dense_causal"] = dense_block
        if headline_result is not None:
            headline_result["detail"]["dense_causal"] = dense_block
        del dws, out, lse
        torch.cuda.empty_cache()
        log(f"bench: {wl.name}: dense causal {dense_ms:.2f} ms")
    if cpu_budget is not None:
        cpu = cpu_baseline(wl, seed, q, k, v, groups_np, r, c, cpu_budget)
        block["cpu_oracle"] = cpu
        if headline_result is not None:
            headline_result["cpu_baseline"] = cpu
    del q, k, v, rt, ct
    torch.cuda.empty_cache()
    if headline_result is not None:
        block["headline"] = headline_result
    return block


if __name__ == "__main__":
    sys.exit(main())
