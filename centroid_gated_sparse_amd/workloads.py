"""Seeded synthetic workloads for the Focus attention forward path.

This module only draws inputs; it holds none of the method's arithmetic, and
it is the one piece shared by the GPU path's tests, the benchmark and the CPU
oracle's checks.

Shapes follow the workloads the Focus pages measure: GPT-2 124M layers
(12 heads of 64, the Table 2 / Figure 1 model, 64K context in Figure 1) and
7B-class grouped-query layers (32 query heads, 8 key/value heads of 128) up to
the 1M-token context of Table 6.  Routing vectors are drawn around random unit
centroids, standing in for the learned groups (Table 7's ~25% of pairs kept
at top-1 of 4 groups shows near-balanced groups; the skewed 0.4/0.3/0.2/0.1
mix follows Table 9's 40% group dominance at K=4).

Recipe (per workload, one integer seed):
  SeedSequence(seed).spawn(5) -> streams for centroids, group labels z,
  routing noise, q/k/v, sampled rows.
  centroids: standard normal [K, 16] float32, rows scaled to unit length,
             the same set for every routing head.
  z[h, t]  : categorical over K groups (uniform, or the workload's mix).
  r[h, t]  : centroids[z] + noise * standard normal, float32.
  q, k, v  : torch normal(0, 1) * qkv_std on the requested device, rounded to
             the workload dtype (bf16 by round-to-nearest-even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

D_ROUTE = 16  # routing dimension d_g (16 on every page that states it)


@dataclass(frozen=True)
class Workload:
    name: str
    n: int          # tokens (batch 1; batch folds into heads)
    hq: int         # query heads
    hkv: int        # key/value heads == routing heads
    d: int          # head dim
    K: int          # centroids (groups)
    topk: int       # groups per token
    window: int     # local window w (keys j with i - j < w)
    dtype: str      # "f32" or "bf16" for q, k, v, o
    z_probs: tuple | None = None   # None: uniform
    qkv_std: float = 1.0
    noise: float = 0.3

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def resized(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_fp32_n512": Workload("tiny_fp32_n512", 512, 2, 2, 64, 4, 1, 64, "f32"),
    "gpt2_n8k": Workload("gpt2_n8k", 8192, 12, 12, 64, 4, 2, 256, "bf16",
                         qkv_std=1.0 / math.sqrt(64)),
    "gpt2_n64k": Workload("gpt2_n64k", 65536, 12, 12, 64, 4, 2, 512, "bf16",
                          qkv_std=1.0 / math.sqrt(64)),
    "gqa7b_n128k_skew": Workload("gqa7b_n128k_skew", 131072, 32, 8, 128, 4, 2, 1024,
                                 "bf16", z_probs=(0.4, 0.3, 0.2, 0.1),
                                 qkv_std=1.0 / math.sqrt(128)),
    "gqa7b_n1m_k8": Workload("gqa7b_n1m_k8", 1048576, 32, 8, 128, 8, 2, 2048, "bf16",
                             qkv_std=1.0 / math.sqrt(128)),
}
WORKLOAD_ORDER = list(WORKLOADS)


# Context-length sweep in the shape of Table 6 (speed against full attention
# from 1K to 1M tokens, K = 4 and K = 8 centroid groups).  The pages give
# neither the model nor the window there; the sweep uses the 7B-style
# grouped-query layer above, top-1 membership (the O(n^2/K + n*w) reading)
# and w = 1024.
TABLE6_CONTEXTS = (1024, 4096, 16384, 32768, 65536, 262144, 1048576)
TABLE6_GROUPS = (4, 8)


def table6_workload(n: int, K: int) -> Workload:
    return Workload(f"table6_gqa7b_n{n}_k{K}", n, 32, 8, 128, K, 1, 1024, "bf16",
                    qkv_std=1.0 / math.sqrt(128))


# the top-k trade-off at K = 4 (thelatestinai.com Table 7), on the same layer
TABLE7_TOPK = (1, 2, 3, 4)


def table7_workload(n: int, topk: int, K: int = 4) -> Workload:
    name = f"table7_gqa7b_n{n}_top{topk}" + ("" if K == 4 else f"_k{K}")
    return Workload(name, n, 32, 8, 128, K, topk, 1024, "bf16", qkv_std=1.0 / math.sqrt(128))


def seed_for(name: str) -> int:
    if name in WORKLOAD_ORDER:
        return 1000 + WORKLOAD_ORDER.index(name)
    for i, n in enumerate(TABLE6_CONTEXTS):
        for j, K in enumerate(TABLE6_GROUPS):
            if name == f"table6_gqa7b_n{n}_k{K}":
                return 2000 + 10 * i + j
    if name.startswith("table7_gqa7b_n"):  # one routing draw per n, shared by every top-k
        return 3000 + int(name[len("table7_gqa7b_n"):].split("_")[0]) % 997
    return 4242


def _streams(seed: int):
    return np.random.SeedSequence(seed).spawn(5)


def routing_inputs(wl: Workload, seed: int):
    """(centroids float32 [Hkv, K, 16], r float32 [Hkv, n, 16], z int64 [Hkv, n])."""
    s_c, s_z, s_noise, _, _ = _streams(seed)
    c = np.random.default_rng(s_c).standard_normal((wl.K, D_ROUTE), dtype=np.float32)
    c /= np.linalg.norm(c, axis=1, keepdims=True).astype(np.float32)
    centroids = np.broadcast_to(c, (wl.hkv, wl.K, D_ROUTE)).copy()  # writable, contiguous
    p = None if wl.z_probs is None else np.asarray(wl.z_probs, np.float64)
    z = np.random.default_rng(s_z).choice(wl.K, size=(wl.hkv, wl.n), p=p)
    noise = np.random.default_rng(s_noise).standard_normal(
        (wl.hkv, wl.n, D_ROUTE), dtype=np.float32)
    r = (c[z] + np.float32(wl.noise) * noise).astype(np.float32)
    return centroids, np.ascontiguousarray(r), z


def qkv_inputs(wl: Workload, seed: int, device="cpu"):
    """q [Hq, n, d], k and v [Hkv, n, d] as torch tensors in the workload dtype."""
    import torch

    _, _, _, s_qkv, _ = _streams(seed)
    torch_seed = int(s_qkv.generate_state(1, np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)
    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16

    def draw(heads):
        out = torch.empty((heads, wl.n, wl.d), dtype=dt, device=device)
        for h in range(heads):  # per head keeps the float32 staging small
            x = torch.randn((wl.n, wl.d), generator=gen, device=device,
                            dtype=torch.float32)
            out[h] = (x * wl.qkv_std).to(dt)
        return out

    return draw(wl.hq), draw(wl.hkv), draw(wl.hkv)


def sample_rows(wl: Workload, seed: int, count: int, heads_per_pos: int = 1):
    """Seeded (query head, position) samples: the window and sequence edges
    first, then distinct random positions, each with a random query head.

    With heads_per_pos > 1 every sampled position is taken with that many
    distinct random query heads (count positions, count * heads_per_pos
    rows); the first head of each position is the one heads_per_pos = 1
    would give."""
    _, _, _, _, s_rows = _streams(seed)
    rng = np.random.default_rng(s_rows)
    n, w = wl.n, wl.window
    fixed = [p for p in (0, 1, w - 1, w, w + 1, n - 1) if 0 <= p < n]
    fixed = list(dict.fromkeys(fixed))
    want = max(0, min(count, n) - len(fixed))
    pool = np.setdiff1d(np.arange(n), np.asarray(fixed))
    extra = rng.choice(pool, size=min(want, pool.size), replace=False)
    pos = np.concatenate([np.asarray(fixed, np.int64), np.sort(extra).astype(np.int64)])
    heads = rng.integers(0, wl.hq, size=pos.size).astype(np.int32)
    if heads_per_pos <= 1:
        return heads, pos
    hp = min(heads_per_pos, wl.hq)
    more = np.empty((pos.size, hp), np.int32)
    more[:, 0] = heads
    for i in range(pos.size):  # the other heads: distinct, drawn without replacement
        others = np.delete(np.arange(wl.hq, dtype=np.int32), heads[i])
        more[i, 1:] = rng.choice(others, size=hp - 1, replace=False)
    return more.reshape(-1), np.repeat(pos, hp)


def to_bf16_bits(t) -> np.ndarray:
    """bf16 torch tensor -> numpy uint16 bit patterns (for the oracle)."""
    import torch

    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# Routing projection inputs (the step before routing: r_t = W x_t maps a
# d_model hidden state to the 16-dimensional routing space, one W per layer
# shared by its routing heads; 12 x 768 x 16 = 148K parameters for GPT-2 and
# 32 x 4096 x 16 = 2.1M for Mistral-7B, Tables 2 and 3).
@dataclass(frozen=True)
class ProjectionWorkload:
    name: str
    n: int          # tokens
    d_model: int    # hidden size
    heads: int      # routing heads (each with its own centroids)
    K: int
    topk: int
    dtype: str      # hidden-state dtype: "bf16" or "f32"


PROJECTION_WORKLOADS = {
    "gpt2_proj_n64k": ProjectionWorkload("gpt2_proj_n64k", 65536, 768, 12, 4, 2, "bf16"),
    "gqa7b_proj_n1m_k8": ProjectionWorkload("gqa7b_proj_n1m_k8", 1048576, 4096, 8, 8, 2,
                                            "bf16"),
}


def projection_inputs(pw: ProjectionWorkload, seed: int, device="cpu"):
    """(x torch [n, d_model] in pw.dtype on `device`, W float32 [16, d_model],
    centroids float32 [heads, K, 16]).

    x: standard normal hidden states; W: normal(0, 1/d_model) so that each
    routing coordinate has unit variance; centroids: standard normal rows
    scaled to unit length, drawn per routing head."""
    import torch

    s_c, s_w, s_x, _, _ = _streams(seed)
    c = np.random.default_rng(s_c).standard_normal((pw.heads, pw.K, D_ROUTE),
                                                   dtype=np.float32)
    c /= np.linalg.norm(c, axis=2, keepdims=True).astype(np.float32)
    W = (np.random.default_rng(s_w).standard_normal((D_ROUTE, pw.d_model), dtype=np.float32)
         * np.float32(1.0 / math.sqrt(pw.d_model))).astype(np.float32)
    torch_seed = int(s_x.generate_state(1, np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)
    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed)
    dt = torch.float32 if pw.dtype == "f32" else torch.bfloat16
    x = torch.empty((pw.n, pw.d_model), dtype=dt, device=device)
    rows = max(1, (1 << 26) // pw.d_model)   # float32 staging of at most 256 MiB
    for a in range(0, pw.n, rows):
        b = min(pw.n, a + rows)
        x[a:b] = torch.randn((b - a, pw.d_model), generator=gen, device=device,
                             dtype=torch.float32).to(dt)
    return x, np.ascontiguousarray(W), np.ascontiguousarray(c)


def dout_input(wl: Workload, seed: int, device="cpu"):
    """dL/dO for the backward: standard normal [Hq, n, d] in the workload
    dtype, from a stream of its own (seed + 7919, so it never repeats q)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) + 7919)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    out = torch.empty((wl.hq, wl.n, wl.d), dtype=dt, device=device)
    for h in range(wl.hq):
        out[h] = torch.randn((wl.n, wl.d), generator=gen, device=device,
                             dtype=torch.float32).to(dt)
    return out
