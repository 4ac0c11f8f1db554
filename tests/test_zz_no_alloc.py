"""focus_bucket_noalloc (the bucketing with its counts in the library's fixed
per-device scratch) against focus_bucket with a caller workspace, through the
C ABI: two calls in a row on the same device, the second on a smaller input,
each bit-identical to the workspace form.  Collected last, so that it also
runs after every other test in the process."""
import numpy as np
import pytest
import torch

from centroid_gated_sparse_amd import focus as F

pytestmark = pytest.mark.gpu
DEV = "cuda"


def random_groups(H, n, K, topk, seed):
    rng = np.random.default_rng(seed)
    g = np.argsort(rng.random((H, n, K), dtype=np.float32), axis=-1)[..., :topk]
    return torch.from_numpy(np.ascontiguousarray(g, dtype=np.int32)).to(DEV)


def test_bucket_noalloc_matches_workspace_form():
    # the 1M-token 7B layer's bucketing (8 heads, K = 8, top-2: 4.5 MiB of
    # counts), then a smaller one that uses less of the scratch
    for H, n, K, topk, seed in [(8, 1 << 20, 8, 2, 11), (3, 5000, 6, 3, 12)]:
        print(f"noalloc bucket H={H} n={n} K={K} top{topk}", flush=True)
        need = F.focus_bucket_workspace_bytes(H, n, K, topk)
        assert need <= F.BUCKET_NOALLOC_SCRATCH_BYTES
        groups = random_groups(H, n, K, topk, seed)
        ref = F.focus_bucket(groups, K)
        # outputs pre-filled with garbage: every element must be written
        outs = [torch.full_like(t, -3) for t in ref]
        got = F.focus_bucket_noalloc(groups, K, *outs)
        torch.cuda.synchronize()
        for name, a, b in zip(("offsets", "tokens", "slot_entry"), got, ref):
            assert torch.equal(a, b), name
