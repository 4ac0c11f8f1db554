"""Host-side logic of bench.py (no GPU): the surviving-pair count that every
reported TFLOP/s figure divides by, checked against brute force."""
import numpy as np
import pytest

import bench


def _brute(groups, w):
    """|A(i)| summed over rows by the definition: j <= i with i - j < w, or
    sharing a group."""
    H, n, _ = groups.shape
    out = []
    for h in range(H):
        sets = [set(groups[h, t].tolist()) for t in range(n)]
        out.append(sum(1 for i in range(n) for j in range(i + 1)
                       if i - j < w or sets[i] & sets[j]))
    return np.array(out)


@pytest.mark.parametrize("K,topk,n,w", [(4, 1, 200, 16), (8, 2, 300, 0), (8, 3, 257, 40),
                                        (32, 4, 200, 7), (5, 5, 120, 3), (16, 2, 150, 500),
                                        (1, 1, 50, 5), (32, 3, 180, 1), (32, 1, 100, 0)])
def test_surviving_pairs_brute_force(K, topk, n, w):
    rng = np.random.default_rng(K * 1000 + topk * 10 + w)
    g = np.stack([np.stack([rng.permutation(K)[:topk] for _ in range(n)])
                  for _ in range(2)]).astype(np.int32)
    np.testing.assert_array_equal(bench.surviving_pairs(g, K, w), _brute(g, w))


def test_window_pairs_closed_form():
    for n, w in [(1, 1), (10, 3), (10, 10), (10, 50), (1000, 0)]:
        assert bench.window_pairs(n, w) == sum(min(i + 1, w) for i in range(n))
