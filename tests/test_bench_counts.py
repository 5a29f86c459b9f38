"""The flop counts behind bench.py's metric (CPU only): the attended (query,
key) pairs of the MoBA forward, split into historical and own-block pairs,
and the causal pairs of the dense baseline, against a brute-force count over
the oracle's own selection rule and attended-token sets (the count does not
depend on which blocks win, so random gate scores serve)."""

import os
import sys

import numpy as np
import pytest

from oracle import moba_oracle as mo

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _brute(seqlens, B, k, H, seed=0):
    rng = np.random.default_rng(seed)
    tot = hist = own = 0
    for L in seqlens:
        for t in range(L):
            c = t // B
            idx, _, _ = mo.select_row(rng.standard_normal(c), c, k)
            J = mo.attended_tokens(idx, t, B)
            tot += len(J)
            own += int(np.sum(J >= c * B))
    hist = tot - own
    return H * tot, H * hist, H * own


@pytest.mark.parametrize("seqlens,B,k,H", [
    ([1000, 0, 129, 1, 300], 64, 4, 3),
    ([4096 + 17], 256, 12, 2),
    ([640, 333], 128, 1, 1),
    ([520, 1100], 128, 16, 2),
])
def test_attended_pairs_matches_brute_force(seqlens, B, k, H):
    assert bench.attended_pairs(seqlens, B, k, H) == _brute(seqlens, B, k, H)


def test_dense_pairs_is_the_causal_count():
    seqlens = [300, 0, 17, 1000]
    assert bench.dense_pairs(seqlens, 3) == 3 * sum(L * (L + 1) // 2 for L in seqlens)
    # k >= n: MoBA attends exactly the causal pairs
    assert bench.attended_pairs(seqlens, 64, 64, 3)[0] == bench.dense_pairs(seqlens, 3)
