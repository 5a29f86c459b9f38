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


def test_issued_pairs_hand_cases():
    # resident tiles (B 64, d 128): rows round up to 32 per wave pass
    hist, own, pre = bench.issued_pairs([33, 0, 64], [100], 64, 128)
    assert hist == (64 + 0 + 64) * 64 and pre == 0
    # own block: blocks of 64 and 36 queries, one 128-column tile of one
    # 64-key chunk each
    assert own == 2 * 128 * 64
    # B 1024: 8-wave tiles of 256 rows; the own block of a 1500-token
    # sequence: block 0 has 8 tiles (chunks up to 2, 4, .., 16), block 1
    # (476 queries) 4 tiles (chunks 2, 4, 6, 8)
    hist, own, _ = bench.issued_pairs([300, 256, 1], [1500], 1024, 128)
    assert hist == (512 + 256 + 256) * 1024
    assert own == 128 * 64 * (sum(range(2, 17, 2)) + (2 + 4 + 6 + 8))
    # B 512 at d 128 is not resident: 4-wave tiles of 128 rows
    hist, _, _ = bench.issued_pairs([129], [512], 512, 128)
    assert hist == 256 * 512
    # d 64 keeps B 512 resident
    hist, _, _ = bench.issued_pairs([129], [512], 512, 64)
    assert hist == 160 * 512
    # the dense-prefix route at k 2, B 64: the own block of block 0 and 1 is
    # not issued (blocks 2..: 100 - 128 < 0, none here), the prefix launch
    # covers the first 128 positions in 4-wave tiles of 128 columns, 64-key
    # chunks up to the tile's last query
    _, own, pre = bench.issued_pairs([0, 0], [100], 64, 128, k=2, route=True)
    assert own == 0 and pre == 128 * 64 * 2
    _, own, pre = bench.issued_pairs([0, 0, 0], [150], 64, 128, k=2, route=True)
    assert own == 128 * 64 * 1 and pre == 128 * 64 * 2


@pytest.mark.parametrize("seqlens,B,k,H", [
    ([1000, 0, 129, 1, 300], 64, 4, 3),
    ([4096 + 17], 256, 12, 2),
    ([520, 1100], 128, 16, 2),
])
def test_pairs_by_kernel(seqlens, B, k, H):
    tot, hist, own = bench.attended_pairs(seqlens, B, k, H)
    assert bench.attended_pairs_by_kernel(seqlens, B, k, H, False) == (hist, own, 0)
    h2, o2, p2 = bench.attended_pairs_by_kernel(seqlens, B, k, H, True)
    assert h2 + o2 + p2 == tot
    # the prefix rows (own block below k) attend t + 1 keys each
    assert p2 == H * sum(min(L, k * B) * (min(L, k * B) + 1) // 2 for L in seqlens)


def test_prefix_route_follows_the_library():
    """bench.prefix_route mirrors moba_attn_fwd's choice (api.cpp: at least
    kPrefixMinGrid = 256 workgroups of a dense launch over all heads)."""
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    api = open(os.path.join(root, "block_sparse_long_03_amd", "csrc", "api.cpp")).read()
    launch = open(os.path.join(root, "block_sparse_long_03_amd", "csrc", "launch.h")).read()
    assert re.search(r"constexpr long long kPrefixMinGrid = 256;", api)
    assert "dense_grid(g, q_limit) >= moba::kPrefixMinGrid" in api
    assert "* g.num_seqs * g.num_heads;" in launch
    # 8K (16 heads, B 512, k 4): 8 tiles of 256 x 16 heads = 128 workgroups
    assert not bench.prefix_route([8192], 512, 4, 16, "bf16")
    # 32K (32 heads, B 256, k 32): 32 tiles x 32 heads
    assert bench.prefix_route([32768], 256, 32, 32, "bf16")
    assert bench.prefix_route([65536, 32768, 16384, 16384], 4096, 12, 32, "bf16")
    assert bench.prefix_route([1 << 20], 4096, 12, 32, "bf16")
    assert not bench.prefix_route([1 << 20], 4096, 12, 32, "f32")


def test_list_lengths_counts_historical_selections():
    import torch
    rng = np.random.default_rng(3)
    seqlens, B, k, H = [700, 0, 129, 300], 64, 4, 3
    rows = []
    for L in seqlens:
        for t in range(L):
            c = t // B
            rows.append([mo.select_row(rng.standard_normal(c), c, k)[0] for _ in range(H)])
    idx = torch.tensor(np.array(rows), dtype=torch.int32)
    got = bench.list_lengths(torch, idx, seqlens, B)
    cb = np.concatenate([[0], np.cumsum([(L + B - 1) // B for L in seqlens])])
    nb = int(cb[-1])
    want = np.zeros(H * nb, dtype=np.int64)
    t0 = 0
    for s, L in enumerate(seqlens):
        for t in range(L):
            c = t // B
            for h in range(H):
                for b in rows[t0 + t][h]:
                    if 0 <= b < c:
                        want[h * nb + cb[s] + b] += 1
        t0 += L
    assert np.array_equal(got, want)
    # every historical selection of a row lands in exactly one list
    assert got.sum() == sum(H * min(k - 1, t // B) for L in seqlens for t in range(L))
    # rows whose own block is below min_c are left out
    got2 = bench.list_lengths(torch, idx, seqlens, B, min_c=k)
    assert got2.sum() == sum(H * min(k - 1, t // B) for L in seqlens for t in range(L)
                             if t // B >= k)


def test_issued_pairs_follows_the_launch_policy():
    """bench.issued_pairs mirrors the tile policy of launch.h: keep the two
    in step (resident LDS budget, the 8-wave threshold)."""
    import re
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "block_sparse_long_03_amd", "csrc", "launch.h")).read()
    m = re.search(r"constexpr int kResidentLdsBytes = (\d+) \* (\d+);", src)
    assert m and int(m.group(1)) * int(m.group(2)) == bench.RESIDENT_LDS_BYTES
    assert re.search(r"return key_range >= 1024 \? 8 : 4;", src)
    assert re.search(r"return \(long long\)block_size \* head_dim \* 4 <= kResidentLdsBytes;", src)


def test_code_tokens_ignores_comments_only():
    """The traffic record stays valid across comment edits, not code edits."""
    a = "int x = 1;  // one\n/* block\n comment */ float y;\n"
    b = "int x = 1;\nfloat   y;  // another note\n"
    assert bench.code_tokens(a) == bench.code_tokens(b) == "int x = 1; float y;"
    assert bench.code_tokens("int x = 2;") != bench.code_tokens(a)
