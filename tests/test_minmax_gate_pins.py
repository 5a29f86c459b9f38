"""Pins of the oracle's min/max pooled gate (CPU only).

Quest reads as MoBA with min/max pooling (research.elamur.ai, "Key points");
the score of a block is the largest value q . x takes over the box spanned by
the block's elementwise key minima and maxima.  Pinned to a hand-worked
example, to brute force over the box corners, to the upper-bound property, and
to the mean gate where the two must agree (one-token blocks).
"""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import moba_oracle as mo


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "minmax_example.json")) as f:
        return json.load(f)


def test_hand_worked_example(golden_dir):
    g = _golden(golden_dir)
    K = np.array(g["keys"], dtype=np.float64)
    B, k = g["block_size"], g["topk"]
    kmax, kmin = mo.pool_minmax_head(K, len(K), B)
    np.testing.assert_array_equal(kmax, g["kmax"])
    np.testing.assert_array_equal(kmin, g["kmin"])
    q = np.array(g["q"], dtype=np.float64)
    np.testing.assert_array_equal(mo.minmax_scores_row(q, kmax, kmin, 3), g["scores"])
    Q = np.zeros((len(K), 1, 2))
    Q[7, 0] = q
    res = mo.minmax_gate_reference(Q, K[:, None, :], [0, len(K)], B, k, rows=[[7, 0]])
    assert res["idx"][0].tolist() == g["idx_minmax"]
    mean = mo.gate_reference(Q, K[:, None, :], [0, len(K)], B, k, rows=[[7, 0]])
    assert mean["idx"][0].tolist() == g["idx_mean"]


def test_score_is_the_maximum_over_the_box_corners():
    rng = np.random.default_rng(7)
    d, B, L = 3, 5, 23
    K = rng.standard_normal((L, d))
    kmax, kmin = mo.pool_minmax_head(K, L, B)
    for _ in range(20):
        q = rng.standard_normal(d)
        s = mo.minmax_scores_row(q, kmax, kmin, len(kmax))
        for i in range(len(kmax)):
            corners = [np.dot(q, [kmin[i, e] if b[e] else kmax[i, e] for e in range(d)])
                       for b in itertools.product([0, 1], repeat=d)]
            assert s[i] == pytest.approx(max(corners), abs=1e-12)


def test_score_bounds_every_key_of_the_block():
    rng = np.random.default_rng(8)
    d, B, L = 16, 8, 61          # ragged last block of 5 tokens
    K = rng.standard_normal((L, d))
    kmax, kmin = mo.pool_minmax_head(K, L, B)
    for _ in range(10):
        q = rng.standard_normal(d)
        s = mo.minmax_scores_row(q, kmax, kmin, len(kmax))
        for i in range(len(kmax)):
            lo, hi = mo.block_range(i, L, B)
            assert np.all(K[lo:hi] @ q <= s[i] + 1e-12)
    # a block holding one token: the bound is that token's score
    kmax1, kmin1 = mo.pool_minmax_head(K[:1], 1, B)
    q = rng.standard_normal(d)
    assert mo.minmax_scores_row(q, kmax1, kmin1, 1)[0] == pytest.approx(K[0] @ q, abs=1e-12)


def test_one_token_blocks_select_like_the_mean_gate():
    rng = np.random.default_rng(9)
    T, H, d = 40, 2, 8
    Q = rng.standard_normal((T, H, d))
    K = rng.standard_normal((T, H, d))
    cu = [0, 25, 40]
    a = mo.minmax_gate_reference(Q, K, cu, 1, 4)
    b = mo.gate_reference(Q, K, cu, 1, 4)
    np.testing.assert_array_equal(a["idx"], b["idx"])


def test_pool_minmax_batch_layout():
    rng = np.random.default_rng(10)
    cu = [0, 13, 13, 40]
    K = rng.standard_normal((40, 3, 4))
    kmm = mo.pool_minmax(K, cu, 8)
    assert kmm.shape == (2 + 4, 3, 2, 4)
    np.testing.assert_array_equal(kmm[1, 2, 0], K[8:13, 2].max(axis=0))   # tail block
    np.testing.assert_array_equal(kmm[2, 1, 1], K[13:21, 1].min(axis=0))  # second sequence


def test_validity_checker_accepts_only_top_sets(golden_dir):
    g = _golden(golden_dir)
    K = np.array(g["keys"], dtype=np.float64)[:, None, :]
    Q = np.zeros((8, 1, 2))
    Q[7, 0] = g["q"]
    ok = lambda idx: mo.minmax_selection_is_valid(Q, K, [0, 8], 2, 2, (7, 0), idx)
    assert ok([2, 3]) and not ok([0, 3]) and not ok([3, -1]) and not ok([2, 4])


def test_pins_catch_planted_mistakes(golden_dir, monkeypatch):
    def min_instead_of_max(q, kmax, kmin, c):
        q = np.asarray(q, dtype=np.float64)
        return np.minimum(q * kmin[:c], q * kmax[:c]).sum(axis=1)

    def kmax_only(q, kmax, kmin, c):
        return (np.asarray(kmax[:c]) @ np.asarray(q, dtype=np.float64))

    def swapped_pool(K, L, B):
        kmax, kmin = orig_pool(K, L, B)
        return kmin, kmax

    orig_pool = mo.pool_minmax_head
    for fname, bad in (("minmax_scores_row", min_instead_of_max),
                       ("minmax_scores_row", kmax_only),
                       ("pool_minmax_head", swapped_pool)):
        with monkeypatch.context() as m:
            m.setattr(mo, fname, bad)
            caught = False
            for pin in (lambda: test_hand_worked_example(golden_dir),
                        test_score_is_the_maximum_over_the_box_corners):
                try:
                    pin()
                except (AssertionError, ValueError, IndexError):
                    caught = True
                    break
            assert caught, f"planted mistake {bad.__name__} not caught"
