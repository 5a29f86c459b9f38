"""Pins of the oracle's static routing rules (CPU only).

Sliding-window, attention-sink and full attention are fixed gates run through
the MoBA attention (wispaper review, "Why the Change Is Plausible"; the
sherconan.github.io summary, relations to other methods).  The oracle's
``static_select_row`` takes the rule step by step; these tests pin it to
hand-worked sets, to a closed-form token band built independently, to torch
SDPA in fp64 and to the learned gate on inputs whose scores grow with the
block index.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moba_oracle as mo


def _static_band_mask(cu, B, topk, sink):
    """Token mask of the static rule written as a band: with s = min(sink,
    k - 1), a query in block c attends to every block when c <= k - 1, else to
    blocks below s and blocks c - (k - 1 - s) .. c; causal inside, no
    cross-sequence attention."""
    T = int(cu[-1])
    M = np.zeros((T, T), dtype=bool)
    s = min(sink, topk - 1)
    for a, L in mo.sequences(cu):
        for t in range(L):
            c = t // B
            for j in range(t + 1):
                b = j // B
                if c <= topk - 1 or b < s or b >= c - (topk - 1 - s):
                    M[a + t, a + j] = True
    return M


def _rand(T, H, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((T, H, d)) for _ in range(3)]


def _sdpa_masked(q, k, v, mask, scale):
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x))[None, None] for x in (q, k, v))
    m = torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    lse = torch.logsumexp((qt @ kt.transpose(-1, -2) * scale).masked_fill(~m, -math.inf), dim=-1)
    return o[0, 0].numpy(), lse[0, 0].numpy()


def test_hand_worked_sets(golden_dir):
    with open(os.path.join(golden_dir, "static_sets.json")) as f:
        g = json.load(f)
    for c, k, sink, want in g["cases"]:
        got = mo.static_select_row(c, k, sink).tolist()
        assert got == want, (c, k, sink, got, want)


@pytest.mark.parametrize("topk,sink", [(3, 0), (3, 1), (4, 2), (2, 5), (1, 1)])
def test_static_matches_band_mask_sdpa(topk, sink):
    cu = np.array([0, 70, 70, 133, 200])  # ragged tails and an empty sequence
    T, H, d, B = 200, 2, 8, 8
    q, k, v = _rand(T, H, d, 11 + topk + 7 * sink)
    res = mo.static_reference(q, k, v, cu, B, topk, sink, 0.35)
    M = _static_band_mask(cu, B, topk, sink)
    for h in range(H):
        o_ref, lse_ref = _sdpa_masked(q[:, h], k[:, h], v[:, h], M, 0.35)
        sel = res["rows"][:, 1] == h
        np.testing.assert_allclose(res["out"][sel], o_ref, atol=1e-12)
        np.testing.assert_allclose(res["lse"][sel], lse_ref, atol=1e-12)


def test_static_full_is_dense_causal():
    # k >= n: the degenerate static gate is full causal attention
    cu = np.array([0, 61, 100])
    T, H, d, B = 100, 1, 8, 16
    q, k, v = _rand(T, H, d, 5)
    for sink in (0, 2):
        res = mo.static_reference(q, k, v, cu, B, 8, sink, 0.5)
        o_d, lse_d = mo.dense_causal_reference(q, k, v, cu, 0.5)
        np.testing.assert_allclose(res["out"], o_d, atol=1e-12)
        np.testing.assert_allclose(res["lse"], lse_d, atol=1e-12)


def test_window_equals_learned_gate_when_recent_blocks_score_highest():
    # keys of block i all equal i * u and every query is u: the gate score of
    # block i is i |u|^2, so the learned top-k keeps the most recent blocks
    # (a sliding window); with the first block made the strongest instead it
    # keeps block 0 plus the recent ones (a sink of one block)
    T, d, B, k = 96, 4, 8, 4
    u = np.array([1.0, 0.5, -0.25, 2.0])
    q = np.tile(u, (T, 1, 1))
    v = np.random.default_rng(2).standard_normal((T, 1, d))
    kk = np.stack([(j // B) * u for j in range(T)])[:, None, :]
    learned = mo.moba_reference(q, kk, v, [0, T], B, k, 0.1)
    static = mo.static_reference(q, kk, v, [0, T], B, k, 0, 0.1)
    np.testing.assert_array_equal(learned["idx"], static["idx"])
    kk[:B] = 100.0 * u
    learned = mo.moba_reference(q, kk, v, [0, T], B, k, 0.1)
    static = mo.static_reference(q, kk, v, [0, T], B, k, 1, 0.1)
    np.testing.assert_array_equal(learned["idx"], static["idx"])


def test_batch_selection_matches_rows():
    cu = np.array([0, 33, 33, 97, 100])
    idx = mo.static_select(cu, 8, 3, 1)
    for a, L in mo.sequences(cu):
        for t in range(L):
            np.testing.assert_array_equal(idx[a + t], mo.static_select_row(t // 8, 3, 1))


def test_static_rule_invariants():
    for c in range(0, 40):
        for k in (1, 2, 3, 5, 12):
            for sink in (0, 1, 2, 3, 20):
                idx = mo.static_select_row(c, k, sink)
                valid = [int(x) for x in idx if x >= 0]
                assert valid == sorted(set(valid)) and valid[-1] == c
                assert len(valid) == min(k, c + 1)
                assert list(idx[len(valid):]) == [-1] * (k - len(valid))
                s = min(sink, k - 1, c)
                assert valid[:s] == list(range(s))


def test_pins_catch_planted_mistakes(golden_dir, monkeypatch):
    orig = mo.static_select_row

    def window_off_by_one(c, topk, sink):      # walks back from c - 2
        taken = [c] + [i for i in range(min(sink, c, topk - 1))]
        j = c - 2
        while j >= 0 and len(taken) < topk:
            if j not in taken:
                taken.append(j)
            j -= 1
        idx = np.full(topk, -1, dtype=np.int64)
        idx[:len(taken)] = sorted(taken)
        return idx

    def sink_not_capped(c, topk, sink):        # sink crowds out the own block
        taken = list(range(min(sink, c + 1)))[:topk]
        j = c
        while j >= 0 and len(taken) < topk:
            if j not in taken:
                taken.append(j)
            j -= 1
        idx = np.full(topk, -1, dtype=np.int64)
        idx[:len(taken)] = sorted(taken)
        return idx

    def k_excludes_own(c, topk, sink):
        idx = orig(c, topk + 1, sink)
        return idx[:topk] if idx[topk] < 0 else idx[1:]

    for bad in (window_off_by_one, sink_not_capped, k_excludes_own):
        with monkeypatch.context() as m:
            m.setattr(mo, "static_select_row", bad)
            caught = False
            for pin in (lambda: test_hand_worked_sets(golden_dir),
                        lambda: test_static_matches_band_mask_sdpa(3, 1)):
                try:
                    pin()
                except (AssertionError, ValueError, IndexError):
                    caught = True
                    break
            assert caught, f"planted mistake {bad.__name__} not caught"
