"""Pins for the fp64 CPU oracle: every check here compares the oracle with
something other than itself -- hand-worked examples, the sparsity values the
pages print, library routines (torch SDPA in fp64) for the cases the pages say
MoBA reduces to, closed forms, brute force and invariants.  The last group
plants plausible mistakes into the oracle and checks that a pin catches each.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import moba_oracle as mo

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------

def _num(x):
    """Parse a golden-file number: int, float, 'p/q', 'ln2', 'e/(e+1)' ..."""
    if isinstance(x, (int, float)):
        return float(x)
    s = str(x)
    if s.startswith("ln"):
        return math.log(float(s[2:]))
    if "e" in s:
        return float(eval(s, {"__builtins__": {}}, {"e": math.e}))
    return float(Fraction(s))


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        g = json.load(f)
    arr = lambda key: np.array([[_num(v) for v in row] for row in g[key]], dtype=np.float64)
    q, k, v = arr("q"), arr("k"), arr("v")
    return g, q[:, None, :], k[:, None, :], v[:, None, :]


def _rand(T, H, d, seed, dtype=np.float64):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((T, H, d)).astype(dtype) for _ in range(3)]


def _sdpa_masked(q, k, v, mask, scale):
    """torch SDPA in fp64 on one head: q, k, v [T, d], mask [T, T] bool."""
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, None]
    kt = torch.from_numpy(np.ascontiguousarray(k))[None, None]
    vt = torch.from_numpy(np.ascontiguousarray(v))[None, None]
    m = torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    x = (qt @ kt.transpose(-1, -2)) * scale
    lse = torch.logsumexp(x.masked_fill(~m, -math.inf), dim=-1)
    return o[0, 0].numpy(), lse[0, 0].numpy()


# --------------------------------------------------------------------------
# hand-worked examples
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["e1_two_blocks.json", "e2_three_blocks.json", "e2_tie.json"])
def test_golden_examples(golden_dir, name):
    g, q, k, v = _load(golden_dir, name)
    T = q.shape[0]
    cu = [0, T]
    for case in g["cases"]:
        rows = case.get("rows", list(range(T)))
        rr = np.array([[t, 0] for t in rows])
        res = mo.moba_reference(q, k, v, cu, g["block_size"], case["topk"], g["scale"], rows=rr)
        assert res["idx"].tolist() == case["idx"], case["what"]
        o_exp = np.array([[_num(x) for x in row] for row in case["o"]])
        np.testing.assert_allclose(res["out"], o_exp, rtol=0, atol=1e-12, err_msg=case["what"])
        lse_exp = np.log([_num(x) for x in case["exp_lse"]])
        np.testing.assert_allclose(res["lse"], lse_exp, rtol=0, atol=1e-12, err_msg=case["what"])


def test_tie_is_flagged_as_near_tie(golden_dir):
    g, q, k, v = _load(golden_dir, "e2_tie.json")
    # with k = 2 and c = 2 there is a k-th candidate, and the gap is exactly 0
    res = mo.moba_reference(q, k, v, [0, 6], 2, 2, 1.0, rows=np.array([[5, 0]]))
    assert res["gap"][0] == 0.0 and res["near_tie"][0]


# --------------------------------------------------------------------------
# the sparsity values the pages print
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N,B,k,printed", [
    (8192, 512, 3, 0.8125),      # wispaper "The Change": 1536 of 8192 positions, 81.25 %
    (32768, 512, 3, 0.9531),     # wispaper "The Change": 32K trailing-loss setting, 95.31 %
    (1 << 20, 4096, 12, 0.9531),  # wispaper "Real-World LLM ...": 1M, B 4096, k 12, 95.31 %
    (131072, 4096, 12, 0.625),   # cn-summary benchmark table: RULER @128K, 62.5 %
])
def test_printed_sparsity(N, B, k, printed):
    assert round(mo.sparsity(N, B, k), 4) == printed


def test_1536_of_8192_positions():
    # wispaper "The Change": B = 512, k = 3 -> the model attends to 1536 of 8192
    c = 8191 // 512
    idx, _, _ = mo.select_row(np.random.default_rng(1).standard_normal(c), c, 3)
    assert len(mo.attended_tokens(idx, 8191, 512)) == 1536


# --------------------------------------------------------------------------
# reductions to library routines
# --------------------------------------------------------------------------

def _causal_mask(cu, T):
    M = np.zeros((T, T), dtype=bool)
    for a, L in mo.sequences(cu):
        M[a:a + L, a:a + L] = np.tril(np.ones((L, L), dtype=bool))
    return M


def test_k_ge_n_is_dense_causal_sdpa():
    # wispaper "The Change": k = n recovers full attention
    cu = [0, 37, 37, 100, 164]       # ragged tails and an empty sequence
    T, H, d, B = 164, 2, 8, 16
    q, k, v = _rand(T, H, d, 3)
    scale = 0.3
    res = mo.moba_reference(q, k, v, cu, B, topk=8, scale=scale)
    M = _causal_mask(cu, T)
    for h in range(H):
        o_ref, lse_ref = _sdpa_masked(q[:, h], k[:, h], v[:, h], M, scale)
        sel = res["rows"][:, 1] == h
        np.testing.assert_allclose(res["out"][sel], o_ref, atol=1e-12)
        np.testing.assert_allclose(res["lse"][sel], lse_ref, atol=1e-12)
    o_d, lse_d = mo.dense_causal_reference(q, k, v, cu, scale)
    np.testing.assert_allclose(o_d, res["out"], atol=1e-12)
    np.testing.assert_allclose(lse_d, res["lse"], atol=1e-12)


def test_k1_is_block_diagonal_causal_sdpa():
    # elamur "Related methods": top-1 gating (LongHeads); with k = 1 only the
    # forced own block remains: block-diagonal causal attention
    cu = [0, 50, 96]
    T, H, d, B = 96, 2, 4, 8
    q, k, v = _rand(T, H, d, 4)
    res = mo.moba_reference(q, k, v, cu, B, topk=1, scale=1.0)
    M = np.zeros((T, T), dtype=bool)
    for a, L in mo.sequences(cu):
        for t in range(L):
            c = t // B
            M[a + t, a + c * B:a + t + 1] = True
    for h in range(H):
        o_ref, lse_ref = _sdpa_masked(q[:, h], k[:, h], v[:, h], M, 1.0)
        sel = res["rows"][:, 1] == h
        np.testing.assert_allclose(res["out"][sel], o_ref, atol=1e-12)
        np.testing.assert_allclose(res["lse"][sel], lse_ref, atol=1e-12)


def test_dense_reference_against_sdpa_is_causal():
    T, d = 70, 16
    q, k, v = _rand(T, 1, d, 5)
    o, lse = mo.dense_causal_reference(q, k, v, [0, T], 0.25)
    qt, kt, vt = (torch.from_numpy(x[:, 0])[None, None] for x in (q, k, v))
    o_ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.25)
    np.testing.assert_allclose(o, o_ref[0, 0].numpy(), atol=1e-12)


# --------------------------------------------------------------------------
# second formulation: the token-level block mask
# --------------------------------------------------------------------------

def test_brute_force_mask_matches_rowwise():
    cu = [0, 45, 64, 131]
    T, H, d, B, k = 131, 2, 6, 8, 3
    q, kk, v = _rand(T, H, d, 6)
    res = mo.moba_reference(q, kk, v, cu, B, k, 0.5)
    for h in range(H):
        sel = res["rows"][:, 1] == h
        M = mo.brute_force_mask(cu, B, res["idx"][sel])
        # the mask never reaches the future or another sequence
        assert not np.any(M & ~_causal_mask(cu, T))
        o, lse = mo.masked_softmax_attention(q[:, h], kk[:, h], v[:, h], M, 0.5)
        np.testing.assert_allclose(res["out"][sel], o, atol=1e-12)
        np.testing.assert_allclose(res["lse"][sel], lse, atol=1e-12)
        # at most k*B keys per query (glossary "Mathematical and complexity implications")
        assert M.sum(axis=1).max() <= k * B


# --------------------------------------------------------------------------
# selection: brute force and causality invariants
# --------------------------------------------------------------------------

def _rank_count_select(scores, topk):
    c = len(scores)
    chosen = []
    for i in range(c):
        rank = sum(1 for j in range(c) if scores[j] > scores[i] or (scores[j] == scores[i] and j < i))
        if rank < topk - 1:
            chosen.append(i)
    return chosen


def test_selection_equals_rank_counting_with_ties():
    rng = np.random.default_rng(7)
    for trial in range(400):
        c = int(rng.integers(0, 14))
        topk = int(rng.integers(1, 9))
        scores = rng.integers(-3, 4, size=c).astype(np.float64)  # many exact ties
        idx, _, _ = mo.select_row(scores, c, topk)
        want = _rank_count_select(scores, topk) + [c]
        assert [x for x in idx if x >= 0] == want
        assert list(idx[len(want):]) == [-1] * (topk - len(want))


def test_causality_invariants():
    cu = [0, 300, 333]
    T, H, d, B, k = 333, 3, 5, 16, 5
    q, kk, v = _rand(T, H, d, 8)
    g = mo.gate_reference(q, kk, cu, B, k)
    for (t, h), row in zip(g["rows"], g["idx"]):
        a = 0 if t < 300 else 300
        c = (t - a) // B
        valid = [x for x in row if x >= 0]
        assert valid == sorted(valid) and len(set(valid)) == len(valid)
        assert valid[-1] == c                     # own block always selected
        assert all(x <= c for x in valid)         # no future block
        assert len(valid) == min(k, c + 1)        # k counts the own block
        assert list(row[len(valid):]) == [-1] * (k - len(valid))


def test_gate_reference_agrees_with_rowwise_driver():
    cu = [0, 200]
    q, kk, v = _rand(200, 2, 4, 9)
    a = mo.gate_reference(q, kk, cu, 8, 4)
    b = mo.moba_reference(q, kk, v, cu, 8, 4, 1.0)
    assert np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(a["near_tie"], b["near_tie"])


def test_vectorised_selection_matches_rowwise_with_ties():
    rng = np.random.default_rng(19)
    for trial in range(60):
        c = int(rng.integers(0, 12))
        topk = int(rng.integers(1, 8))
        S = rng.integers(-2, 3, size=(9, c)).astype(np.float64)
        S[::3] += rng.standard_normal((3, c)) * 1e-7   # near-ties as well
        idx, gap, near = mo.select_rows(S, c, topk)
        for r in range(9):
            i1, g1, n1 = mo.select_row(S[r], c, topk)
            assert idx[r].tolist() == i1.tolist()
            assert near[r] == n1 and (gap[r] == g1 or (np.isinf(gap[r]) and np.isinf(g1)))


def test_near_tie_threshold():
    idx, gap, near = mo.select_row(np.array([1.0, 1.0 + 5e-6, 3.0]), 3, 3)
    assert near and idx.tolist() == [1, 2, 3]
    idx, gap, near = mo.select_row(np.array([1.0, 1.0 + 5e-5, 3.0]), 3, 3)
    assert not near


def test_selection_validity_checker():
    cu = [0, 64]
    q, kk, v = _rand(64, 1, 4, 10)
    g = mo.gate_reference(q, kk, cu, 8, 3)
    for (t, h), row in zip(g["rows"], g["idx"]):
        assert mo.selection_is_valid(q, kk, cu, 8, 3, (t, h), row)
    t = 63  # c = 7: swap a chosen past block for an unchosen one
    row = list(g["idx"][t])
    other = [i for i in range(7) if i not in row][0]
    bad = sorted([row[0], other]) + [7]
    assert not mo.selection_is_valid(q, kk, cu, 8, 3, (t, 0), bad)
    assert not mo.selection_is_valid(q, kk, cu, 8, 3, (t, 0), [row[0], 7, -1][:3])


# --------------------------------------------------------------------------
# pooling: closed forms
# --------------------------------------------------------------------------

def test_pool_closed_form_and_tail():
    L, B, d = 21, 8, 3
    K = np.arange(L * d, dtype=np.float64).reshape(L, d)   # K[j, e] = 3j + e
    kb = mo.pool_keys_head(K, L, B)
    # block i mean over j in [8i, min(8i+8, 21)) of 3j + e = 3 * mean(j) + e
    for i, (lo, hi) in enumerate([(0, 8), (8, 16), (16, 21)]):
        np.testing.assert_array_equal(kb[i], 3 * (lo + hi - 1) / 2 + np.arange(d))


def test_pool_batch_layout():
    cu = [0, 10, 10, 25]
    K = np.random.default_rng(11).standard_normal((25, 2, 3))
    kb = mo.pool_keys(K, cu, 4)
    assert kb.shape == (3 + 0 + 4, 2, 3)
    np.testing.assert_allclose(kb[3], K[10:14].mean(axis=0))
    np.testing.assert_allclose(kb[6], K[22:25].mean(axis=0))


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def test_weights_sum_to_one():
    cu = [0, 90]
    q, k, _ = _rand(90, 2, 4, 12)
    res = mo.moba_reference(q, k, np.ones_like(q), cu, 8, 3, 0.7)
    np.testing.assert_allclose(res["out"], 1.0, atol=1e-13)


def test_linear_in_v():
    cu = [0, 70]
    q, k, v1 = _rand(70, 1, 4, 13)
    v2 = np.random.default_rng(14).standard_normal(v1.shape)
    r1 = mo.moba_reference(q, k, v1, cu, 8, 3, 0.7)
    r2 = mo.moba_reference(q, k, v2, cu, 8, 3, 0.7)
    r3 = mo.moba_reference(q, k, 2 * v1 - 3 * v2, cu, 8, 3, 0.7)
    np.testing.assert_allclose(r3["out"], 2 * r1["out"] - 3 * r2["out"], atol=1e-12)


def test_constant_key_shift():
    cu = [0, 96]
    q, k, v = _rand(96, 2, 4, 15)
    shift = np.array([0.5, -1.0, 2.0, 0.25])
    r1 = mo.moba_reference(q, k, v, cu, 8, 4, 0.6)
    r2 = mo.moba_reference(q, k + shift, v, cu, 8, 4, 0.6)
    assert np.array_equal(r1["idx"], r2["idx"])
    np.testing.assert_allclose(r1["out"], r2["out"], atol=1e-12)
    qs = q[r1["rows"][:, 0], r1["rows"][:, 1]] @ shift
    np.testing.assert_allclose(r2["lse"], r1["lse"] + 0.6 * qs, atol=1e-12)


def test_permutation_inside_a_past_block():
    cu = [0, 64]
    q, k, v = _rand(64, 1, 4, 16)
    perm = np.arange(64)
    perm[8:16] = np.random.default_rng(17).permutation(np.arange(8, 16))
    r1 = mo.moba_reference(q, k, v, cu, 8, 3, 1.0)
    r2 = mo.moba_reference(q, k[perm], v[perm], cu, 8, 3, 1.0)
    later = r1["rows"][:, 0] >= 16
    assert np.array_equal(r1["idx"][later], r2["idx"][later])
    np.testing.assert_allclose(r1["out"][later], r2["out"][later], atol=1e-12)
    np.testing.assert_allclose(r1["lse"][later], r2["lse"][later], atol=1e-12)


def test_sequences_do_not_interact():
    cu = [0, 40, 73]
    q, k, v = _rand(73, 2, 4, 18)
    rb = mo.moba_reference(q, k, v, cu, 8, 3, 1.0)
    r0 = mo.moba_reference(q[:40], k[:40], v[:40], [0, 40], 8, 3, 1.0)
    r1 = mo.moba_reference(q[40:], k[40:], v[40:], [0, 33], 8, 3, 1.0)
    np.testing.assert_allclose(rb["out"], np.concatenate([r0["out"], r1["out"]]), atol=1e-13)
    assert np.array_equal(rb["idx"], np.concatenate([r0["idx"], r1["idx"]]))


# --------------------------------------------------------------------------
# planted mistakes: each must be caught by a pin above
# --------------------------------------------------------------------------

def _golden_ok(golden_dir):
    try:
        for n in ["e1_two_blocks.json", "e2_three_blocks.json", "e2_tie.json"]:
            test_golden_examples(golden_dir, n)
        return True
    except (AssertionError, ValueError, IndexError):
        return False


def test_pins_catch_planted_mistakes(golden_dir, monkeypatch):
    assert _golden_ok(golden_dir)

    def reversed_tiebreak(scores, c, topk):
        order = np.lexsort((-np.arange(c), -scores))
        take = min(topk - 1, c)
        chosen = sorted(int(i) for i in order[:take]) + [c]
        idx = np.full(topk, -1, dtype=np.int64)
        idx[:len(chosen)] = chosen
        return idx, np.inf, False

    def no_diagonal(idx_row, t, B):
        c = t // B
        parts = [np.arange(i * B, (i + 1) * B) for i in idx_row if 0 <= i < c]
        parts.append(np.arange(c * B, t))          # drops the query itself
        return np.concatenate(parts)

    def whole_own_block(idx_row, t, B):
        parts = [np.arange(i * B, (i + 1) * B) for i in idx_row if i >= 0]
        return np.concatenate(parts)                # leaks the future

    def sum_pool(K, L, B):
        n = mo.num_blocks(L, B)
        return np.stack([np.asarray(K[i * B:min(L, i * B + B)], np.float64).sum(0) for i in range(n)])

    def k_excludes_own(scores, c, topk):
        order = np.lexsort((np.arange(c), -scores))
        chosen = sorted(int(i) for i in order[:min(topk, c)]) + [c]
        idx = np.full(topk + 1, -1, dtype=np.int64)
        idx[:len(chosen)] = chosen
        return idx[:topk] if len(chosen) <= topk else idx, np.inf, False

    def unscaled_attend(q, K, V, J, scale):
        return orig_attend(q, K, V, J, 1.0 if scale != 1.0 else 2.0)

    orig_attend = mo.attend_row
    mutants = [("select_row", reversed_tiebreak), ("attended_tokens", no_diagonal),
               ("attended_tokens", whole_own_block), ("pool_keys_head", sum_pool),
               ("select_row", k_excludes_own), ("attend_row", unscaled_attend)]
    for fname, bad in mutants:
        with monkeypatch.context() as m:
            m.setattr(mo, fname, bad)
            caught = not _golden_ok(golden_dir)
            for pin in (test_k_ge_n_is_dense_causal_sdpa,
                        lambda: test_printed_sparsity(8192, 512, 3, 0.8125),
                        test_pool_closed_form_and_tail):
                if caught:
                    break
                try:
                    pin()
                except (AssertionError, ValueError, IndexError):
                    caught = True
            assert caught, f"planted mistake in {fname} ({bad.__name__}) not caught"
