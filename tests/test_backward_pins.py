"""Pins of the oracle's backward pass (CPU only).

Gradients flow through the softmax attention over the selected tokens; the
hard top-k selection is not differentiated (wispaper review, "The Change";
research.elamur.ai, "Key points").  The oracle writes the softmax-attention
gradients out; these tests pin it to torch autograd in fp64 where MoBA
reduces to a library routine (k >= n: dense causal; k = 1: block-diagonal
causal), to central finite differences of the oracle's own forward on a real
MoBA selection, and to identities the gradients satisfy exactly.
"""

import numpy as np
import pytest
import torch

from oracle import moba_oracle as mo


def _rand(T, H, d, seed, n=4):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((T, H, d)) for _ in range(n)]


def _autograd_masked(q, k, v, do, mask, scale):
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        qt[None, None], kt[None, None], vt[None, None], attn_mask=torch.from_numpy(mask)[None, None],
        scale=scale)[0, 0]
    (o * torch.from_numpy(do)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def _selection(q, k, cu, B, topk):
    T, H, _ = q.shape
    res = mo.moba_reference(q, k, k, cu, B, topk, 1.0)
    idx = np.full((T, H, topk), -1, dtype=np.int64)
    idx[res["rows"][:, 0], res["rows"][:, 1]] = res["idx"]
    return idx


def test_k_ge_n_is_dense_causal_autograd():
    cu = [0, 37, 37, 100]            # ragged, an empty sequence
    T, H, d, B = 100, 2, 8, 16
    q, k, v, do = _rand(T, H, d, 1)
    idx = _selection(q, k, cu, B, 8)
    dq, dk, dv = mo.moba_backward_reference(q, k, v, do, cu, B, idx, 0.3)
    for h in range(H):
        for a, L in mo.sequences(cu):
            if L == 0:
                continue
            M = np.tril(np.ones((L, L), dtype=bool))
            g = _autograd_masked(q[a:a + L, h], k[a:a + L, h], v[a:a + L, h], do[a:a + L, h], M, 0.3)
            for mine, ref in zip((dq, dk, dv), g):
                np.testing.assert_allclose(mine[a:a + L, h], ref, atol=1e-12)


def test_k1_is_block_diagonal_causal_autograd():
    cu = [0, 50, 96]
    T, H, d, B = 96, 1, 4, 8
    q, k, v, do = _rand(T, H, d, 2)
    idx = _selection(q, k, cu, B, 1)
    dq, dk, dv = mo.moba_backward_reference(q, k, v, do, cu, B, idx, 1.0)
    for a, L in mo.sequences(cu):
        M = np.zeros((L, L), dtype=bool)
        for t in range(L):
            M[t, (t // B) * B:t + 1] = True
        g = _autograd_masked(q[a:a + L, 0], k[a:a + L, 0], v[a:a + L, 0], do[a:a + L, 0], M, 1.0)
        for mine, ref in zip((dq, dk, dv), g):
            np.testing.assert_allclose(mine[a:a + L, 0], ref, atol=1e-12)


def test_finite_differences_on_a_moba_selection():
    # L(q, K, V) = sum(O * dO) through the oracle's forward with the selection
    # held fixed; central differences against the analytic gradients
    cu = [0, 29]
    T, H, d, B, topk = 29, 1, 3, 4, 3
    q, k, v, do = _rand(T, H, d, 3)
    idx = _selection(q, k, cu, B, topk)
    scale = 0.7

    def loss(q_, k_, v_):
        rows = np.stack([np.arange(T), np.zeros(T, dtype=np.int64)], axis=1)
        o, _ = mo.attend_given_selection(q_, k_, v_, cu, B, idx[:, 0], scale, rows)
        return float((o * do[:, 0]).sum())

    dq, dk, dv = mo.moba_backward_reference(q, k, v, do, cu, B, idx, scale)
    rng = np.random.default_rng(4)
    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(12):
            t, e = int(rng.integers(T)), int(rng.integers(d))
            args = [q.copy(), k.copy(), v.copy()]
            args[which][t, 0, e] += eps
            up = loss(*args)
            args[which][t, 0, e] -= 2 * eps
            dn = loss(*args)
            assert grad[t, 0, e] == pytest.approx((up - dn) / (2 * eps), abs=1e-7)


def test_gradient_identities():
    # rows of dS sum to zero, so the dK of a (sequence, head) sums to zero;
    # rows of P sum to one, so the dV of a sequence sums to the sum of dO;
    # a constant shift of every key leaves dQ (and dV) unchanged
    cu = [0, 40, 75]
    T, H, d, B = 75, 2, 6, 8
    q, k, v, do = _rand(T, H, d, 5)
    idx = _selection(q, k, cu, B, 3)
    dq, dk, dv = mo.moba_backward_reference(q, k, v, do, cu, B, idx, 0.5)
    for a, L in mo.sequences(cu):
        np.testing.assert_allclose(dk[a:a + L].sum(axis=0), 0.0, atol=1e-12)
        np.testing.assert_allclose(dv[a:a + L].sum(axis=0), do[a:a + L].sum(axis=0), atol=1e-12)
    shift = np.random.default_rng(6).standard_normal(d)
    dq2, dk2, dv2 = mo.moba_backward_reference(q, k + shift, v, do, cu, B, idx, 0.5)
    np.testing.assert_allclose(dq2, dq, atol=1e-12)
    np.testing.assert_allclose(dv2, dv, atol=1e-12)


def test_row_dq_matches_the_full_backward():
    # the row-local dQ (used where the full backward is too large) against
    # the full reference, which autograd and finite differences pin
    cu = [0, 61, 61, 130]
    T, H, d, B = 130, 2, 8, 8
    q, k, v, do = _rand(T, H, d, 8)
    idx = _selection(q, k, cu, B, 3)
    dq, _, _ = mo.moba_backward_reference(q, k, v, do, cu, B, idx, 0.4)
    rows = np.stack(np.meshgrid(np.arange(T), np.arange(H), indexing="ij"), -1).reshape(-1, 2)
    got = mo.backward_dq_rows(q, k, v, do, cu, B, idx[rows[:, 0], rows[:, 1]], 0.4, rows)
    np.testing.assert_allclose(got, dq[rows[:, 0], rows[:, 1]], atol=1e-12)


def test_key_rows_match_the_full_backward():
    # the key-local dK, dV (used at sizes where the full backward is too
    # large) against the full reference
    cu = [0, 61, 61, 130]
    T, H, d, B = 130, 2, 8, 8
    q, k, v, do = _rand(T, H, d, 9)
    idx = _selection(q, k, cu, B, 3)
    _, dk, dv = mo.moba_backward_reference(q, k, v, do, cu, B, idx, 0.4)
    keys = np.stack(np.meshgrid(np.arange(T), np.arange(H), indexing="ij"), -1).reshape(-1, 2)
    gk, gv = mo.backward_dkdv_keys(q, k, v, do, cu, B, idx, 0.4, keys)
    np.testing.assert_allclose(gk, dk[keys[:, 0], keys[:, 1]], atol=1e-12)
    np.testing.assert_allclose(gv, dv[keys[:, 0], keys[:, 1]], atol=1e-12)


def test_token_mask_matches_brute_force_mask():
    cu = [0, 45]
    T, H, d, B = 45, 1, 4, 8
    q, k, _, _ = _rand(T, H, d, 7)
    idx = _selection(q, k, cu, B, 3)
    np.testing.assert_array_equal(mo.token_mask(idx[:, 0], T, B),
                                  mo.brute_force_mask(cu, B, idx[:, 0]))


def test_pins_catch_planted_mistakes(monkeypatch):
    orig = mo.attention_backward_masked

    def no_softmax_jacobian_term(Q, K, V, dO, M, scale):
        Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dO))
        X = np.where(M, scale * (Q @ K.T), -np.inf)
        P = np.exp(X - X.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        dS = P * (dO @ V.T)                       # drops rowsum(dO * O)
        return scale * dS @ K, scale * dS.T @ Q, P.T @ dO

    def unscaled_dk(Q, K, V, dO, M, scale):
        dq, dk, dv = orig(Q, K, V, dO, M, scale)
        return dq, dk / scale, dv

    def transposed_dv(Q, K, V, dO, M, scale):
        dq, dk, dv = orig(Q, K, V, dO, M, scale)
        X = np.where(M, scale * (np.asarray(Q) @ np.asarray(K).T), -np.inf)
        P = np.exp(X - X.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        return dq, dk, P @ np.asarray(dO, dtype=np.float64)

    for bad in (no_softmax_jacobian_term, unscaled_dk, transposed_dv):
        with monkeypatch.context() as m:
            m.setattr(mo, "attention_backward_masked", bad)
            caught = False
            for pin in (test_k_ge_n_is_dense_causal_autograd, test_finite_differences_on_a_moba_selection):
                try:
                    pin()
                except AssertionError:
                    caught = True
                    break
            assert caught, f"planted mistake {bad.__name__} not caught"
