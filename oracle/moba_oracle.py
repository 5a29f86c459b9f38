"""Plain fp64 CPU oracle for the MoBA causal prefill forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and imports nothing from it.

Sources (the pages are cited by title and section):

* [wispaper] "MoBA: Learned Block Sparsity for Long-Context Attention"
  (wispaper.ai review), sections "Starting Point: Exact Softmax Attention and
  Its Cost", "The Change: Treat KV Blocks as Experts and Route Queries with
  Top-k Gating" and "Efficiency and Implementation" (Algorithm 1).
* [glossary] "Mixture of Block Attention (MoBA)" (globaladvisors.biz),
  section "Underlying computational mechanism" (the text formula
  MoBA(q,K,V) = Softmax(q K[I]^T) V[I]) and "Mathematical and complexity
  implications" (at most k*B keys per query).
* [cn-summary] "MoBA: 面向长上下文大语言模型的混合块注意力机制"
  (sherconan.github.io), 技术实现 steps 1-4 (block partition, mean-pooled
  affinity s_i = <q, mean_pool(K[I_i])>, top-k gate, causality rules).
* [elamur] "MoBA: Mixture of Block Attention for Long-Context LLMs"
  (research.elamur.ai), "Key points" (causality: future blocks masked out of
  routing, own block always selected with a causal mask).

What is computed, per sequence s (start a, length L), head h and local query
position t with own block c = t // B:

1. pool:   kbar_i = mean of K[a+j] over j in [iB, min((i+1)B, L))
2. gate:   s_i = <Q[a+t], kbar_i> for past blocks i < c (no scale: a positive
           scale cannot change a ranking)
3. select: the first min(k-1, c) of 0..c-1 ordered by (-s_i, i); the own block
           c is added (k counts it); idx = sorted selection, -1 padded to k
4. tokens: J = union of the selected past blocks' tokens, plus [cB, t]
5. attend: x_j = scale * <Q[a+t], K[a+j]>, lse = ln sum_{j in J} exp(x_j),
           o = sum_j exp(x_j - lse) V[a+j]

Blockwise attention followed by an online-softmax merge reaches exactly this
softmax over J (the merge is an exact identity), so the oracle computes the
softmax over J directly and never merges.

Every function here is pinned by ``tests/test_oracle_pins.py`` (the static
routing rules by ``tests/test_static_gate_pins.py``, the min/max pooled gate
by ``tests/test_minmax_gate_pins.py``, the backward pass by
``tests/test_backward_pins.py``) against hand
worked examples, library routines (torch SDPA in fp64 for the k >= n and k = 1
reductions), closed forms and invariants.  The pages print no numeric output
of the operator itself; the only printed numbers this oracle reproduces are
the sparsity values of the selection geometry.
"""

from __future__ import annotations

import numpy as np

# Relative gap below which the k-1-th and k-th largest past scores count as a
# near-tie (selection then is ambiguous at fp32 score precision).
NEAR_TIE_REL = 1e-5


# --------------------------------------------------------------------------
# geometry
# --------------------------------------------------------------------------

def sequences(cu_seqlens):
    """(start, length) of every sequence of a packed batch."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(int(cu[i]), int(cu[i + 1] - cu[i])) for i in range(len(cu) - 1)]


def num_blocks(length, block_size):
    """Blocks of size B covering L tokens; the last may be partial."""
    return (length + block_size - 1) // block_size


def block_range(i, length, block_size):
    """Local token range [lo, hi) of block i ([wispaper] "The Change": block
    partition I_i; 0-based here, partial last block allowed)."""
    lo = i * block_size
    return lo, min(lo + block_size, length)


# --------------------------------------------------------------------------
# steps 1-3: pool, gate, select (one sequence, one head)
# --------------------------------------------------------------------------

def pool_keys_head(K, length, block_size):
    """Step 1: mean-pooled key of every block of one sequence and head.

    K: [L, d] (any float dtype, converted to fp64 block by block).
    Returns kbar [n, d] fp64.  [wispaper] "The Change" (mean_pool(K[I_i]));
    [cn-summary] step 2.
    """
    n = num_blocks(length, block_size)
    d = K.shape[1]
    kbar = np.zeros((n, d), dtype=np.float64)
    for i in range(n):
        lo, hi = block_range(i, length, block_size)
        kbar[i] = np.asarray(K[lo:hi], dtype=np.float64).mean(axis=0)
    return kbar


def gate_scores_row(q, kbar, c):
    """Step 2: affinity of query q with every past block i < c."""
    return np.asarray(kbar[:c], dtype=np.float64) @ np.asarray(q, dtype=np.float64)


def select_row(scores, c, topk):
    """Step 3: causal top-k selection for a query whose own block is c.

    scores: the c past-block scores.  Future blocks are never candidates, the
    own block is always taken and counts toward k, the remaining k-1 slots go
    to the highest scores with ties broken toward the lower block index.
    When c < k-1 there are not enough eligible blocks and the row keeps every
    block 0..c (masked blocks are never selected to fill slots).

    Returns (idx [topk] int64 ascending, -1 padded; gap; near_tie).
    gap is s_(k-1) - s_(k) between the (k-1)-th and k-th largest past scores
    when a k-th candidate exists (c >= k), else +inf.
    """
    order = np.lexsort((np.arange(c), -scores))  # primary: -s, secondary: index
    take = min(topk - 1, c)
    chosen = sorted(int(i) for i in order[:take]) + [c]
    idx = np.full(topk, -1, dtype=np.int64)
    idx[:len(chosen)] = chosen
    gap, near = np.inf, False
    if topk >= 2 and c >= topk:
        a = scores[order[topk - 2]]
        b = scores[order[topk - 1]]
        gap = float(a - b)
        near = bool(gap < NEAR_TIE_REL * max(abs(a), abs(b)))
    return idx, gap, near


def attended_tokens(idx_row, t, block_size):
    """Step 4: local key positions attended by local query t given its idx row.

    Past blocks contribute all their tokens; the own block contributes
    [cB, t] (causal mask inside the own block, diagonal included).
    [wispaper] "The Change" (causality rule); [elamur] "Key points".
    """
    c = t // block_size
    parts = []
    for i in idx_row:
        i = int(i)
        if i < 0:
            continue
        if i < c:
            parts.append(np.arange(i * block_size, (i + 1) * block_size))
        elif i == c:
            parts.append(np.arange(c * block_size, t + 1))
        else:
            raise ValueError("future block in selection")
    return np.concatenate(parts)


def attend_row(q, K, V, J, scale):
    """Step 5: exact softmax attention of q over key positions J.

    [glossary] "Underlying computational mechanism": Softmax(q K[I]^T) V[I].
    Returns (o [d] fp64, lse fp64 natural log).
    """
    q = np.asarray(q, dtype=np.float64)
    Kj = np.asarray(K[J], dtype=np.float64)
    Vj = np.asarray(V[J], dtype=np.float64)
    x = scale * (Kj @ q)
    mx = x.max()
    w = np.exp(x - mx)
    den = w.sum()
    lse = mx + np.log(den)
    o = (w / den) @ Vj
    return o, lse


# --------------------------------------------------------------------------
# whole-batch drivers
# --------------------------------------------------------------------------

def _rows_by_head(rows, T, H):
    """rows: None (all) or an int array of (token, head) pairs [R, 2]."""
    if rows is None:
        tt, hh = np.meshgrid(np.arange(T), np.arange(H), indexing="ij")
        return np.stack([tt.ravel(), hh.ravel()], axis=1)
    return np.asarray(rows, dtype=np.int64).reshape(-1, 2)


def _seq_of_token(cu_seqlens, t):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    s = int(np.searchsorted(cu, t, side="right") - 1)
    return s, int(cu[s]), int(cu[s + 1] - cu[s])


def pool_keys(K, cu_seqlens, block_size):
    """Step 1 over a packed batch: K [T, H, d] -> kbar [NB, H, d] fp64, blocks
    numbered sequence by sequence (blocks never cross sequences)."""
    T, H, d = K.shape
    out = []
    for a, L in sequences(cu_seqlens):
        n = num_blocks(L, block_size)
        kb = np.zeros((n, H, d))
        for h in range(H):
            kb[:, h, :] = pool_keys_head(K[a:a + L, h, :], L, block_size)
        out.append(kb)
    return np.concatenate(out, axis=0) if out else np.zeros((0, H, d))


def moba_reference(Q, K, V, cu_seqlens, block_size, topk, scale, rows=None):
    """The MoBA forward on (token, head) rows of a packed batch.

    Q, K, V: [T, H, d] arrays (bf16 values held exactly in fp32, or fp32/fp64).
    rows: None for every row, else [R, 2] (global token, head) pairs.
    Returns dict with rows, out [R, d], lse [R], idx [R, topk], gap [R],
    near_tie [R] (bool).
    """
    T, H, d = Q.shape
    rows = _rows_by_head(rows, T, H)
    R = len(rows)
    out = np.zeros((R, d))
    lse = np.zeros(R)
    idx = np.full((R, topk), -1, dtype=np.int64)
    gap = np.full(R, np.inf)
    near = np.zeros(R, dtype=bool)
    kbar_cache = {}
    for r, (t, h) in enumerate(rows):
        s, a, L = _seq_of_token(cu_seqlens, int(t))
        key = (s, int(h))
        if key not in kbar_cache:
            kbar_cache[key] = pool_keys_head(K[a:a + L, h, :], L, block_size)
        kbar = kbar_cache[key]
        tl = int(t) - a
        c = tl // block_size
        sc = gate_scores_row(Q[t, h, :], kbar, c)
        idx[r], gap[r], near[r] = select_row(sc, c, topk)
        J = attended_tokens(idx[r], tl, block_size)
        out[r], lse[r] = attend_row(Q[t, h, :], K[a:a + L, h, :], V[a:a + L, h, :], J, scale)
    return dict(rows=rows, out=out, lse=lse, idx=idx, gap=gap, near_tie=near)


def select_rows(S, c, topk):
    """Step 3 for many queries that share their own block c: S [R, c] past
    scores.  Same rule as ``select_row`` (a stable descending sort keeps the
    lower block index first among equal scores), vectorised over rows.
    Returns (idx [R, topk], gap [R], near_tie [R])."""
    R = S.shape[0]
    idx = np.full((R, topk), -1, dtype=np.int64)
    take = min(topk - 1, c)
    order = np.argsort(-S, axis=1, kind="stable")
    if take > 0:
        idx[:, :take] = np.sort(order[:, :take], axis=1)
    idx[:, take] = c
    gap = np.full(R, np.inf)
    near = np.zeros(R, dtype=bool)
    if topk >= 2 and c >= topk:
        rr = np.arange(R)
        a = S[rr, order[:, topk - 2]]
        b = S[rr, order[:, topk - 1]]
        gap = a - b
        near = gap < NEAR_TIE_REL * np.maximum(np.abs(a), np.abs(b))
    return idx, gap, near


def gate_reference(Q, K, cu_seqlens, block_size, topk, rows=None):
    """Steps 1-3 only (block selection), vectorised: per sequence and head one
    fp64 product of the queries with the pooled keys, then ``select_rows``
    for each group of queries sharing an own block."""
    T, H, d = Q.shape
    rows = _rows_by_head(rows, T, H)
    R = len(rows)
    idx = np.full((R, topk), -1, dtype=np.int64)
    gap = np.full(R, np.inf)
    near = np.zeros(R, dtype=bool)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    seq_of = np.searchsorted(cu, rows[:, 0], side="right") - 1
    for s in np.unique(seq_of):
        a, L = int(cu[s]), int(cu[s + 1] - cu[s])
        for h in np.unique(rows[seq_of == s, 1]):
            sel = np.nonzero((seq_of == s) & (rows[:, 1] == h))[0]
            kbar = pool_keys_head(K[a:a + L, h, :], L, block_size)
            tl = rows[sel, 0] - a
            cs = tl // block_size
            for c in np.unique(cs):
                g = sel[cs == c]
                S = np.asarray(Q[rows[g, 0], h, :], dtype=np.float64) @ kbar[:c].T
                idx[g], gap[g], near[g] = select_rows(S, int(c), topk)
    return dict(rows=rows, idx=idx, gap=gap, near_tie=near)


def attend_given_selection(Q, K, V, cu_seqlens, block_size, idx, scale, rows):
    """Steps 4-5 for given (token, head) rows and a given selection per row.

    Used for rows whose selection is ambiguous (near-ties): the selection to
    use is checked for validity first by ``selection_is_valid``.
    """
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
    R = len(rows)
    d = Q.shape[2]
    out = np.zeros((R, d))
    lse = np.zeros(R)
    for r, (t, h) in enumerate(rows):
        s, a, L = _seq_of_token(cu_seqlens, int(t))
        J = attended_tokens(idx[r], int(t) - a, block_size)
        out[r], lse[r] = attend_row(Q[t, h, :], K[a:a + L, h, :], V[a:a + L, h, :], J, scale)
    return out, lse


def selection_is_valid(Q, K, cu_seqlens, block_size, topk, row, idx_row,
                       rel=NEAR_TIE_REL):
    """Whether idx_row is a correct causal top-k for (token, head) ``row`` up
    to score differences below ``rel`` relative: ascending, own block last,
    no future block, the right count, and no unselected past block scoring
    higher than a selected one by more than the tolerance."""
    t, h = int(row[0]), int(row[1])
    s, a, L = _seq_of_token(cu_seqlens, t)
    tl = t - a
    c = tl // block_size
    idx_row = [int(x) for x in idx_row]
    valid = [x for x in idx_row if x >= 0]
    if idx_row[len(valid):] != [-1] * (topk - len(valid)):
        return False
    if valid != sorted(set(valid)) or not valid or valid[-1] != c:
        return False
    past = valid[:-1]
    if len(past) != min(topk - 1, c) or any(x < 0 or x >= c for x in past):
        return False
    if not past:
        return True
    kbar = pool_keys_head(K[a:a + L, h, :], L, block_size)
    sc = gate_scores_row(Q[t, h, :], kbar, c)
    worst_in = min(sc[x] for x in past)
    others = [sc[i] for i in range(c) if i not in past]
    if not others:
        return True
    best_out = max(others)
    return bool(best_out - worst_in <= rel * max(abs(best_out), abs(worst_in)))


# --------------------------------------------------------------------------
# backward pass: gradients of the attention over the selected tokens
# --------------------------------------------------------------------------
# [wispaper] "The Change" and [elamur] "Key points": MoBA is trained end to end
# with the block selection made by a hard top-k, so gradients reach q, K and V
# through the softmax attention over the selected tokens only; the selection
# itself is not differentiated.  For one (sequence, head), with M the token
# mask of the selection (step 4), X = scale Q K^T on M (-inf elsewhere),
# P = softmax_rows(X), O = P V and an upstream gradient dO:
#   dV = P^T dO
#   dP = dO V^T
#   dS = P * (dP - rowsum(dO * O))        (softmax Jacobian, elementwise *)
#   dQ = scale dS K,   dK = scale dS^T Q

def token_mask(idx_seq, L, block_size):
    """Token mask of one sequence from its per-token selections idx_seq
    [L, topk]: M[t, j] = j is in a selected block of t and j <= t (step 4)."""
    M = np.zeros((L, L), dtype=bool)
    for t in range(L):
        M[t, attended_tokens(idx_seq[t], t, block_size)] = True
    return M


def attention_backward_masked(Q, K, V, dO, M, scale):
    """Gradients of O = softmax(scale Q K^T on M) V for one head:
    Q, K, V, dO [L, d]; M [L, L] bool with at least one True per row.
    Returns (dQ, dK, dV) fp64."""
    Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dO))
    X = np.where(M, scale * (Q @ K.T), -np.inf)
    mx = X.max(axis=1, keepdims=True)
    W = np.exp(X - mx)
    P = W / W.sum(axis=1, keepdims=True)
    O = P @ V
    dV = P.T @ dO
    dP = dO @ V.T
    Drow = (dO * O).sum(axis=1, keepdims=True)
    dS = P * (dP - Drow)
    return scale * dS @ K, scale * dS.T @ Q, dV


def backward_dq_rows(Q, K, V, dO, cu_seqlens, block_size, idx, scale, rows):
    """dQ of single (token, head) rows, from the row alone: with J the row's
    attended tokens (step 4), p = softmax(scale K[J] q), o = p V[J],
    dp = V[J] dO_t and ds = p * (dp - dO_t . o), dQ_t = scale ds K[J].
    idx: [R, topk] selections of the rows.  Returns [R, d] fp64."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
    out = np.zeros((len(rows), Q.shape[2]))
    for r, (t, h) in enumerate(rows):
        s, a, L = _seq_of_token(cu_seqlens, int(t))
        J = attended_tokens(idx[r], int(t) - a, block_size)
        q = np.asarray(Q[t, h], dtype=np.float64)
        Kj = np.asarray(K[a + J, h], dtype=np.float64)
        Vj = np.asarray(V[a + J, h], dtype=np.float64)
        g = np.asarray(dO[t, h], dtype=np.float64)
        x = scale * (Kj @ q)
        p = np.exp(x - x.max())
        p /= p.sum()
        o = p @ Vj
        ds = p * (Vj @ g - g @ o)
        out[r] = scale * (ds @ Kj)
    return out


def backward_dkdv_keys(Q, K, V, dO, cu_seqlens, block_size, idx, scale, keys):
    """dK, dV of single (key token, head) rows: the sums over every query t
    that attends the key (the own-block queries at or after it, and the later
    queries whose selection lists its block) of scale dS_tj q_t and P_tj dO_t,
    each query's softmax taken over its own attended tokens.  idx [T, H, topk]
    holds every row's selection.  Returns ([R, d], [R, d]) fp64."""
    keys = np.asarray(keys, dtype=np.int64).reshape(-1, 2)
    d = Q.shape[2]
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), d))
    rows_cache = {}

    def row(t, h):  # (p over J, J, o) of query row (t, h)
        if (t, h) not in rows_cache:
            s, a, L = _seq_of_token(cu_seqlens, t)
            J = attended_tokens(idx[t, h], t - a, block_size)
            q = np.asarray(Q[t, h], dtype=np.float64)
            x = scale * (np.asarray(K[a + J, h], dtype=np.float64) @ q)
            p = np.exp(x - x.max())
            p /= p.sum()
            o = p @ np.asarray(V[a + J, h], dtype=np.float64)
            rows_cache[(t, h)] = (p, a + J, o)
        return rows_cache[(t, h)]

    for r, (j, h) in enumerate(keys):
        j, h = int(j), int(h)
        s, a, L = _seq_of_token(cu_seqlens, j)
        b = (j - a) // block_size
        later = np.arange(a + (b + 1) * block_size, a + L)
        sel = later[np.any(idx[later, h] == b, axis=1)] if len(later) else later
        own = np.arange(j, min(a + (b + 1) * block_size, a + L))
        kj = np.asarray(K[j, h], dtype=np.float64)
        vj = np.asarray(V[j, h], dtype=np.float64)
        for t in np.concatenate([own, sel]):
            p, Jg, o = row(int(t), h)
            ptj = p[np.searchsorted(Jg, j)]
            g = np.asarray(dO[t, h], dtype=np.float64)
            dstj = ptj * (g @ vj - g @ o)
            dk[r] += scale * dstj * np.asarray(Q[t, h], dtype=np.float64)
            dv[r] += ptj * g
    return dk, dv


def moba_backward_reference(Q, K, V, dO, cu_seqlens, block_size, idx, scale, heads=None):
    """dQ, dK, dV [T, H, d] fp64 of the attention over the given selections
    idx [T, H, topk] (the heads listed, default all; other heads are zero)."""
    T, H, d = Q.shape
    dQ, dK, dV = (np.zeros((T, H, d)) for _ in range(3))
    for h in (range(H) if heads is None else heads):
        for a, L in sequences(cu_seqlens):
            if L == 0:
                continue
            M = token_mask(idx[a:a + L, h], L, block_size)
            g = attention_backward_masked(Q[a:a + L, h], K[a:a + L, h], V[a:a + L, h],
                                          dO[a:a + L, h], M, scale)
            dQ[a:a + L, h], dK[a:a + L, h], dV[a:a + L, h] = g
    return dQ, dK, dV


# --------------------------------------------------------------------------
# min/max pooled gate (the Quest-style variant)
# --------------------------------------------------------------------------
# [elamur] "Key points" (related methods): Quest reads as MoBA with smaller
# blocks and min/max pooling.  Read here as: each block keeps the elementwise
# maximum and minimum of its keys, and a query scores the block by the largest
# value q . x can take over the box [kmin, kmax] of the block, which is
# sum_e max(q_e kmin_e, q_e kmax_e), an upper bound of q . k for every key k
# of the block.  Selection and attention are those of MoBA.

def pool_minmax_head(K, length, block_size):
    """Elementwise max and min of each block's keys (one head): K [L, d] ->
    (kmax [n, d], kmin [n, d]) fp64."""
    n = num_blocks(length, block_size)
    d = K.shape[1]
    kmax = np.zeros((n, d))
    kmin = np.zeros((n, d))
    for i in range(n):
        lo, hi = block_range(i, length, block_size)
        blk = np.asarray(K[lo:hi], dtype=np.float64)
        kmax[i] = blk.max(axis=0)
        kmin[i] = blk.min(axis=0)
    return kmax, kmin


def minmax_scores_row(q, kmax, kmin, c):
    """Upper-bound affinity of q with every past block i < c:
    sum over e of max(q_e kmin_e, q_e kmax_e)."""
    q = np.asarray(q, dtype=np.float64)
    return np.maximum(q * kmin[:c], q * kmax[:c]).sum(axis=1)


def pool_minmax(K, cu_seqlens, block_size):
    """``pool_minmax_head`` over a packed batch: K [T, H, d] -> kmm [NB, H, 2, d]
    with kmm[:, :, 0] the block maxima and kmm[:, :, 1] the minima."""
    T, H, d = K.shape
    out = []
    for a, L in sequences(cu_seqlens):
        n = num_blocks(L, block_size)
        kb = np.zeros((n, H, 2, d))
        for h in range(H):
            kb[:, h, 0], kb[:, h, 1] = pool_minmax_head(K[a:a + L, h, :], L, block_size)
        out.append(kb)
    return np.concatenate(out, axis=0) if out else np.zeros((0, H, 2, d))


def minmax_gate_reference(Q, K, cu_seqlens, block_size, topk, rows=None):
    """Block selection with the min/max pooled gate on (token, head) rows:
    the scores of ``minmax_scores_row``, then the MoBA selection rule
    (``select_rows``).  Returns dict(rows, idx, gap, near_tie)."""
    T, H, d = Q.shape
    rows = _rows_by_head(rows, T, H)
    R = len(rows)
    idx = np.full((R, topk), -1, dtype=np.int64)
    gap = np.full(R, np.inf)
    near = np.zeros(R, dtype=bool)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    seq_of = np.searchsorted(cu, rows[:, 0], side="right") - 1
    for s in np.unique(seq_of):
        a, L = int(cu[s]), int(cu[s + 1] - cu[s])
        for h in np.unique(rows[seq_of == s, 1]):
            sel = np.nonzero((seq_of == s) & (rows[:, 1] == h))[0]
            kmax, kmin = pool_minmax_head(K[a:a + L, h, :], L, block_size)
            cs = (rows[sel, 0] - a) // block_size
            for c in np.unique(cs):
                g = sel[cs == c]
                S = np.stack([minmax_scores_row(Q[t, h, :], kmax, kmin, int(c))
                              for t in rows[g, 0]]) if c > 0 else np.zeros((len(g), 0))
                idx[g], gap[g], near[g] = select_rows(S, int(c), topk)
    return dict(rows=rows, idx=idx, gap=gap, near_tie=near)


def minmax_selection_is_valid(Q, K, cu_seqlens, block_size, topk, row, idx_row,
                              rel=NEAR_TIE_REL):
    """``selection_is_valid`` with the min/max pooled scores."""
    t, h = int(row[0]), int(row[1])
    s, a, L = _seq_of_token(cu_seqlens, t)
    c = (t - a) // block_size
    idx_row = [int(x) for x in idx_row]
    valid = [x for x in idx_row if x >= 0]
    if idx_row[len(valid):] != [-1] * (topk - len(valid)):
        return False
    if valid != sorted(set(valid)) or not valid or valid[-1] != c:
        return False
    past = valid[:-1]
    if len(past) != min(topk - 1, c) or any(x < 0 or x >= c for x in past):
        return False
    if not past:
        return True
    kmax, kmin = pool_minmax_head(K[a:a + L, h, :], L, block_size)
    sc = minmax_scores_row(Q[t, h, :], kmax, kmin, c)
    worst_in = min(sc[x] for x in past)
    others = [sc[i] for i in range(c) if i not in past]
    if not others:
        return True
    best_out = max(others)
    return bool(best_out - worst_in <= rel * max(abs(best_out), abs(worst_in)))


# --------------------------------------------------------------------------
# static gates: fixed routing rules run through the same attention
# --------------------------------------------------------------------------

def static_select_row(c, topk, sink):
    """Static routing for a query whose own block is c.

    [wispaper] "Why the Change Is Plausible" (first paragraph) and
    [cn-summary] 与其他方法的关系: sliding-window attention is a gate that
    always picks the most recent blocks, attention-sink attention one that
    always picks the initial blocks plus the recent ones, and full attention
    the degenerate gate with k = n.  Read here as one rule with the same
    causality as the learned gate (own block always taken and counted in k,
    never a future block):

    1. take the own block c;
    2. take the initial blocks 0, 1, ... while fewer than ``sink`` of them are
       taken, a past block is left and fewer than k blocks are taken;
    3. walk back from c - 1 over the past blocks not yet taken, taking each
       while fewer than k blocks are taken.

    sink = 0 is a sliding window of k blocks; topk >= c + 1 takes every block
    0..c (full causal attention).  Returns idx [topk] int64 ascending, -1
    padded.
    """
    taken = [c]
    i = 0
    while i < sink and i < c and len(taken) < topk:
        taken.append(i)
        i += 1
    j = c - 1
    while j >= 0 and len(taken) < topk:
        if j not in taken:
            taken.append(j)
        j -= 1
    idx = np.full(topk, -1, dtype=np.int64)
    chosen = sorted(taken)
    idx[:len(chosen)] = chosen
    return idx


def static_reference(Q, K, V, cu_seqlens, block_size, topk, sink, scale, rows=None):
    """Attention with the static routing of ``static_select_row`` on (token,
    head) rows: steps 4-5 over the statically chosen blocks.  Returns dict with
    rows, out [R, d], lse [R], idx [R, topk]."""
    T, H, d = Q.shape
    rows = _rows_by_head(rows, T, H)
    R = len(rows)
    out = np.zeros((R, d))
    lse = np.zeros(R)
    idx = np.full((R, topk), -1, dtype=np.int64)
    for r, (t, h) in enumerate(rows):
        s, a, L = _seq_of_token(cu_seqlens, int(t))
        tl = int(t) - a
        idx[r] = static_select_row(tl // block_size, topk, sink)
        J = attended_tokens(idx[r], tl, block_size)
        out[r], lse[r] = attend_row(Q[t, h, :], K[a:a + L, h, :], V[a:a + L, h, :], J, scale)
    return dict(rows=rows, out=out, lse=lse, idx=idx)


def static_select(cu_seqlens, block_size, topk, sink):
    """``static_select_row`` for every token of a packed batch: idx [T, topk]
    (the rule does not depend on the head)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    idx = np.full((T, topk), -1, dtype=np.int64)
    for a, L in sequences(cu):
        for c in range(num_blocks(L, block_size)):
            row = static_select_row(c, topk, sink)
            idx[a + c * block_size:a + min((c + 1) * block_size, L)] = row
    return idx


# --------------------------------------------------------------------------
# second, independent formulation and the dense baseline
# --------------------------------------------------------------------------

def brute_force_mask(cu_seqlens, block_size, idx):
    """Token-level mask M[t, j] = [block(j) selected by t] and [j <= t] and
    [same sequence], built from per-row selections idx [T, topk] (one head).

    [glossary] "Mathematical and complexity implications": the learned block
    mask over the N x N score matrix.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    M = np.zeros((T, T), dtype=bool)
    for a, L in sequences(cu):
        for tl in range(L):
            sel = {int(x) for x in idx[a + tl] if x >= 0}
            for jl in range(tl + 1):
                if jl // block_size in sel:
                    M[a + tl, a + jl] = True
    return M


def masked_softmax_attention(Q, K, V, M, scale):
    """Dense softmax over the allowed positions of mask M (one head):
    Q, K, V [T, d]; returns out [T, d], lse [T]."""
    X = scale * (np.asarray(Q, np.float64) @ np.asarray(K, np.float64).T)
    X = np.where(M, X, -np.inf)
    mx = X.max(axis=1, keepdims=True)
    W = np.exp(X - mx)
    den = W.sum(axis=1, keepdims=True)
    out = (W / den) @ np.asarray(V, np.float64)
    lse = (mx + np.log(den))[:, 0]
    return out, lse


def dense_causal_reference(Q, K, V, cu_seqlens, scale, rows=None):
    """Full causal softmax attention per sequence (the exact baseline of
    [wispaper] "Starting Point"), on (token, head) rows."""
    T, H, d = Q.shape
    rows = _rows_by_head(rows, T, H)
    out = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for r, (t, h) in enumerate(rows):
        s, a, L = _seq_of_token(cu_seqlens, int(t))
        J = np.arange(0, int(t) - a + 1)
        out[r], lse[r] = attend_row(Q[t, h, :], K[a:a + L, h, :], V[a:a + L, h, :], J, scale)
    return out, lse


def sparsity(seq_len, block_size, topk, seed=0):
    """Fraction of the seq_len positions that the last query of a sequence
    does not attend to, through the oracle's own selection on random scores
    ([wispaper] "The Change", the sparsity paragraph: 1 - k*B/N when N is a
    multiple of B; the count does not depend on which blocks win)."""
    last = seq_len - 1
    c = last // block_size
    scores = np.random.default_rng(seed).standard_normal(c)
    idx, _, _ = select_row(scores, c, topk)
    J = attended_tokens(idx, last, block_size)
    return 1.0 - len(J) / seq_len
