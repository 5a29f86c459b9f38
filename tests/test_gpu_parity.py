"""Parity of the HIP library (through its C ABI) with the CPU oracle on MI355X.

Every case prints its name, shape and seed before it touches the GPU.
"""

import sys

import numpy as np
import pytest
import torch

from block_sparse_long_03_amd import inputs, moba
from oracle import moba_oracle as mo
from tests import parity

import bench  # list lengths of a selection (measurement helper)

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _run(w, dev, seed=None, out_dtype=None):
    _say(w.name, w.seqlens[:6], "H", w.heads, "d", w.head_dim, "B", w.block_size, "k", w.topk,
         w.dtype, "seed", seed)
    x = inputs.make_inputs(w, device=dev, seed=seed)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    out, lse, idx = moba.forward(x["q"], x["k"], x["v"], geom, w.topk, w.scale,
                                 out_dtype=out_dtype)
    torch.cuda.synchronize()
    return x, geom, out, lse, idx


# ---------------------------------------------------------------------------
# step by step
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("w", [
    inputs.WORKLOADS["tiny"],
    inputs.custom([700, 0, 129, 64, 1, 300], 3, 128, 64, 4, "bf16", name="ragged-bf16"),
    inputs.custom([333, 64, 200], 2, 64, 128, 3, "f32", name="ragged-f32-d64"),
])
def test_pool_keys(dev, w):
    _say("pool", w.name)
    x = inputs.make_inputs(w, device=dev)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    pooled = moba.moba_pool_keys(x["k"], geom)
    kbar = pooled.kbar.cpu().numpy()
    # the three bf16 terms add up to the fp32 means exactly, hi being the
    # upper half of the fp32 pattern
    NB, H, d = pooled.kbar.shape
    k3 = moba.kbar3_terms(pooled.kbar3, H, d, NB).float()
    assert torch.equal((k3[:, :, 0] + k3[:, :, 1]) + k3[:, :, 2], pooled.kbar)
    bits = pooled.kbar.contiguous().view(torch.int32)
    assert torch.equal(k3[:, :, 0].contiguous().view(torch.int32), bits & -65536)
    ref = mo.pool_keys(x["k"].float().cpu().numpy(), x["cu_seqlens"], w.block_size)
    assert kbar.shape == ref.shape
    np.testing.assert_allclose(kbar, ref, rtol=0, atol=2e-6 * max(1.0, np.abs(ref).max()))


@pytest.mark.parametrize("name", ["tiny", "8k"])
def test_gate_topk_all_rows(dev, name):
    w = inputs.WORKLOADS[name]
    _say("gate", name)
    x = inputs.make_inputs(w, device=dev)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    kbar = moba.moba_pool_keys(x["k"], geom)
    idx = moba.moba_gate_topk(x["q"], kbar, geom, w.topk)
    st = parity.check_idx_all_rows(x["q"], x["k"], x["cu_seqlens"], w.block_size, w.topk, idx)
    print(name, st)


def test_gate_topk_32k_fine_grained(dev):
    w = inputs.WORKLOADS["32k"]
    _say("gate 32k (all heads, all rows)")
    x = inputs.make_inputs(w, device=dev)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    idx = moba.moba_gate_topk(x["q"], moba.moba_pool_keys(x["k"], geom), geom, w.topk)
    st = parity.check_idx_all_rows(x["q"], x["k"], x["cu_seqlens"], w.block_size, w.topk, idx)
    print("32k", st)


@pytest.mark.parametrize("w", [
    # more than 256 past blocks: the selection runs over two spans and merges
    # the first span's kept set; k - 1 = 4 (sorted-list threshold) and 20
    # (radix threshold); ragged second sequence, d 64 and 128
    inputs.custom([300 * 64 + 5, 700], 2, 128, 64, 5, "bf16", name="gate-2span-k5"),
    inputs.custom([290 * 64], 2, 64, 64, 21, "bf16", name="gate-2span-k21"),
    # k - 1 = 16: the largest k of the sorted-list threshold
    inputs.custom([64 * 40 + 17], 3, 128, 64, 17, "bf16", name="gate-k17"),
], ids=lambda w: w.name)
def test_gate_topk_spans(dev, w):
    _say("gate", w.name)
    x = inputs.make_inputs(w, device=dev, seed=5)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    idx = moba.moba_gate_topk(x["q"], moba.moba_pool_keys(x["k"], geom), geom, w.topk)
    st = parity.check_idx_all_rows(x["q"], x["k"], x["cu_seqlens"], w.block_size, w.topk, idx)
    print(w.name, st)


@pytest.mark.parametrize("k", [4, 12, 21, 33])
def test_gate_topk_exact_ties(dev, k):
    """Exact ties: in each sequence, blocks 2, 5, 9, ... repeat the keys of
    block 1 (equal pooled keys, so bitwise equal scores), and every third
    query is zero (all its scores are 0: every past block ties, more
    candidates than the candidate selection takes, so those waves select row
    by row).  The lower block index wins every tie: on rows whose boundary
    is an exact tie the selection must equal the oracle's; other rows follow
    the usual near-tie rule."""
    B = 64
    w = inputs.custom([B * 40 + 17, B * 20, B * 300 + 3], 2, 128, B, k, "bf16",
                      name=f"gate-ties-k{k}")
    _say("gate ties", w.seqlens, "k", k)
    x = inputs.make_inputs(w, device=dev, seed=9)
    cu = x["cu_seqlens"]
    for s in range(len(w.seqlens)):
        a, L = cu[s], cu[s + 1] - cu[s]
        for b in (2, 5, 9, 13, 17, 21, 29, 33, 100, 257, 290):
            if (b + 1) * B <= L:
                x["k"][a + b * B:a + (b + 1) * B] = x["k"][a + B:a + 2 * B]
    x["q"][0::3] = 0
    geom = moba.Geometry.make(cu, B, dev)
    idx = moba.moba_gate_topk(x["q"], moba.moba_pool_keys(x["k"], geom), geom, k)
    torch.cuda.synchronize()
    qn, kn = x["q"].float().cpu().numpy(), x["k"].float().cpu().numpy()
    ref = mo.gate_reference(qn, kn, cu, B, k)
    rows = ref["rows"]
    gi = idx.cpu().numpy()[rows[:, 0], rows[:, 1]].astype(np.int64)
    exact = ref["gap"] == 0
    assert exact.sum() > 1000
    assert np.array_equal(gi[exact], ref["idx"][exact])
    st = parity.check_idx_all_rows(x["q"], x["k"], cu, B, k, idx)
    print(w.name, "exact-tie rows", int(exact.sum()), st)


# ---------------------------------------------------------------------------
# the whole forward
# ---------------------------------------------------------------------------

def test_moba_tiny_fp32_all_rows(dev):
    w = inputs.WORKLOADS["tiny"]
    x, geom, out, lse, idx = _run(w, dev)
    rows = np.stack(np.meshgrid(np.arange(w.total_tokens), np.arange(w.heads), indexing="ij"),
                    -1).reshape(-1, 2)
    st = parity.check_moba_rows(x["q"], x["k"], x["v"], x["cu_seqlens"], w.block_size, w.topk,
                                w.scale, out, lse, idx, rows, parity.F32_TOL)
    print("tiny", st)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_moba_8k(dev, out_dtype):
    w = inputs.WORKLOADS["8k"]
    x, geom, out, lse, idx = _run(w, dev, out_dtype=out_dtype)
    st = parity.check_idx_all_rows(x["q"], x["k"], x["cu_seqlens"], w.block_size, w.topk, idx)
    rows = inputs.sample_rows(w, 512)
    st2 = parity.check_moba_rows(x["q"], x["k"], x["v"], x["cu_seqlens"], w.block_size, w.topk,
                                 w.scale, out, lse, idx, rows, parity.BF16_TOL)
    print("8k", out_dtype, st, st2)


@pytest.mark.parametrize("name,per_head,heads,sel_heads", [
    ("32k", 512, [0, 5, 11, 19, 26, 31], []),
    ("varlen", 512, [0, 9, 17, 30], list(range(32))),
])
def test_moba_sampled(dev, name, per_head, heads, sel_heads):
    """Outputs of seeded rows (per_head per listed head) against the oracle
    on the selection the oracle confirms, and (sel_heads) the selections of
    every row of further heads."""
    w = inputs.WORKLOADS[name]
    x, geom, out, lse, idx = _run(w, dev)
    rows = inputs.sample_rows(w, per_head, heads=heads)
    st = parity.check_moba_rows(x["q"], x["k"], x["v"], x["cu_seqlens"], w.block_size, w.topk,
                                w.scale, out, lse, idx, rows, parity.BF16_TOL)
    print(name, st)
    if sel_heads:
        st = parity.check_idx_all_rows(x["q"], x["k"], x["cu_seqlens"], w.block_size, w.topk,
                                       idx, heads=sel_heads)
        print(name, "selections of heads", sel_heads, st)


def test_moba_1m_sampled(dev):
    """The 1M-token workload in the launch configuration bench.py times:
    outputs on 2048 seeded rows (8 heads), selections on every row of two
    heads and on 4096 seeded rows of every head, and causal validity of
    every selection row; then the same attention in passes of 8 heads,
    which must reproduce it bit for bit."""
    w = inputs.WORKLOADS["1m"]
    x, geom, out, lse, idx = _run(w, dev)
    rows = inputs.sample_rows(w, 256, heads=[0, 3, 9, 14, 17, 22, 28, 31])
    st = parity.check_moba_rows(x["q"], x["k"], x["v"], x["cu_seqlens"], w.block_size, w.topk,
                                w.scale, out, lse, idx, rows, parity.BF16_TOL)
    print("1m", st)
    st = parity.check_idx_all_rows(x["q"], x["k"], x["cu_seqlens"], w.block_size, w.topk, idx,
                                   heads=[5, 26])
    print("1m heads 5, 26 selections", st)
    _say("1m: selections of 4096 seeded rows of every head")
    st = parity.check_idx_rows(x["q"], x["k"], x["cu_seqlens"], w.block_size, w.topk, idx,
                               inputs.sample_rows(w, 4096))
    print("1m 4096 rows x 32 heads selections", st)
    _check_rows_valid(w, idx, out, lse)
    _say("1m: attention again in passes of 8 heads")
    torch.cuda.empty_cache()
    out2, lse2 = moba.moba_attn_fwd(x["q"], x["k"], x["v"], geom, w.topk, idx, w.scale,
                                    head_chunk=8)
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(lse2, lse)


def test_moba_10m_streamed(dev):
    """Constant sparsity at 10M tokens (B 40960 keeps the 1M workload's 256
    blocks) with all 32 heads on one GPU, streamed group by group
    (forward_head_streamed, groups of 4 heads in passes of 2): the first
    and the last of the 8 head groups run; outputs and selections on 48
    seeded rows of four heads in them, causal validity of every selection
    row of both groups."""
    w = inputs.WORKLOADS["10m32"]
    _say(w.name, "groups 0 and 7 of", w.heads // w.head_group, "B", w.block_size, "k", w.topk)
    geom = moba.Geometry.make(inputs.cu_seqlens_of(w.seqlens), w.block_size, dev)
    check_heads = {0: [1, 3], 7: [28, 31]}

    def source(h0, h1):
        _say(w.name, "heads", h0, "..", h1 - 1)
        x = inputs.make_head_group(w, h0 // w.head_group, device=dev)
        return x["q"], x["k"], x["v"]

    def on_group(h0, out, lse, idx):
        torch.cuda.synchronize()
        g = h0 // w.head_group
        wg = inputs.custom(w.seqlens, out.shape[1], w.head_dim, w.block_size, w.topk, w.dtype)
        _check_rows_valid(wg, idx, out, lse)
        x = inputs.make_head_group(w, g, device=dev)  # the same draw again
        hs = [h - h0 for h in check_heads[g]]
        rows = inputs.sample_rows(w, 24, heads=hs)
        st = parity.check_moba_rows(x["q"], x["k"], x["v"], inputs.cu_seqlens_of(w.seqlens),
                                    w.block_size, w.topk, w.scale, out, lse, idx, rows,
                                    parity.BF16_TOL)
        print("10m32 group", g, st)
        del x

    moba.forward_head_streamed(source, geom, w.heads, w.head_group, w.topk, w.scale,
                               head_chunk=2, groups=[0, 7], on_group=on_group)
    torch.cuda.empty_cache()


def _check_rows_valid(w, idx, out, lse):
    """Every row: ascending past blocks, then the own block, then -1 padding,
    min(k, c + 1) entries; finite outputs (one sequence)."""
    T, H, k = idx.shape
    c = (torch.arange(T, device=idx.device) // w.block_size).view(T, 1, 1)
    valid = idx >= 0
    n = valid.sum(-1, keepdim=True)
    assert torch.equal(n, torch.clamp(c, max=k - 1).expand(T, H, 1) + 1)
    pos = torch.arange(k, device=idx.device).view(1, 1, k)
    assert bool((valid == (pos < n)).all())
    own = torch.gather(idx, 2, n - 1)
    assert torch.equal(own, c.expand(T, H, 1))
    past = torch.where(pos < n - 1, idx, torch.full_like(idx, -1))
    assert bool(((past < c) | (past == -1)).all())
    inc = past[..., 1:] > past[..., :-1]
    assert bool((inc | (past[..., 1:] == -1)).all())
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(lse).all())


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

EDGE = [
    # ragged tails, an empty sequence, a 1-token sequence, sequences shorter than B
    inputs.custom([700, 0, 129, 1, 64, 300], 3, 128, 64, 4, "bf16", name="ragged-B64"),
    # k larger than every sequence's block count: MoBA == dense causal
    inputs.custom([520, 1000], 2, 128, 128, 16, "bf16", name="k>n"),
    # k = 1: own block only
    inputs.custom([1024, 777], 2, 128, 256, 1, "bf16", name="k1"),
    # d = 64, maximum topk
    inputs.custom([64 * 70 + 13], 2, 64, 64, 64, "bf16", name="d64-k64"),
    # fp32 with ragged tails and d = 128
    inputs.custom([300, 77, 512], 2, 128, 64, 3, "f32", name="f32-ragged"),
    # block size >= 1024: 256-query historical tiles (8 waves), ragged tails
    inputs.custom([3000, 2100, 700], 2, 128, 1024, 3, "bf16", name="B1024-ragged"),
    inputs.custom([4100], 2, 64, 1024, 3, "bf16", name="d64-B1024"),
    # whole KV block resident in LDS: lists longer than one 4096-query tile,
    # each tile run as up to 16 passes per wave; d = 64 at the largest
    # resident B
    inputs.custom([12000, 2500], 2, 128, 256, 12, "bf16", name="B256-resident-multitile"),
    inputs.custom([5000, 1500], 2, 64, 512, 4, "bf16", name="d64-B512-resident"),
]


@pytest.mark.parametrize("w", EDGE, ids=[w.name for w in EDGE])
def test_moba_edge_cases(dev, w):
    x, geom, out, lse, idx = _run(w, dev, seed=77, out_dtype=torch.float32)
    if w.name == "B256-resident-multitile":
        # the case must reach a list longer than one resident tile
        lengths = bench.list_lengths(torch, idx, w.seqlens, w.block_size)
        assert lengths.max() > 4096, lengths.max()
    T = w.total_tokens
    rows = np.stack(np.meshgrid(np.arange(T), np.arange(w.heads), indexing="ij"), -1).reshape(-1, 2)
    if len(rows) > 3000:
        rows = rows[np.random.default_rng(5).choice(len(rows), 3000, replace=False)]
        rows = rows[np.lexsort((rows[:, 0], rows[:, 1]))]
    tol = parity.F32_TOL if w.dtype == "f32" else parity.BF16_TOL
    st = parity.check_moba_rows(x["q"], x["k"], x["v"], x["cu_seqlens"], w.block_size, w.topk,
                                w.scale, out, lse, idx, rows, tol)
    print(w.name, st)


def _stages(fn):
    """Names of the library stages that fn() launches."""
    prof = moba.Profiler().attach()
    try:
        prof.reset()
        fn()
        torch.cuda.synchronize()
        return set(prof.names())
    finally:
        prof.detach()
        prof.close()


@pytest.mark.parametrize("w", [
    # 6 query tiles of 128 x 3 sequences x 16 heads: a dense-prefix launch of
    # 288 workgroups
    inputs.custom([3000, 1700, 600], 16, 128, 128, 6, "bf16", name="prefix-B128-k6"),
    # 12 tiles of 256 x 2 sequences x 12 heads
    inputs.custom([5000, 2100], 12, 64, 1024, 3, "bf16", name="prefix-d64-B1024-k3"),
], ids=lambda w: w.name)
def test_prefix_rows_missing_blocks(dev, w):
    """Rows of the first k blocks normally select every earlier block and are
    computed as dense causal rows.  Here a given selection drops one past
    block from some of them (odd rows of blocks 2 and 4 of each sequence,
    every row of block 1 of the first sequence), so blocks hold both kinds
    of rows.  Every prefix row and a sample of the others, on three heads,
    are checked against the oracle on the selection actually passed, and a
    run in passes of 4 heads (the per-block flags indexed by the head's place
    in its pass) must reproduce it bit for bit."""
    _say(w.name, w.seqlens, "H", w.heads, "d", w.head_dim, "B", w.block_size, "k", w.topk)
    x = inputs.make_inputs(w, device=dev, seed=31)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    _, _, idx = moba.forward(x["q"], x["k"], x["v"], geom, w.topk, w.scale)
    torch.cuda.synchronize()
    sel = idx.cpu().numpy().copy()
    cu = x["cu_seqlens"]
    rng = np.random.default_rng(8)
    changed = 0
    for s in range(len(w.seqlens)):
        a, L = cu[s], cu[s + 1] - cu[s]
        for p in range(min(L, w.topk * w.block_size)):
            c = p // w.block_size
            drop = (c in (2, 4) and p % 2 == 1) or (s == 0 and c == 1)
            if c == 0 or not drop:
                continue
            for h in range(w.heads):
                row = [e for e in sel[a + p, h] if e >= 0]
                assert row == list(range(c + 1)), row  # full prefix from the gate
                del row[int(rng.integers(0, c))]
                sel[a + p, h] = row + [-1] * (w.topk - len(row))
                changed += 1
    assert changed > 0
    block_idx = torch.as_tensor(sel, device=dev)
    res = {}

    def run(chunk):
        res[chunk] = moba.moba_attn_fwd(x["q"], x["k"], x["v"], geom, w.topk, block_idx,
                                        w.scale, out_dtype=torch.float32, head_chunk=chunk)

    assert "attn_prefix" in _stages(lambda: run(0))
    assert "attn_prefix" in _stages(lambda: run(4))
    out, lse = res[0]
    prefix = [cu[s] + p for s in range(len(w.seqlens))
              for p in range(min(cu[s + 1] - cu[s], w.topk * w.block_size))]
    rest = np.setdiff1d(np.arange(w.total_tokens), prefix)
    rest = rng.choice(rest, min(len(rest), 400), replace=False)
    toks = np.sort(np.concatenate([np.asarray(prefix, dtype=np.int64), rest]))
    stats = []
    for h in (0, w.heads // 2, w.heads - 1):
        rows_h = np.stack([toks, np.zeros_like(toks)], axis=1)
        o_ref, l_ref = mo.attend_given_selection(
            parity.host_head(x["q"], h), parity.host_head(x["k"], h), parity.host_head(x["v"], h),
            cu, w.block_size, sel[toks, h].astype(np.int64), w.scale, rows_h)
        tt = torch.as_tensor(toks, device=dev)
        st = parity.error_stats(out[tt, h].cpu().numpy(), o_ref, lse[tt, h].cpu().numpy(), l_ref)
        parity.assert_within(st, parity.BF16_TOL, f"{w.name} head {h}")
        stats.append(st)
    o4, l4 = res[4]
    assert torch.equal(out, o4) and torch.equal(lse, l4)
    print(w.name, "changed rows", changed, stats)


def test_moba_peaky_softmax(dev):
    """Sharp attention (queries scaled by 4, scores of std ~4): a few keys
    dominate each softmax, the regime where rounding of the probabilities
    shows most in the output and the log-sum-exp."""
    w = inputs.custom([2048, 900], 2, 128, 128, 4, "bf16", name="peaky")
    _say(w.name)
    x = inputs.make_inputs(w, device=dev, seed=21)
    x["q"].mul_(4)  # exact in bf16
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    out, lse, idx = moba.forward(x["q"], x["k"], x["v"], geom, w.topk, w.scale,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.stack(np.meshgrid(np.arange(0, w.total_tokens, 3), np.arange(w.heads),
                                indexing="ij"), -1).reshape(-1, 2)
    st = parity.check_moba_rows(x["q"], x["k"], x["v"], x["cu_seqlens"], w.block_size, w.topk,
                                w.scale, out, lse, idx, rows, parity.BF16_TOL)
    print("peaky", st)


def test_k_ge_n_matches_own_dense_kernel(dev):
    # the longest sequence reaches 1024 tokens: the dense kernel runs 8 waves
    w = inputs.custom([520, 1100], 2, 128, 128, 16, "bf16", name="k>n-vs-dense")
    x, geom, out, lse, idx = _run(w, dev, seed=3, out_dtype=torch.float32)
    o_d, l_d = moba.dense(x["q"], x["k"], x["v"], geom, w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    # both are bf16-MFMA results of the same softmax; they differ only in
    # rounding order and the bf16 rounding of the partials
    assert (out - o_d).abs().max().item() < 1e-2
    assert (lse - l_d).abs().max().item() < 1e-4


@pytest.mark.parametrize("w", [
    inputs.custom([1000, 0, 64, 2000], 2, 128, 128, 2, "bf16", name="dense-varlen"),
    # 8-wave tiles (a 2000-token sequence in the batch) over sequences of 1,
    # 2 and 3 key chunks: the four-slot ring's short tails
    inputs.custom([2000, 100, 150, 40], 2, 128, 128, 2, "bf16", name="dense-ring-tails"),
    inputs.custom([900, 35], 2, 64, 64, 2, "bf16", name="dense-d64"),
    inputs.custom([1500, 35], 2, 64, 64, 2, "bf16", name="dense-d64-long"),
    inputs.custom([300, 129], 2, 128, 64, 2, "f32", name="dense-f32"),
], ids=lambda w: w.name)
def test_dense_causal(dev, w):
    _say("dense", w.name)
    x = inputs.make_inputs(w, device=dev, seed=11)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    out, lse = moba.dense(x["q"], x["k"], x["v"], geom, w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    T = w.total_tokens
    rows = np.stack(np.meshgrid(np.arange(T), np.arange(w.heads), indexing="ij"), -1).reshape(-1, 2)
    rows = rows[np.random.default_rng(2).choice(len(rows), min(len(rows), 1500), replace=False)]
    o_ref, l_ref = mo.dense_causal_reference(x["q"].float().cpu().numpy(),
                                             x["k"].float().cpu().numpy(),
                                             x["v"].float().cpu().numpy(), x["cu_seqlens"],
                                             w.scale, rows=rows)
    o_g = out[torch.as_tensor(rows[:, 0]), torch.as_tensor(rows[:, 1])].cpu().numpy()
    l_g = lse[torch.as_tensor(rows[:, 0]), torch.as_tensor(rows[:, 1])].cpu().numpy()
    st = parity.error_stats(o_g, o_ref, l_g, l_ref)
    parity.assert_within(st, parity.F32_TOL if w.dtype == "f32" else parity.BF16_TOL, w.name)
    print(w.name, st)


def test_deterministic(dev):
    w = inputs.WORKLOADS["8k"]
    x, geom, out1, lse1, idx1 = _run(w, dev)
    out2, lse2, idx2 = moba.forward(x["q"], x["k"], x["v"], geom, w.topk, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2)
    assert torch.equal(out1, out2)
    assert torch.equal(lse1, lse2)


@pytest.mark.parametrize("heads", [2, 32])
def test_bucket_lists_rebuild_selection(dev, heads):
    """The per-block query lists hold exactly the historical selections.
    With 32 heads the dense-prefix launch fills the chip, so rows of the
    first k blocks that select every earlier block (each such row under the
    gate) are computed by the dense kernel and have no list entries; with 2
    heads that launch would be too small and every row is bucketed."""
    w = inputs.custom([3000, 1100], heads, 128, 128, 5, "bf16", name="lists")
    _say(w.name, w.seqlens, "H", heads, "B", w.block_size, "k", w.topk)
    x = inputs.make_inputs(w, device=dev, seed=4)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    out, lse, idx = moba.forward(x["q"], x["k"], x["v"], geom, w.topk, w.scale)
    ws = torch.empty(moba.moba_attn_workspace_bytes(moba.MOBA_BF16, geom.total_tokens,
                                                    geom.total_blocks, w.heads, 128, 128, 5, 0),
                     dtype=torch.uint8, device=dev)
    prof = moba.Profiler().attach()
    try:
        prof.reset()
        moba.moba_attn_fwd(x["q"], x["k"], x["v"], geom, w.topk, idx, w.scale, workspace=ws)
        torch.cuda.synchronize()
        prefix_route = "attn_prefix" in prof.names()
    finally:
        prof.detach()
        prof.close()
    assert prefix_route == (heads == 32)
    H, NB, k, T = w.heads, geom.total_blocks, w.topk, geom.total_tokens
    al = lambda n: (n + 255) // 256 * 256
    off_counts = 0
    off_offsets = al(H * NB * 4)
    off_tiles = off_offsets + al((H * NB + 1) * 4)
    off_list = off_tiles + al((H * NB + 1) * 4)
    offsets = ws[off_offsets:off_offsets + (H * NB + 1) * 4].view(torch.int32).cpu().numpy()
    lst = ws[off_list:off_list + offsets[-1] * 4].view(torch.int32).cpu().numpy()
    idx_h = idx.cpu().numpy()
    cu = np.array(x["cu_seqlens"])
    cb = np.array(x["cu_blocks"])
    got = set()
    for key in range(H * NB):
        h, gb = divmod(key, NB)
        for e in lst[offsets[key]:offsets[key + 1]]:
            t, slot = divmod(int(e), k)
            got.add((t, h, slot, gb))
    want = set()
    for t in range(T):
        s = int(np.searchsorted(cu, t, side="right") - 1)
        c = (t - cu[s]) // w.block_size
        for h in range(H):
            row = [int(v) for v in idx_h[t, h] if 0 <= v < c]
            if prefix_route and c < k:
                assert row == list(range(c))
                continue
            for slot, b in enumerate(row):
                want.add((t, h, slot, int(cb[s] + b)))
    assert got == want
    assert len(lst) == len(want)
