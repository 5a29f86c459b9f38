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
    kbar = moba.moba_pool_keys(x["k"], geom).cpu().numpy()
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
    _say("gate 32k (4 heads, all rows)")
    x = inputs.make_inputs(w, device=dev)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    idx = moba.moba_gate_topk(x["q"], moba.moba_pool_keys(x["k"], geom), geom, w.topk)
    st = parity.check_idx_all_rows(x["q"], x["k"], x["cu_seqlens"], w.block_size, w.topk, idx,
                                   heads=[0, 7, 19, 31])
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


@pytest.mark.parametrize("name,per_head,heads", [
    ("32k", 128, [0, 5, 31]),
    ("varlen", 96, [0, 17]),
])
def test_moba_sampled(dev, name, per_head, heads):
    w = inputs.WORKLOADS[name]
    x, geom, out, lse, idx = _run(w, dev)
    rows = inputs.sample_rows(w, per_head, heads=heads)
    st = parity.check_moba_rows(x["q"], x["k"], x["v"], x["cu_seqlens"], w.block_size, w.topk,
                                w.scale, out, lse, idx, rows, parity.BF16_TOL)
    print(name, st)


def test_moba_1m_sampled(dev):
    """The 1M-token workload in the launch configuration bench.py times:
    outputs on 512 seeded rows (4 heads), selections on every row of one
    head, and causal validity of every selection row."""
    w = inputs.WORKLOADS["1m"]
    x, geom, out, lse, idx = _run(w, dev)
    rows = inputs.sample_rows(w, 128, heads=[0, 3, 17, 28])
    st = parity.check_moba_rows(x["q"], x["k"], x["v"], x["cu_seqlens"], w.block_size, w.topk,
                                w.scale, out, lse, idx, rows, parity.BF16_TOL)
    print("1m", st)
    st = parity.check_idx_all_rows(x["q"], x["k"], x["cu_seqlens"], w.block_size, w.topk, idx,
                                   heads=[5])
    print("1m head 5 selections", st)
    _check_rows_valid(w, idx, out, lse)


def test_moba_10m_sampled(dev):
    """Constant sparsity at 10M tokens (B 40960 keeps the 1M workload's 256
    blocks), one GPU's 4-head share: outputs and selections on 64 seeded
    rows of two heads, causal validity of every selection row."""
    w = inputs.WORKLOADS["10m"]
    x, geom, out, lse, idx = _run(w, dev)
    rows = inputs.sample_rows(w, 32, heads=[0, 3])
    st = parity.check_moba_rows(x["q"], x["k"], x["v"], x["cu_seqlens"], w.block_size, w.topk,
                                w.scale, out, lse, idx, rows, parity.BF16_TOL)
    print("10m", st)
    _check_rows_valid(w, idx, out, lse)
    del x, out, lse, idx
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


def test_bucket_lists_rebuild_selection(dev):
    """The per-block query lists hold exactly the historical selections."""
    w = inputs.custom([3000, 1100], 2, 128, 128, 5, "bf16", name="lists")
    x = inputs.make_inputs(w, device=dev, seed=4)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    out, lse, idx = moba.forward(x["q"], x["k"], x["v"], geom, w.topk, w.scale)
    ws = torch.empty(moba.moba_attn_workspace_bytes(moba.MOBA_BF16, geom.total_tokens,
                                                    geom.total_blocks, w.heads, 128, 128, 5),
                     dtype=torch.uint8, device=dev)
    moba.moba_attn_fwd(x["q"], x["k"], x["v"], geom, w.topk, idx, w.scale, workspace=ws)
    torch.cuda.synchronize()
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
            for slot, b in enumerate(row):
                want.add((t, h, slot, int(cb[s] + b)))
    assert got == want
    assert len(lst) == len(want)
