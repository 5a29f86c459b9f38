"""The min/max pooled gate (Quest read as MoBA with min/max pooling) and the
layer-wise hybrid on MI355X through the C ABI: pooling bit-exact against the
oracle, selections bit-exact except on near-ties (where the GPU's set must be
a valid top-k under the oracle's fp64 scores), and the attention over the
selected blocks within the bf16 tolerances.

Every case prints its name, shape and seed before it touches the GPU.
"""

import sys

import numpy as np
import pytest
import torch

from block_sparse_long_03_amd import inputs, moba
from oracle import moba_oracle as mo
from tests import parity

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


@pytest.mark.parametrize("w", [
    inputs.custom([700, 0, 129, 64, 1, 300], 3, 128, 64, 4, "bf16", name="ragged-bf16"),
    inputs.custom([333, 64, 200], 2, 64, 128, 3, "f32", name="ragged-f32-d64"),
], ids=lambda w: w.name)
def test_pool_minmax(dev, w):
    _say("pool minmax", w.name)
    x = inputs.make_inputs(w, device=dev)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    kmm = moba.moba_pool_minmax(x["k"], geom)
    kmm = moba.kminmax_rows(kmm, w.heads, w.head_dim, geom.total_blocks).cpu().numpy()
    ref = mo.pool_minmax(x["k"].float().cpu().numpy(), x["cu_seqlens"], w.block_size)
    assert kmm.shape == ref.shape
    np.testing.assert_array_equal(kmm, ref)


def _check_minmax_idx(q, k, cu, B, topk, idx, rows):
    """Selections of (token, head) rows against the oracle; returns the
    selection to attend with (the GPU's on validated near-ties)."""
    ref = mo.minmax_gate_reference(q, k, cu, B, topk, rows=rows)
    g = idx[rows[:, 0], rows[:, 1]]
    use = ref["idx"].copy()
    mism = np.nonzero(np.any(ref["idx"] != g, axis=1))[0]
    bad = []
    for r in mism:
        if ref["near_tie"][r] and mo.minmax_selection_is_valid(q, k, cu, B, topk, rows[r], g[r]):
            use[r] = g[r]
        else:
            bad.append(r)
    assert not bad, (f"{len(bad)} rows differ without a near-tie, e.g. {rows[bad[0]].tolist()}: "
                     f"gpu {g[bad[0]].tolist()} oracle {ref['idx'][bad[0]].tolist()}")
    parity.emit(dict(rows=len(rows), near_ties=int(ref["near_tie"].sum()),
                     mismatches=len(mism)))
    return use


@pytest.mark.parametrize("w", [
    inputs.custom([5000, 3192], 4, 128, 512, 4, "bf16", name="minmax-8k"),
    # more than 256 past blocks (two selection spans) and k - 1 above 16
    inputs.custom([300 * 64 + 5, 700], 2, 128, 64, 5, "bf16", name="minmax-2span-k5"),
    inputs.custom([64 * 40 + 17], 3, 64, 64, 21, "bf16", name="minmax-d64-k21"),
], ids=lambda w: w.name)
def test_gate_minmax_all_rows(dev, w):
    _say("gate minmax", w.name, "seed 5")
    x = inputs.make_inputs(w, device=dev, seed=5)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    idx = moba.moba_gate_topk_minmax(x["q"], moba.moba_pool_minmax(x["k"], geom), geom, w.topk)
    idx = idx.cpu().numpy()
    rows = np.stack(np.meshgrid(np.arange(w.total_tokens), np.arange(w.heads), indexing="ij"),
                    -1).reshape(-1, 2)
    _check_minmax_idx(x["q"].float().cpu().numpy(), x["k"].float().cpu().numpy(),
                      x["cu_seqlens"], w.block_size, w.topk, idx, rows)


@pytest.mark.parametrize("w", [
    # one selection span with ragged ends (own blocks not a multiple of 32,
    # a last tile past the sequence end), d 128 and d 64
    inputs.custom([64 * 200 + 37, 1000], 2, 128, 64, 6, "bf16", name="minmax-f32pool-d128"),
    inputs.custom([64 * 90 + 20, 333], 2, 64, 64, 9, "bf16", name="minmax-f32pool-d64"),
], ids=lambda w: w.name)
def test_gate_minmax_fp32_pooled(dev, w):
    # bf16 queries against min/max keys pooled from fp32 keys that are not
    # bf16 values: the gate splits each pooled value into three exact bf16
    # terms, so the selections still follow the exact scores
    _say("gate minmax, fp32 pooled keys", w.name, "seed 7")
    x = inputs.make_inputs(w, device=dev, seed=7)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    gen = torch.Generator(device="cpu").manual_seed(7)
    k32 = x["k"].float().cpu() + 1e-3 * torch.randn(x["k"].shape, generator=gen)
    assert bool((k32 != k32.to(torch.bfloat16).float()).any())
    kmm = moba.moba_pool_minmax(k32.to(dev), geom)
    idx = moba.moba_gate_topk_minmax(x["q"], kmm, geom, w.topk).cpu().numpy()
    rows = np.stack(np.meshgrid(np.arange(w.total_tokens), np.arange(w.heads), indexing="ij"),
                    -1).reshape(-1, 2)
    _check_minmax_idx(x["q"].float().cpu().numpy(), k32.numpy(), x["cu_seqlens"],
                      w.block_size, w.topk, idx, rows)


@pytest.mark.parametrize("w", [
    inputs.custom([5000, 3192], 4, 128, 512, 4, "bf16", name="minmax-fwd-8k"),
    inputs.custom([6000, 2100], 2, 128, 1024, 3, "bf16", name="minmax-fwd-B1024"),
], ids=lambda w: w.name)
def test_forward_minmax(dev, w):
    _say("forward minmax", w.name, "seed 3")
    x = inputs.make_inputs(w, device=dev, seed=3)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    out, lse, idx = moba.forward_minmax(x["q"], x["k"], x["v"], geom, w.topk, w.scale,
                                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = inputs.sample_rows(w, 256, seed=3)
    hq, hk, hv = (x[n].float().cpu().numpy() for n in ("q", "k", "v"))
    use = _check_minmax_idx(hq, hk, x["cu_seqlens"], w.block_size, w.topk, idx.cpu().numpy(),
                            rows)
    o_ref, lse_ref = mo.attend_given_selection(hq, hk, hv, x["cu_seqlens"], w.block_size, use,
                                               w.scale, rows)
    o = out.cpu().numpy()[rows[:, 0], rows[:, 1]]
    l = lse.cpu().numpy()[rows[:, 0], rows[:, 1]]
    parity.assert_within(parity.error_stats(o, o_ref, l, lse_ref), parity.BF16_TOL, w.name)


def test_hybrid_layers(dev):
    # the layer-wise hybrid: MoBA layers run pool/gate/sparse attention, full
    # layers the dense causal kernel, on the same inputs
    w = inputs.custom([3000, 1500], 2, 128, 256, 3, "bf16", name="hybrid")
    _say("hybrid", w.name)
    x = inputs.make_inputs(w, device=dev, seed=4)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    sched = moba.hybrid_schedule(3, 1)
    outs = [moba.layer_forward(m, x["q"], x["k"], x["v"], geom, w.topk, w.scale,
                               out_dtype=torch.float32) for m in sched]
    ref_moba = moba.forward(x["q"], x["k"], x["v"], geom, w.topk, w.scale,
                            out_dtype=torch.float32)
    ref_full = moba.dense(x["q"], x["k"], x["v"], geom, w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for m, (o, l) in zip(sched, outs):
        ro, rl = (ref_moba[0], ref_moba[1]) if m == "moba" else ref_full
        assert torch.equal(o, ro) and torch.equal(l, rl), m
    # and the full layer against the oracle on sampled rows
    rows = inputs.sample_rows(w, 128, seed=4)
    hq, hk, hv = (x[n].float().cpu().numpy() for n in ("q", "k", "v"))
    o_ref, lse_ref = mo.dense_causal_reference(hq, hk, hv, x["cu_seqlens"], w.scale, rows=rows)
    o = outs[-1][0].cpu().numpy()[rows[:, 0], rows[:, 1]]
    l = outs[-1][1].cpu().numpy()[rows[:, 0], rows[:, 1]]
    parity.assert_within(parity.error_stats(o, o_ref, l, lse_ref), parity.BF16_TOL, "hybrid full")
