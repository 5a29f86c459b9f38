"""Measurement support on MI355X through the C ABI: the MFMA rate probes
(every operand kind runs and leaves finite, repeatable sums) and the
per-kernel profiler (one record per stage of a MoBA forward).

Every case prints its name before it touches the GPU.
"""

import sys

import pytest
import torch

from block_sparse_long_03_amd import inputs, moba

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


@pytest.mark.parametrize("operands", [0, 1, 2])
def test_mfma_probe_kinds(dev, operands):
    _say("mfma probe", "operands", operands)
    wg, iters = 8, 64
    sink = torch.full((wg * 256,), float("nan"), dtype=torch.float32, device=dev)
    flops = moba.probe_mfma_rate(wg, iters, sink, operands)
    assert flops == wg * 4 * 4 * iters * 2 * 32 * 32 * 16
    first = sink.clone()
    moba.probe_mfma_rate(wg, iters, sink, operands)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(first).all())
    assert torch.equal(first, sink)  # the same products in the same order
    assert float(first.abs().sum()) > 0.0


def test_profiler_records_each_stage(dev):
    w = inputs.custom([3000, 1100], 2, 128, 256, 4, "bf16", name="profiler")
    _say("profiler", w.seqlens, "B", w.block_size, "k", w.topk)
    x = inputs.make_inputs(w, device=dev, seed=3)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    p = moba.Profiler().attach()
    try:
        p.reset()
        moba.forward(x["q"], x["k"], x["v"], geom, w.topk, w.scale)
        torch.cuda.synchronize()
        names = set(p.names())
        for stage in ("pool_keys", "gate_topk", "v_stage", "bucket", "attn_hist", "attn_own",
                      "merge"):
            assert stage in names, (stage, names)
            n, ms = p.read(stage)
            assert n == 1 and ms > 0.0, (stage, n, ms)
    finally:
        p.detach()
