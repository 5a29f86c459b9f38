"""Static routing (sliding window, sink + window, full attention) on MI355X
through the C ABI: the rows of moba_static_select bit-exact against the
oracle's rule, and the attention over them against the oracle's softmax over
the statically chosen tokens.

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


@pytest.mark.parametrize("seqlens,B,H", [
    ([1000, 0, 64, 777, 4161], 64, 3),     # ragged tails, an empty sequence
    ([8192 + 100, 300], 256, 2),
    ([5000], 1024, 1),
])
@pytest.mark.parametrize("topk,sink", [(1, 0), (1, 3), (3, 0), (3, 1), (5, 2), (12, 1),
                                       (12, 0), (64, 0), (4, 30)])
def test_static_select_rows(dev, seqlens, B, H, topk, sink):
    _say("static select", seqlens, "B", B, "H", H, "k", topk, "sink", sink)
    geom = moba.Geometry.make(seqlens, B, dev, is_cu=False)
    idx = moba.moba_static_select(geom, H, topk, sink).cpu().numpy()
    cu = inputs.cu_seqlens_of(seqlens)
    ref = mo.static_select(cu, B, topk, sink)
    assert idx.shape == (geom.total_tokens, H, topk)
    for h in range(H):
        bad = np.nonzero(np.any(idx[:, h, :] != ref, axis=1))[0]
        assert bad.size == 0, (f"head {h}: {bad.size} rows differ, e.g. token {bad[0]}: "
                               f"gpu {idx[bad[0], h].tolist()} oracle {ref[bad[0]].tolist()}")


def _static_case(dev, w, sink, rows_per_head, seed=3, out_dtype=torch.float32):
    _say("static forward", w.name, w.seqlens[:4], "H", w.heads, "d", w.head_dim, "B",
         w.block_size, "k", w.topk, "sink", sink, "seed", seed)
    x = inputs.make_inputs(w, device=dev, seed=seed)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    out, lse, idx = moba.forward_static(x["q"], x["k"], x["v"], geom, w.topk, sink, w.scale,
                                        out_dtype=out_dtype)
    torch.cuda.synchronize()
    rows = inputs.sample_rows(w, rows_per_head, seed=seed)
    hq = x["q"].float().cpu().numpy()
    hk = x["k"].float().cpu().numpy()
    hv = x["v"].float().cpu().numpy()
    ref = mo.static_reference(hq, hk, hv, x["cu_seqlens"], w.block_size, w.topk, sink, w.scale,
                              rows=rows)
    gi = idx.cpu().numpy()[rows[:, 0], rows[:, 1]]
    assert np.array_equal(gi, ref["idx"]), "static rows differ from the oracle"
    o = out.float().cpu().numpy()[rows[:, 0], rows[:, 1]]
    l = lse.cpu().numpy()[rows[:, 0], rows[:, 1]]
    tol = parity.F32_TOL if w.dtype == "f32" else parity.BF16_TOL
    st = parity.error_stats(o, ref["out"], l, ref["lse"])
    parity.assert_within(st, tol, w.name)
    return x, geom, out, lse


@pytest.mark.parametrize("w,sink", [
    (inputs.custom([3000, 5192], 4, 128, 256, 4, "bf16", name="window-B256-k4"), 0),
    (inputs.custom([3000, 5192], 4, 128, 256, 4, "bf16", name="sink1-B256-k4"), 1),
    (inputs.custom([6000, 2100], 2, 128, 1024, 3, "bf16", name="sink1-B1024-k3"), 1),
    (inputs.custom([777, 2000], 2, 64, 128, 5, "bf16", name="sink2-d64-k5"), 2),
    (inputs.custom([1024, 600], 2, 64, 128, 3, "f32", name="window-f32"), 0),
], ids=lambda a: a.name if hasattr(a, "name") else str(a))
def test_static_forward(dev, w, sink):
    _static_case(dev, w, sink, 256)


def test_static_full_equals_dense(dev):
    # k covering every block: full causal attention, checked against the
    # oracle and against the library's own dense kernel
    w = inputs.custom([2500, 1100], 2, 128, 256, 10, "bf16", name="static-full")
    x, geom, out, lse = _static_case(dev, w, 0, 192)
    od, lsed = moba.dense(x["q"], x["k"], x["v"], geom, w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    d = (out.float() - od.float()).abs().max().item()
    dl = (lse - lsed).abs().max().item()
    print("[stats] full vs dense kernel", d, dl, flush=True)
    assert d <= 1e-2 and dl <= 1e-3
