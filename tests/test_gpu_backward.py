"""Backward of the MoBA attention on MI355X through the C ABI against the
oracle's fp64 gradients (the softmax-attention gradients over each query's
selected tokens; the hard top-k is not differentiated), on every (token,
head) row of the case.

The selection is an input of the backward: both sides use the selection the
GPU forward made.  Gradient tolerance (derived from the arithmetic): P and dS
enter the products as bf16 (relative rounding <= 2^-9 per element) while
every other operand is exact and accumulation is fp32, so each gradient
element carries a relative error of order 2^-9 of its terms' magnitudes.
The bar is a relative L2 error <= 1e-2 per tensor and a max abs error
<= 1e-2 of the tensor's largest reference magnitude.

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

GRAD_TOL = dict(rel_l2=1e-2, max_abs_rel=1e-2)


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _grad_stats(name, got, ref):
    diff = np.asarray(got, np.float64) - ref
    scale = float(np.abs(ref).max())
    return {f"{name}_rel_l2": float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)),
            f"{name}_max_abs": float(np.abs(diff).max()),
            f"{name}_max_ref": scale}


def _backward_case(dev, w, seed, out_dtype=torch.float32, static_sink=None):
    _say("backward", w.name, w.seqlens[:4], "H", w.heads, "d", w.head_dim, "B", w.block_size,
         "k", w.topk, "seed", seed, "out", out_dtype)
    x = inputs.make_inputs(w, device=dev, seed=seed)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    if static_sink is None:
        out, lse, idx = moba.forward(x["q"], x["k"], x["v"], geom, w.topk, w.scale,
                                     out_dtype=out_dtype)
    else:
        out, lse, idx = moba.forward_static(x["q"], x["k"], x["v"], geom, w.topk, static_sink,
                                            w.scale, out_dtype=out_dtype)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 1)
    dout = torch.randn(x["q"].shape, generator=gen, device=dev, dtype=torch.float32)
    dout = dout.to(torch.bfloat16)
    dq, dk, dv = moba.moba_attn_bwd(x["q"], x["k"], x["v"], out, dout, lse, geom, w.topk, idx,
                                    w.scale)
    torch.cuda.synchronize()
    hq, hk, hv, hg = (t.float().cpu().numpy() for t in (x["q"], x["k"], x["v"], dout))
    ref = mo.moba_backward_reference(hq, hk, hv, hg, x["cu_seqlens"], w.block_size,
                                     idx.cpu().numpy().astype(np.int64), w.scale)
    st = {}
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        st.update(_grad_stats(name, got.cpu().numpy(), r))
    parity.emit(st)
    for name in ("dq", "dk", "dv"):
        assert st[f"{name}_rel_l2"] <= GRAD_TOL["rel_l2"], (name, st)
        assert st[f"{name}_max_abs"] <= GRAD_TOL["max_abs_rel"] * st[f"{name}_max_ref"], (name, st)
    return st


CASES = [
    # ragged tails, an empty and a 1-token sequence, B 64, k 4
    inputs.custom([700, 0, 129, 1, 300], 2, 128, 64, 4, "bf16", name="bwd-ragged-B64"),
    # d 64, B 128, k 3
    inputs.custom([1024, 777], 2, 64, 128, 3, "bf16", name="bwd-d64"),
    # B 256, k 5, one long sequence with a ragged tail
    inputs.custom([2048 + 33], 2, 128, 256, 5, "bf16", name="bwd-B256-k5"),
    # B 1024 (four 128-key groups per block), ragged
    inputs.custom([3000, 1100], 1, 128, 1024, 3, "bf16", name="bwd-B1024"),
    # k = 1: own block only
    inputs.custom([1000, 500], 2, 128, 128, 1, "bf16", name="bwd-k1"),
    # k larger than every block count: dense causal
    inputs.custom([520, 900], 2, 128, 128, 16, "bf16", name="bwd-k>n"),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_backward_all_rows(dev, w):
    _backward_case(dev, w, seed=21)


def test_backward_bf16_out_and_static_window(dev):
    # the forward's bf16 output feeds D = rowsum(dO * O); a sliding-window
    # selection (perfectly regular lists)
    w = inputs.custom([1500, 700], 2, 128, 128, 4, "bf16", name="bwd-window-bf16out")
    _backward_case(dev, w, seed=22, out_dtype=torch.bfloat16, static_sink=0)


def test_backward_1m_sampled(dev):
    """The backward at the 1M-token workload (H 32, B 4096, k 12) in the
    configuration bench.py times: dq on 32 seeded rows of two heads (each row
    from its own attended tokens), dk and dv on 16 seeded keys of the last two
    blocks' tails of head 0 (every query attending them), and over every row the
    exact identities of the gradients: per head, dk sums to zero over the
    sequence and dv sums to the sum of dout."""
    w = inputs.WORKLOADS["1m"]
    _say("backward 1m", "seed default")
    x = inputs.make_inputs(w, device=dev)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    out, lse, idx = moba.forward(x["q"], x["k"], x["v"], geom, w.topk, w.scale)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    dout = torch.randn(x["q"].shape, generator=gen, device=dev, dtype=torch.float32)
    dout = dout.to(torch.bfloat16)
    dq, dk, dv = moba.moba_attn_bwd(x["q"], x["k"], x["v"], out, dout, lse, geom, w.topk, idx,
                                    w.scale)
    torch.cuda.synchronize()
    T = w.total_tokens
    # identities over every row, in fp64
    sk = dk.double().sum(0)                        # [H, d]
    nk = dk.double().norm(dim=2).sum(0)            # [H]
    sv = dv.double().sum(0) - dout.double().sum(0)
    nv = dout.double().norm(dim=2).sum(0)
    rk = (sk.norm(dim=1) / nk).max().item()
    rv = (sv.norm(dim=1) / nv).max().item()
    print("[stats] identities", rk, rv, flush=True)
    assert rk <= 1e-4 and rv <= 1e-4, (rk, rv)
    assert bool(torch.isfinite(dq).all()) and bool(torch.isfinite(dk).all())
    # sampled rows against the oracle (host copies of the two heads used)
    st = {}
    heads = [0, 9]
    host = {h: tuple(t[:, h:h + 1].float().cpu().numpy() for t in (x["q"], x["k"], x["v"], dout))
            for h in heads}
    idx_h = {h: idx[:, h:h + 1].cpu().numpy().astype(np.int64) for h in heads}
    got, ref = [], []
    rows = inputs.sample_rows(w, 16, seed=31, heads=heads)
    for h in heads:
        r_h = rows[rows[:, 1] == h]
        r0 = np.stack([r_h[:, 0], np.zeros(len(r_h), dtype=np.int64)], axis=1)
        qh, kh, vh, gh = host[h]
        ref.append(mo.backward_dq_rows(qh, kh, vh, gh, x["cu_seqlens"], w.block_size,
                                       idx_h[h][r_h[:, 0], 0], w.scale, r0))
        got.append(dq[torch.as_tensor(r_h[:, 0], device=dev), h].cpu().numpy())
    st.update(_grad_stats("dq", np.concatenate(got), np.concatenate(ref)))
    # keys in the last 128 positions of the last two blocks: each is attended
    # by at most 128 own-block queries plus the later queries that selected
    # its block, which keeps the oracle's work to a few hundred rows
    rng = np.random.default_rng(32)
    tails = np.concatenate([np.arange(T - w.block_size - 128, T - w.block_size),
                            np.arange(T - 128, T)])
    keys = np.sort(rng.choice(tails, 16, replace=False))
    qh, kh, vh, gh = host[0]
    k0 = np.stack([keys, np.zeros(16, dtype=np.int64)], axis=1)
    rk_, rv_ = mo.backward_dkdv_keys(qh, kh, vh, gh, x["cu_seqlens"], w.block_size, idx_h[0],
                                     w.scale, k0)
    kt = torch.as_tensor(keys, device=dev)
    st.update(_grad_stats("dk", dk[kt, 0].cpu().numpy(), rk_))
    st.update(_grad_stats("dv", dv[kt, 0].cpu().numpy(), rv_))
    parity.emit(st)
    for name in ("dq", "dk", "dv"):
        assert st[f"{name}_rel_l2"] <= GRAD_TOL["rel_l2"], (name, st)
        assert st[f"{name}_max_abs"] <= GRAD_TOL["max_abs_rel"] * st[f"{name}_max_ref"], (name, st)
    del x, out, lse, idx, dout, dq, dk, dv
    torch.cuda.empty_cache()
