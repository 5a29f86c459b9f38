"""Value magnitudes, head-group passes, reproducibility and guard bands of the
forward pass (through the C ABI) on MI355X.

- V scaled by exact powers of two (2^-20, 2^+20, and a batch mixing a small,
  a large and an unscaled head): the fp16 staging of V must follow each
  head's magnitude.  Scaling V by 2^s scales the exact output by 2^s and
  leaves lse unchanged, so the GPU output divided by 2^s is checked against
  the oracle on the unscaled V with the usual tolerances.
- head_chunk < num_heads: the same results, bit for bit, as one pass over
  all heads, and the oracle's on sampled rows.
- Two runs of the same forward are bitwise identical (the order of the
  bucket lists depends on scheduling, the results must not).
- Guard bands around out, lse, block_idx, kbar and the workspace (sized
  exactly as the library asks) are untouched.

Every case prints its name and shape before it touches the GPU.
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


def _all_rows(T, H, limit, seed):
    rows = np.stack(np.meshgrid(np.arange(T), np.arange(H), indexing="ij"), -1).reshape(-1, 2)
    if len(rows) > limit:
        rows = rows[np.random.default_rng(seed).choice(len(rows), limit, replace=False)]
        rows = rows[np.lexsort((rows[:, 0], rows[:, 1]))]
    return rows


# ---------------------------------------------------------------------------
# V magnitude
# ---------------------------------------------------------------------------

SCALE_CASES = [
    # resident historical tiles (B 128), own block, merge
    (inputs.custom([3000, 1100], 3, 128, 128, 4, "bf16", name="vscale-B128"), "small"),
    (inputs.custom([3000, 1100], 3, 128, 128, 4, "bf16", name="vscale-B128"), "large"),
    (inputs.custom([3000, 1100], 3, 128, 128, 4, "bf16", name="vscale-B128"), "mixed"),
    # streamed historical tiles (B 1024, 8 waves) and d 64
    (inputs.custom([5000, 700], 3, 128, 1024, 3, "bf16", name="vscale-B1024"), "mixed"),
    (inputs.custom([2600], 3, 64, 256, 5, "bf16", name="vscale-d64"), "mixed"),
]

EXPONENTS = {"small": [-20, -20, -20], "large": [20, 20, 20], "mixed": [-20, 20, 0]}


def _scaled_v(x, exps):
    """V with head h multiplied by 2^exps[h] (exact in bf16)."""
    v = x["v"].clone()
    for h, e in enumerate(exps):
        v[:, h, :].mul_(2.0 ** e)
    return v


@pytest.mark.parametrize("w,kind", SCALE_CASES, ids=[f"{w.name}-{k}" for w, k in SCALE_CASES])
def test_forward_v_magnitude(dev, w, kind):
    exps = EXPONENTS[kind]
    _say("v magnitude", w.name, kind, exps, w.seqlens, "H", w.heads, "d", w.head_dim,
         "B", w.block_size, "k", w.topk)
    x = inputs.make_inputs(w, device=dev, seed=31)
    v = _scaled_v(x, exps)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    out, lse, idx = moba.forward(x["q"], x["k"], v, geom, w.topk, w.scale,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    unscaled = out.clone()
    for h, e in enumerate(exps):
        unscaled[:, h, :].mul_(2.0 ** -e)
    rows = _all_rows(w.total_tokens, w.heads, 3000, 9)
    st = parity.check_moba_rows(x["q"], x["k"], x["v"], x["cu_seqlens"], w.block_size, w.topk,
                                w.scale, unscaled, lse, idx, rows, parity.BF16_TOL)
    print(w.name, kind, st)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dense_v_magnitude(dev, out_dtype):
    w = inputs.custom([1500, 700], 3, 128, 128, 2, "bf16", name="dense-vscale")
    exps = EXPONENTS["mixed"]
    _say("dense v magnitude", w.seqlens, exps, out_dtype)
    x = inputs.make_inputs(w, device=dev, seed=32)
    v = _scaled_v(x, exps)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    out, lse = moba.dense(x["q"], x["k"], v, geom, w.scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    unscaled = out.float()
    for h, e in enumerate(exps):
        unscaled[:, h, :].mul_(2.0 ** -e)
    rows = _all_rows(w.total_tokens, w.heads, 1500, 3)
    o_ref, l_ref = mo.dense_causal_reference(x["q"].float().cpu().numpy(),
                                             x["k"].float().cpu().numpy(),
                                             x["v"].float().cpu().numpy(), x["cu_seqlens"],
                                             w.scale, rows=rows)
    tt, hh = torch.as_tensor(rows[:, 0]), torch.as_tensor(rows[:, 1])
    st = parity.error_stats(unscaled[tt, hh].cpu().numpy(), o_ref, lse[tt, hh].cpu().numpy(),
                            l_ref)
    parity.assert_within(st, parity.BF16_TOL, w.name)


# ---------------------------------------------------------------------------
# head-group passes
# ---------------------------------------------------------------------------

CHUNK_CASES = [
    inputs.custom([3000, 0, 1100], 3, 128, 128, 4, "bf16", name="chunk-resident"),
    inputs.custom([5000, 700], 5, 128, 1024, 3, "bf16", name="chunk-B1024"),
    inputs.custom([700, 301], 3, 64, 64, 3, "f32", name="chunk-f32"),
]


@pytest.mark.parametrize("w", CHUNK_CASES, ids=[w.name for w in CHUNK_CASES])
def test_head_chunk(dev, w):
    _say("head chunk", w.name, w.seqlens, "H", w.heads, "d", w.head_dim, "B", w.block_size,
         "k", w.topk, w.dtype)
    x = inputs.make_inputs(w, device=dev, seed=41)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    q, k, v = x["q"], x["k"], x["v"]
    out0, lse0, idx = moba.forward(q, k, v, geom, w.topk, w.scale, out_dtype=torch.float32)
    for hc in (1, 2):
        ws_bytes = moba.moba_attn_workspace_bytes(moba._dtype_code(q.dtype), geom.total_tokens,
                                                  geom.total_blocks, w.heads, w.head_dim,
                                                  w.block_size, w.topk, hc)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        out, lse = moba.moba_attn_fwd(q, k, v, geom, w.topk, idx, w.scale,
                                      out_dtype=torch.float32, workspace=ws, head_chunk=hc)
        torch.cuda.synchronize()
        assert torch.equal(out, out0), f"head_chunk {hc}: out differs from one pass"
        assert torch.equal(lse, lse0), f"head_chunk {hc}: lse differs from one pass"
    rows = _all_rows(w.total_tokens, w.heads, 2000, 4)
    tol = parity.F32_TOL if w.dtype == "f32" else parity.BF16_TOL
    st = parity.check_moba_rows(q, k, v, x["cu_seqlens"], w.block_size, w.topk, w.scale, out,
                                lse, idx, rows, tol)
    print(w.name, st)


# ---------------------------------------------------------------------------
# reproducibility
# ---------------------------------------------------------------------------

def test_deterministic_32k(dev):
    """The fine-grained 32K workload (lists of up to ~19K queries per block,
    cut into resident tiles) run twice: bitwise identical results."""
    w = inputs.WORKLOADS["32k"]
    _say("deterministic", w.name)
    x = inputs.make_inputs(w, device=dev)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    out1, lse1, idx1 = moba.forward(x["q"], x["k"], x["v"], geom, w.topk, w.scale)
    out2, lse2, idx2 = moba.forward(x["q"], x["k"], x["v"], geom, w.topk, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2)
    assert torch.equal(out1, out2)
    assert torch.equal(lse1, lse2)


# ---------------------------------------------------------------------------
# guard bands
# ---------------------------------------------------------------------------

GUARD = 4096  # elements (bytes for the workspace) on each side


def _guarded(n, dtype, dev, fill_bits):
    """A flat buffer of n elements between two guard bands whose bit pattern
    is fill_bits (also written into the payload).  Returns (buffer, payload)."""
    buf = torch.empty(n + 2 * GUARD, dtype=dtype, device=dev)
    int_t = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[buf.element_size()]
    buf.view(int_t).fill_(fill_bits)
    return buf, buf[GUARD:GUARD + n]


def _guards_intact(buf, fill_bits):
    int_t = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[buf.element_size()]
    b = buf.view(int_t)
    return bool((b[:GUARD] == fill_bits).all()) and bool((b[-GUARD:] == fill_bits).all())


@pytest.mark.parametrize("w,hc", [
    (inputs.custom([700, 0, 129, 1, 64, 300], 3, 128, 64, 4, "bf16", name="guard-ragged"), 0),
    (inputs.custom([3000, 1100], 3, 128, 128, 4, "bf16", name="guard-resident"), 2),
    (inputs.custom([5000, 700], 2, 128, 1024, 3, "bf16", name="guard-B1024"), 0),
    (inputs.custom([300, 77, 512], 2, 128, 64, 3, "f32", name="guard-f32"), 1),
], ids=lambda p: p.name if hasattr(p, "name") else f"hc{p}")
def test_guard_bands(dev, w, hc):
    _say("guard bands", w.name, w.seqlens, "H", w.heads, "B", w.block_size, "k", w.topk,
         "head_chunk", hc)
    x = inputs.make_inputs(w, device=dev, seed=12)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    T, H, d, k = w.total_tokens, w.heads, w.head_dim, w.topk
    dt = x["q"].dtype
    kb_buf, kbar = _guarded(geom.total_blocks * H * d, torch.float32, dev, 0x7FC0BEEF)
    ix_buf, idx = _guarded(T * H * k, torch.int32, dev, 0x5A5A5A5A)
    o_buf, out = _guarded(T * H * d, dt, dev, 0x7FBF if dt == torch.bfloat16 else 0x7FC0BEEF)
    l_buf, lse = _guarded(T * H, torch.float32, dev, 0x7FC0BEEF)
    nbytes = moba.moba_attn_workspace_bytes(moba._dtype_code(dt), T, geom.total_blocks, H, d,
                                            w.block_size, k, hc)
    w_buf, ws = _guarded(nbytes, torch.uint8, dev, 0xA5)
    k3_buf, kbar3 = _guarded(geom.total_blocks * H * 3 * d, torch.bfloat16, dev, 0x7FBF)
    pooled = moba.moba_pool_keys(x["k"], geom, kbar=kbar.view(geom.total_blocks, H, d),
                                 kbar3=kbar3.view(H, 3, d // 16, geom.total_blocks, 16))
    moba.moba_gate_topk(x["q"], pooled, geom, k,
                        block_idx=idx.view(T, H, k))
    moba.moba_attn_fwd(x["q"], x["k"], x["v"], geom, k, idx.view(T, H, k), w.scale,
                       out=out.view(T, H, d), lse=lse.view(T, H), workspace=ws, head_chunk=hc)
    torch.cuda.synchronize()
    assert _guards_intact(kb_buf, 0x7FC0BEEF), "kbar guard band overwritten"
    assert _guards_intact(k3_buf, 0x7FBF), "kbar3 guard band overwritten"
    assert _guards_intact(ix_buf, 0x5A5A5A5A), "block_idx guard band overwritten"
    assert _guards_intact(o_buf, 0x7FBF if dt == torch.bfloat16 else 0x7FC0BEEF), \
        "out guard band overwritten"
    assert _guards_intact(l_buf, 0x7FC0BEEF), "lse guard band overwritten"
    assert _guards_intact(w_buf, 0xA5), "workspace guard band overwritten"
    # every output element was written (no payload keeps the fill pattern)
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(lse).all())
    assert bool(((idx >= -1) & (idx < (1 << 20))).all())
    rows = _all_rows(T, H, 1500, 2)
    tol = parity.F32_TOL if w.dtype == "f32" else parity.BF16_TOL
    parity.check_moba_rows(x["q"], x["k"], x["v"], x["cu_seqlens"], w.block_size, k, w.scale,
                           out.view(T, H, d), lse.view(T, H), idx.view(T, H, k), rows, tol)
