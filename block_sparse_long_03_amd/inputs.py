"""Seeded synthetic inputs for the MoBA prefill workloads.

This module only draws random numbers and lays out packed batches; it holds
none of the method's arithmetic, so the tests can feed the same tensors to the
HIP library and to the CPU oracle.

Workloads (shapes follow the pages' settings: the 8K scaling-law block size,
the 32K fine-grained 128-block / 75 % setting, the 128K RULER setting with
B = 4096, k = 12, and the 1M-token Llama setting with B = 4096, k = 12):

  tiny   1 x 1024 tokens, 2 heads, d 64,  B 128,  k 3,  fp32
  8k     1 x 8192,        16 heads, d 128, B 512,  k 4,  bf16
  32k    1 x 32768,       32 heads, d 128, B 256,  k 32, bf16, low-rank K bias
  varlen 65536/32768/16384/16384 packed, 32 heads, d 128, B 4096, k 12, bf16
  1m     1 x 1048576,     32 heads, d 128, B 4096, k 12, bf16
  10m    1 x 10485760,    4 heads (one GPU's share of 32), d 128, B 40960, k 12, bf16
  10m32  1 x 10485760,    32 heads in 8 streamed groups of 4, d 128, B 40960, k 12

Recipe: one torch.Generator seeded with ``seed`` (default 1000 + workload
index) on the target device draws Q, then K, then V, each i.i.d. N(0, 1) in
fp32, token-chunk by token-chunk, then rounds to the workload dtype (round to
nearest even for bf16).  For "32k" the generator then draws, per head,
A_h [T, 4] and C_h [4, d] i.i.d. N(0, 1) and adds 0.25 * A_h C_h (elements of
std 0.5, rank 4) to K in fp32 before rounding.

Streamed workloads (``head_group`` > 0) are too large for one GPU's memory as
a whole layer (10M tokens x 32 heads: 86 GB per bf16 tensor), so their Q/K/V
exist one group of heads at a time: group g (heads g * head_group ..) is drawn
by ``make_head_group`` with the recipe above for head_group heads and the seed
1000 + 100 * index + g, standing in for the projections that produce a head
group's Q/K/V in a model.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seqlens: tuple
    heads: int
    head_dim: int
    block_size: int
    topk: int
    dtype: str  # "f32" or "bf16"
    lowrank_bias: bool = False
    index: int = 0
    head_group: int = 0  # > 0: the layer is streamed in groups of this many heads

    @property
    def total_tokens(self):
        return int(sum(self.seqlens))

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    "tiny": Workload("tiny", (1024,), 2, 64, 128, 3, "f32", index=0),
    "8k": Workload("8k", (8192,), 16, 128, 512, 4, "bf16", index=1),
    "32k": Workload("32k", (32768,), 32, 128, 256, 32, "bf16", lowrank_bias=True, index=2),
    "varlen": Workload("varlen", (65536, 32768, 16384, 16384), 32, 128, 4096, 12, "bf16", index=3),
    "1m": Workload("1m", (1 << 20,), 32, 128, 4096, 12, "bf16", index=4),
    # constant sparsity at 10M tokens: the block count of the 1M workload
    # (256) kept, so B grows to 40960; 4 heads = one GPU's share of 32 heads
    # sharded by head over 8 GPUs
    "10m": Workload("10m", (10 << 20,), 4, 128, 40960, 12, "bf16", index=5),
    # the same 10M-token layer with all 32 heads on one GPU, streamed in
    # groups of 4 heads
    "10m32": Workload("10m32", (10 << 20,), 32, 128, 40960, 12, "bf16", index=6, head_group=4),
}


def custom(seqlens, heads, head_dim, block_size, topk, dtype="bf16", name="custom",
           lowrank_bias=False):
    """A workload of arbitrary geometry (edge-case tests)."""
    return Workload(name, tuple(int(x) for x in seqlens), heads, head_dim, block_size,
                    topk, dtype, lowrank_bias, index=99)


def cu_seqlens_of(seqlens):
    out = [0]
    for L in seqlens:
        out.append(out[-1] + int(L))
    return out


def cu_blocks_of(seqlens, block_size):
    out = [0]
    for L in seqlens:
        out.append(out[-1] + (int(L) + block_size - 1) // block_size)
    return out


def _randn_into(dst, gen, chunk_tokens):
    T = dst.shape[0]
    for a in range(0, T, chunk_tokens):
        b = min(T, a + chunk_tokens)
        x = torch.randn((b - a,) + tuple(dst.shape[1:]), generator=gen,
                        device=dst.device, dtype=torch.float32)
        dst[a:b].copy_(x)
        del x


def make_inputs(w: Workload, device="cpu", seed=None, chunk_tokens=65536):
    """Returns dict(q, k, v [T, H, d] in the workload dtype on ``device``,
    cu_seqlens (python list), cu_blocks (python list))."""
    if seed is None:
        seed = 1000 + w.index
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    T, H, d = w.total_tokens, w.heads, w.head_dim
    shape = (T, H, d)
    q = torch.empty(shape, dtype=w.torch_dtype, device=dev)
    k = torch.empty(shape, dtype=w.torch_dtype, device=dev)
    v = torch.empty(shape, dtype=w.torch_dtype, device=dev)
    _randn_into(q, gen, chunk_tokens)
    if w.lowrank_bias:
        kf = torch.empty(shape, dtype=torch.float32, device=dev)
        _randn_into(kf, gen, chunk_tokens)
        _randn_into(v, gen, chunk_tokens)
        A = torch.randn((H, T, 4), generator=gen, device=dev, dtype=torch.float32)
        C = torch.randn((H, 4, d), generator=gen, device=dev, dtype=torch.float32)
        bias = torch.bmm(A, C).mul_(0.25)  # [H, T, d]
        kf.add_(bias.permute(1, 0, 2))
        del bias, A, C
        k.copy_(kf)
        del kf
    else:
        _randn_into(k, gen, chunk_tokens)
        _randn_into(v, gen, chunk_tokens)
    return dict(q=q, k=k, v=v, cu_seqlens=cu_seqlens_of(w.seqlens),
                cu_blocks=cu_blocks_of(w.seqlens, w.block_size))


def make_head_group(w: Workload, group, device="cpu", chunk_tokens=65536):
    """Q, K, V of head group ``group`` of a streamed workload: heads
    group * w.head_group .. (group + 1) * w.head_group - 1 as [T, head_group,
    d] tensors (same recipe as make_inputs, seed 1000 + 100 * index + group)."""
    if w.head_group <= 0:
        raise ValueError(f"{w.name} is not a streamed workload")
    h0 = group * w.head_group
    hg = min(w.head_group, w.heads - h0)
    if hg <= 0:
        raise ValueError(f"{w.name} has no head group {group}")
    wg = Workload(w.name, w.seqlens, hg, w.head_dim, w.block_size, w.topk, w.dtype,
                  w.lowrank_bias, w.index)
    return make_inputs(wg, device=device, seed=1000 + 100 * w.index + group,
                       chunk_tokens=chunk_tokens)


def sample_rows(w: Workload, per_head, seed=None, heads=None):
    """Seeded sample of (token, head) rows: ``per_head`` distinct tokens for
    each head in ``heads`` (default all), drawn with numpy default_rng(2000 +
    workload index)."""
    import numpy as np
    rng = np.random.default_rng(2000 + w.index if seed is None else seed)
    T = w.total_tokens
    hs = range(w.heads) if heads is None else heads
    rows = []
    for h in hs:
        ts = rng.choice(T, size=min(per_head, T), replace=False)
        ts.sort()
        rows.extend((int(t), int(h)) for t in ts)
    return np.asarray(rows, dtype=np.int64).reshape(-1, 2)
