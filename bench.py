#!/usr/bin/env python3
"""MoBA causal prefill forward on one MI355X: ms per layer, effective TFLOP/s,
speedup over the library's own dense causal kernel, roofline of the dominant
kernel and the CPU oracle on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1m]

One step is one layer of the MoBA forward over all heads: key pooling, gate
and top-k, query bucketing, historical-block and own-block attention, merge
(every call goes through libmoba.so's C ABI).  Inputs, outputs and the
workspace are resident in HBM before timing starts.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoBA prefill ms/layer + effective TFLOP/s at 32K–1M; speedup vs own dense"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def attended_pairs(seqlens, B, k, H):
    """(total, historical, own) attended (query, key) pairs of the MoBA forward:
    per query (t mod B) + 1 own-block keys and B keys per selected past block,
    min(k - 1, c) of them."""
    import numpy as np
    tot = hist = own = 0
    for L in seqlens:
        t = np.arange(L, dtype=np.int64)
        c = t // B
        o = (t % B + 1).sum()
        hh = (B * np.minimum(k - 1, c)).sum()
        own += int(o)
        hist += int(hh)
    return H * (own + hist), H * hist, H * own


def dense_pairs(seqlens, H):
    return H * sum(L * (L + 1) // 2 for L in seqlens)


def mfma_tile_q(key_range):
    """Query columns of a dense / own-block tile (launch.h: 8 waves of 32 for
    key ranges of 1024 and more, else 4)."""
    return 32 * (8 if key_range >= 1024 else 4)


def prefix_route(seqlens, B, k, H, dtype):
    """Whether moba_attn_fwd sends the rows of each sequence's first k blocks
    that select every earlier block through its dense kernel (the library's
    rule, api.cpp: bf16, and a dense launch over the first k B positions of
    every sequence and all heads of at least 256 workgroups)."""
    if dtype != "bf16" or not seqlens:
        return False
    span = min(max(seqlens), k * B)
    if span <= 0:
        return False
    tq = mfma_tile_q(span)
    return (span + tq - 1) // tq * len(seqlens) * H >= 256


def attended_pairs_by_kernel(seqlens, B, k, H, route):
    """(historical, own, prefix) attended pairs as the kernels split them:
    with the dense-prefix route, rows of the first k blocks (each selects every
    earlier block under the gates timed here) attend their t + 1 keys in the
    dense prefix launch, not in the historical and own-block kernels."""
    import numpy as np
    hist = own = pre = 0
    for L in seqlens:
        t = np.arange(L, dtype=np.int64)
        c = t // B
        dense = (c < k) if route else np.zeros(L, dtype=bool)
        pre += int((t + 1)[dense].sum())
        own += int((t % B + 1)[~dense].sum())
        hist += int((B * np.minimum(k - 1, c))[~dense].sum())
    return H * hist, H * own, H * pre


# tile policy of the library's attention grids (launch.h): resident
# historical tiles when K and V^T of a block fit in 128 KiB of LDS, else
# 32-query columns on 8 waves (B >= 1024) or 4; own-block tiles of 4 waves
RESIDENT_LDS_BYTES = 128 * 1024


def issued_pairs(list_lengths, seqlens, B, d, k=0, route=False):
    """(query, key) pairs the attention kernels put through the MFMA units,
    padding included, per head for own and prefix: historical rows rounded up
    to the rows a tile computes (32 per wave pass in resident tiles, whole
    tiles otherwise) against all B keys of the block; own-block tiles of 128
    query columns against 64-key chunks up to their last query (blocks of the
    dense prefix skipped when route); and, when route, the dense prefix
    launch's tiles over the first k B positions against 64-key chunks up to
    their last query.  list_lengths holds the number of historical selections
    of each (head, KV block), prefix rows left out when route."""
    import numpy as np
    n = np.asarray(list_lengths, dtype=np.int64)
    if B * d * 4 <= RESIDENT_LDS_BYTES:
        rows = (n + 31) // 32 * 32
    else:
        tq = mfma_tile_q(B)
        rows = (n + tq - 1) // tq * tq
    hist = int(rows.sum()) * B
    own = pre = 0
    span = min(max(seqlens), k * B) if route else 0
    tqp = mfma_tile_q(span) if route else 0
    for L in seqlens:
        for blo in range(0, L, B):
            if route and blo // B < k:
                continue
            blen = min(B, L - blo)
            for q_lo in range(0, blen, 128):
                q_hi = min(q_lo + 128, blen)
                own += 128 * 64 * ((q_hi + 63) // 64)
        if route:
            for q_lo in range(0, min(L, span), tqp):
                q_hi = min(q_lo + tqp, L, span)
                pre += tqp * 64 * ((q_hi + 63) // 64)
    return hist, own, pre


def list_lengths(torch, idx, seqlens, B, min_c=0):
    """Historical selections per (head, global KV block) of block_idx
    [T, H, k] (entries below the query's own block), of the rows whose own
    block is min_c or later."""
    T, H, _ = idx.shape
    dev = idx.device
    starts, blocks = [0], [0]
    for L in seqlens:
        starts.append(starts[-1] + L)
        blocks.append(blocks[-1] + (L + B - 1) // B)
    nb = blocks[-1]
    cu = torch.tensor(starts, dtype=torch.int64, device=dev)
    cb = torch.tensor(blocks, dtype=torch.int64, device=dev)
    tok = torch.arange(T, dtype=torch.int64, device=dev)
    seq = torch.searchsorted(cu[1:], tok, right=True)
    c = (tok - cu[seq]) // B
    counts = torch.zeros(H * nb, dtype=torch.int64, device=dev)
    for h in range(H):  # one head at a time bounds the temporaries
        row = idx[:, h, :].to(torch.int64)
        valid = (row >= 0) & (row < c[:, None]) & (c[:, None] >= min_c)
        key = h * nb + cb[seq][:, None] + row
        counts += torch.bincount(key[valid], minlength=H * nb)
    return counts.cpu().numpy()


# sources the historical-attention kernel is built from
HIST_SOURCES = ("attn_mfma.hip", "common.h", "launch.h")


def code_tokens(text):
    """C++ source without comments and with whitespace runs collapsed: a
    change to a comment leaves the code, and with it a counter record, valid."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_sparse_long_03_amd", "csrc", n)) as f:
            h.update(code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE scaled by the copy-kernel calibration),
    if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"attn_hist_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(*HIST_SOURCES):
        return None
    return rec.get("hbm_bytes_per_launch")


# per-worker state of the CPU baseline (set in the parent before forking)
_CPU_JOB = {}


def _cpu_worker(h):
    """The oracle on seeded rows of head h of the bench workload: the head's
    block pooling once (the oracle's pool_keys_head), then row after row the
    oracle's own steps 2-5 (gate scores, causal top-k, attended tokens, exact
    softmax), exactly as moba_reference runs them, until the time budget is
    spent.  BLAS runs one thread.  Returns (rows done, attended pairs,
    pooling seconds, row seconds)."""
    import numpy as np
    from oracle import moba_oracle as mo
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        ctx = None
    j = _CPU_JOB
    q, k, v = (j[n][h] for n in ("q", "k", "v"))  # [T, d] fp32 (exact bf16 values)
    cu = j["cu"]
    B, topk, scale = j["B"], j["topk"], j["scale"]
    rng = np.random.default_rng(2000 + j["index"] * 100 + h)
    ts = np.sort(rng.choice(len(q), size=min(j["rows"], len(q)), replace=False))
    try:
        t0 = time.perf_counter()
        kbar = {}
        for s in range(len(cu) - 1):
            a, L = int(cu[s]), int(cu[s + 1] - cu[s])
            kbar[s] = mo.pool_keys_head(k[a:a + L], L, B)
        t_pool = time.perf_counter() - t0
        done = pairs = 0
        t0 = time.perf_counter()
        for t in ts:
            s = int(np.searchsorted(cu, t, side="right") - 1)
            a, L = int(cu[s]), int(cu[s + 1] - cu[s])
            tl = int(t) - a
            c = tl // B
            sc = mo.gate_scores_row(q[t], kbar[s], c)
            idx, _, _ = mo.select_row(sc, c, topk)
            J = mo.attended_tokens(idx, tl, B)
            mo.attend_row(q[t], k[a:a + L], v[a:a + L], J, scale)
            done += 1
            pairs += len(J)
            if time.perf_counter() - t0 > j["seconds"]:
                break
        t_rows = time.perf_counter() - t0
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return done, pairs, t_pool, t_rows


def cpu_baseline(x, w, rows_target, seconds):
    """The fp64 oracle on the host's cores: P = len(os.sched_getaffinity(0))
    forked worker processes (capped at the head count and at the 16 cores a
    one-GPU share of the host holds), worker i taking head
    i: it pools the head's keys once and then runs seeded query rows through
    the oracle's per-row steps for about `seconds`.  Rates are the summed
    attended-pair flops (4d per pair) over the wall time of the row phase."""
    import multiprocessing as mp
    import numpy as np
    P = max(1, min(len(os.sched_getaffinity(0)), 16, w.heads))
    heads = list(range(P))
    # host copies of the workers' heads only (bf16 values, exact in fp32)
    _CPU_JOB.clear()
    for n in ("q", "k", "v"):
        _CPU_JOB[n] = {h: x[n][:, h, :].float().cpu().numpy() for h in heads}
    _CPU_JOB.update(cu=np.asarray(x["cu_seqlens"], dtype=np.int64), B=w.block_size,
                    topk=w.topk, scale=w.scale, index=w.index, rows=rows_target,
                    seconds=seconds)
    t0 = time.perf_counter()
    # fork (no exec): the workers inherit the arrays and never touch the GPU
    with mp.get_context("fork").Pool(P) as pool:
        res = pool.map(_cpu_worker, heads)
    wall = time.perf_counter() - t0
    _CPU_JOB.clear()
    done = sum(r[0] for r in res)
    pairs = sum(r[1] for r in res)
    t_pool = max(r[2] for r in res)
    t_rows = max(r[3] for r in res)
    flops = 4.0 * w.head_dim * pairs
    per_row_s = t_rows * P / max(done, 1)  # one core's time per row
    return {
        "value": flops / t_rows / 1e12,
        "unit": "TFLOP/s",
        "cores": P,
        "kind": "oracle",
        "sample": (f"{done} seeded query rows over heads 0..{P - 1} of the {w.name} workload, "
                   f"one head per worker process ({P} processes, BLAS 1 thread each); each "
                   f"worker pools its head's keys once ({t_pool:.1f} s) and then runs rows "
                   f"through the oracle's per-row steps for {seconds:.0f} s; fp64 NumPy"),
        "seconds": t_rows,
        "wall_seconds": wall,
        "pool_seconds": t_pool,
        "per_row_ms": per_row_s * 1e3,
        "extrapolated_layer_s": (t_pool * w.heads + per_row_s * w.total_tokens * w.heads) / P,
    }


def measure(torch, inputs, moba, w, dev, steps, warmup, dense_reps, keep=False, gate="mean"):
    """Times `steps` MoBA layers (pool, gate + top-k, attention) on one
    workload after `warmup` untimed ones, then the library's own dense causal
    kernel `dense_reps` times.  `gate` picks the routing: "mean" (the MoBA
    gate on mean-pooled keys), "minmax" (min/max pooled keys), "window" or
    "sinkN" (static routing with N initial blocks).  Returns the inputs (if
    keep), the geometry, ms per step, per-stage HIP-event totals, dense ms and
    dense stages."""
    sink = 0 if gate == "window" else int(gate[4:]) if gate.startswith("sink") else None
    if sink is None and gate not in ("mean", "minmax"):
        raise SystemExit(f"unknown gate {gate!r}")
    print(f"[bench] workload {w.name}: {w.seqlens} H{w.heads} d{w.head_dim} B{w.block_size} "
          f"k{w.topk} gate {gate}", file=sys.stderr, flush=True)
    x = inputs.make_inputs(w, device=dev)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    H, d = w.heads, w.head_dim
    dt = moba.MOBA_BF16 if w.dtype == "bf16" else moba.MOBA_F32
    kbar = torch.empty((geom.total_blocks, H, 2 if gate == "minmax" else 1, d),
                       dtype=torch.float32, device=dev)
    kbar3 = torch.empty((H, 3, d // 16, geom.total_blocks, 16), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((geom.total_tokens, H, w.topk), dtype=torch.int32, device=dev)
    out = torch.empty_like(x["q"])
    lse = torch.empty((geom.total_tokens, H), dtype=torch.float32, device=dev)
    ws = torch.empty(moba.moba_attn_workspace_bytes(dt, geom.total_tokens, geom.total_blocks,
                                                    H, d, w.block_size, w.topk),
                     dtype=torch.uint8, device=dev)
    q, k, v = x["q"], x["k"], x["v"]

    def step():
        if gate == "mean":
            pooled = moba.moba_pool_keys(k, geom, kbar=kbar, kbar3=kbar3)
            moba.moba_gate_topk(q, pooled, geom, w.topk, block_idx=idx)
        elif gate == "minmax":
            moba.moba_pool_minmax(k, geom, kminmax=kbar)
            moba.moba_gate_topk_minmax(q, kbar, geom, w.topk, block_idx=idx)
        else:
            moba.moba_static_select(geom, H, w.topk, sink, block_idx=idx)
        moba.moba_attn_fwd(q, k, v, geom, w.topk, idx, w.scale, out=out, lse=lse, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # The timed region runs with no per-launch profiler attached: its two
    # events per kernel cost a few microseconds each, which is 15% of an 8K
    # step.  One event pair per step on the stream the library launches on
    # gives the median and minimum next to the mean of the wall clock.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        step()
        ev[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    per_step = sorted(a.elapsed_time(b) for a, b in ev)
    step_stats = {"mean_ms": ms_step, "median_ms": per_step[len(per_step) // 2],
                  "min_ms": per_step[0], "max_ms": per_step[-1]}
    # per-kernel times: the same number of steps again, each launch
    # bracketed by HIP events on its stream
    prof = moba.Profiler().attach()
    prof.reset()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kern = prof.summary()
    prof.reset()
    print(f"[bench] {w.name}: moba {ms_step:.3f} ms/step (median {step_stats['median_ms']:.3f},"
          f" min {step_stats['min_ms']:.3f})", file=sys.stderr, flush=True)

    # the library's own dense causal kernel on the same inputs
    del ws
    dense_ms = None
    rec_dense_stages = {}
    if dense_reps > 0:
        dws = torch.empty(moba.moba_dense_workspace_bytes(dt, geom.total_tokens,
                                                          geom.total_blocks, H, d, w.block_size),
                          dtype=torch.uint8, device=dev)
        dout = torch.empty_like(q)
        dlse = torch.empty_like(lse)
        moba.moba_dense_causal_fwd(q, k, v, geom, w.scale, out=dout, lse=dlse, workspace=dws)
        torch.cuda.synchronize()
        prof.detach()  # timed like the MoBA steps, then once more for its stages
        t0 = time.perf_counter()
        for _ in range(dense_reps):
            moba.moba_dense_causal_fwd(q, k, v, geom, w.scale, out=dout, lse=dlse, workspace=dws)
        torch.cuda.synchronize()
        dense_ms = (time.perf_counter() - t0) * 1e3 / dense_reps
        prof.attach()
        prof.reset()
        moba.moba_dense_causal_fwd(q, k, v, geom, w.scale, out=dout, lse=dlse, workspace=dws)
        torch.cuda.synchronize()
        rec_dense_stages = prof.summary()
        del dout, dws
        print(f"[bench] {w.name}: dense {dense_ms:.1f} ms", file=sys.stderr, flush=True)
    prof.detach()
    prof.close()
    route = prefix_route(list(w.seqlens), w.block_size, w.topk, H, w.dtype)
    lengths = (list_lengths(torch, idx, w.seqlens, w.block_size, w.topk if route else 0)
               if w.dtype == "bf16" else None)
    del kbar, kbar3, idx, out, lse
    if not keep:
        del x, q, k, v
        x = None
        torch.cuda.empty_cache()
    return x, geom, ms_step, kern, dense_ms, rec_dense_stages, lengths, step_stats


def measured_peaks(torch, moba, dev):
    """The rates this GPU sustains, to set next to the published peaks: the
    library's bf16 MFMA probes (two waves per SIMD; fixed register operands,
    random register operands, random operands with B read from LDS) and a
    plain 4 GiB device copy (read + write), each timed with events on the
    current stream after a warmup."""
    wg = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(wg * 256, dtype=torch.float32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    iters = 1000000
    rates = {}
    for operands, key in ((0, "mfma_bf16_tflops"), (1, "mfma_bf16_random_tflops"),
                          (2, "mfma_bf16_random_lds_tflops")):
        moba.probe_mfma_rate(wg, 1000, sink, operands)
        e0.record()
        flops = moba.probe_mfma_rate(wg, iters, sink, operands)
        e1.record()
        torch.cuda.synchronize()
        rates[key] = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    n = 1 << 30
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0.record()
    for _ in range(3):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy = 3 * 2 * 4 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst, sink
    torch.cuda.empty_cache()
    return {**rates, "hbm_copy_gbps": copy,
            "spec_mfma_bf16_tflops": PEAK_BF16_TFLOPS, "spec_hbm_gbps": PEAK_HBM_GBPS,
            "method": f"moba_probe_mfma_rate: {wg} workgroups x 4 waves x 4 independent chains "
                      f"x {iters} v_mfma_f32_32x32x16_bf16, on one fixed low-entropy operand "
                      "pair, on random bf16 operands cycling through 8 register sets, and on "
                      "random operands with B read from LDS per product; copy: 3 x torch copy "
                      "of 4 GiB fp32 (bytes read + written)"}


def measure_streamed(torch, inputs, moba, w, dev, head_chunk):
    """One layer of a head-streamed workload (w.head_group heads at a time,
    moba.forward_head_streamed): each group's Q/K/V are drawn on the device,
    then the group's pool, gate and sparse attention run and its output stays
    in device memory.  The layer time is the sum of the groups' forward times
    (HIP events around each group's calls, the input draws excluded); the
    wall time including the draws is reported beside it."""
    print(f"[bench] workload {w.name}: {w.seqlens} H{w.heads} in groups of {w.head_group}, "
          f"head_chunk {head_chunk}", file=sys.stderr, flush=True)
    geom = moba.Geometry.make(inputs.cu_seqlens_of(w.seqlens), w.block_size, dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_groups, outs = [], {}

    def source(h0, h1):
        x = inputs.make_head_group(w, h0 // w.head_group, device=dev)
        torch.cuda.synchronize()
        e0.record()
        return x["q"], x["k"], x["v"]

    def on_group(h0, out, lse, idx):
        e1.record()
        torch.cuda.synchronize()
        t_groups.append(e0.elapsed_time(e1))
        outs[h0] = (out, lse)  # the layer's output stays resident, group by group
        print(f"[bench] {w.name}: heads {h0}..{h0 + out.shape[1] - 1} {t_groups[-1]:.1f} ms",
              file=sys.stderr, flush=True)

    prof = moba.Profiler().attach()
    prof.reset()
    t0 = time.perf_counter()
    moba.forward_head_streamed(source, geom, w.heads, w.head_group, w.topk, w.scale,
                               head_chunk=head_chunk, on_group=on_group)
    wall = (time.perf_counter() - t0) * 1e3
    kern = prof.summary()
    prof.detach()
    prof.close()
    assert all(bool(torch.isfinite(o[1]).all()) for o in outs.values())
    del outs
    torch.cuda.empty_cache()
    return sum(t_groups), wall, t_groups, kern


def measure_bwd(torch, inputs, moba, w, dev, steps, warmup):
    """Times `steps` backward passes (moba_attn_bwd: dq, dk, dv for one
    upstream gradient) of one forward's selections, after `warmup`.  Returns
    ms per step and per-stage HIP-event totals."""
    print(f"[bench] workload {w.name}: backward", file=sys.stderr, flush=True)
    x = inputs.make_inputs(w, device=dev)
    geom = moba.Geometry.make(x["cu_seqlens"], w.block_size, dev)
    out, lse, idx = moba.forward(x["q"], x["k"], x["v"], geom, w.topk, w.scale)
    torch.cuda.empty_cache()
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    dout = torch.empty_like(x["q"])
    dout.copy_(torch.randn(x["q"].shape, generator=gen, device=dev, dtype=torch.float32))
    torch.cuda.empty_cache()
    H, d = w.heads, w.head_dim
    dq, dk, dv = (torch.empty(x["q"].shape, dtype=torch.float32, device=dev) for _ in range(3))
    ws = torch.empty(moba.moba_attn_bwd_workspace_bytes(moba.MOBA_BF16, geom.total_tokens,
                                                        geom.total_blocks, H, d, w.block_size,
                                                        w.topk), dtype=torch.uint8, device=dev)

    def step():
        moba.moba_attn_bwd(x["q"], x["k"], x["v"], out, dout, lse, geom, w.topk, idx, w.scale,
                           dq=dq, dk=dk, dv=dv, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    prof = moba.Profiler().attach()
    prof.reset()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    kern = prof.summary()
    prof.detach()
    prof.close()
    print(f"[bench] {w.name}: backward {ms:.3f} ms/step", file=sys.stderr, flush=True)
    del x, out, lse, idx, dout, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return ms, kern


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="1m")
    ap.add_argument("--dense-reps", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="seeded query rows per worker (head), bounded by --cpu-seconds")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--also", default="8k,32k,varlen,10m32,1m:bwd,1m:minmax,1m:window,1m:sink1",
                    help="comma-separated extra workloads reported under other_workloads "
                         "(ms/layer, TFLOP/s, dense, speedup); NAME:minmax uses the min/max "
                         "pooled gate, NAME:window or NAME:sinkN static routing, NAME:bwd the "
                         "backward pass; empty for none")
    ap.add_argument("--also-steps", type=int, default=20,
                    help="timed steps of the extra workloads (3 above 256K tokens)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured MFMA / copy rates reported next to the spec peaks")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 4 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the library runs on one GPU; MoBA shards by head, and "
                          "no multi-GPU path is implemented", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from block_sparse_long_03_amd import inputs, moba

    if args.copy_probe:
        # a plain copy of known size: rocprofv3 FETCH_SIZE / WRITE_SIZE of this
        # kernel calibrate the counters against 4 GiB read + 4 GiB written
        n = 1 << 30
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": 4 * n, "launches": 3}))
        return

    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS[args.workload]
    x, geom, ms_step, kern, dense_ms, rec_dense_stages, lengths, step_stats = measure(
        torch, inputs, moba, w, dev, args.steps, args.warmup, args.dense_reps, keep=True)
    H, d = w.heads, w.head_dim
    q = x["q"]
    pairs, _, _ = attended_pairs(w.seqlens, w.block_size, w.topk, H)
    route = prefix_route(list(w.seqlens), w.block_size, w.topk, H, w.dtype)
    hist_p, own_p, pre_p = attended_pairs_by_kernel(w.seqlens, w.block_size, w.topk, H, route)
    flops = 4.0 * d * pairs
    eff_tflops = flops / (ms_step * 1e-3) / 1e12
    stages = {name: {"launches_per_step": n / args.steps, "ms_per_step": ms / args.steps}
              for name, (n, ms) in kern.items()}

    n_h, ms_h = kern.get("attn_hist", (0, 0.0))
    avg_h = ms_h / max(n_h, 1)
    hist_flops = 4.0 * d * hist_p
    achieved = hist_flops / (avg_h * 1e-3) / 1e12 if avg_h > 0 else 0.0
    traffic = traffic_from_profiles(w.name)
    roofline = {"kernel": "attn_hist (attn_mfma_kernel, historical blocks)", "bound": "mfma",
                "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                "avg_launch_ms": avg_h, "flops_per_launch": hist_flops}
    n_o, ms_o = kern.get("attn_own", (0, 0.0))
    own_tflops = 4.0 * d * own_p / (ms_o / max(n_o, 1) * 1e-3) / 1e12 if ms_o > 0 else None
    n_x, ms_x = kern.get("attn_prefix", (0, 0.0))
    prefix_tflops = 4.0 * d * pre_p / (ms_x / max(n_x, 1) * 1e-3) / 1e12 if ms_x > 0 else None
    # the attention kernels together (historical, own block, dense prefix):
    # 4d flops per attended pair over their summed time
    t_attn = (avg_h + (ms_o / max(n_o, 1) if ms_o > 0 else 0.0)
              + (ms_x / max(n_x, 1) if ms_x > 0 else 0.0))
    attn_frac = (flops / (t_attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS) if t_attn > 0 else None
    mfma_issued = None
    if lengths is not None and t_attn > 0:
        ih, io, ip = issued_pairs(lengths, w.seqlens, w.block_size, d, w.topk, route)
        io *= H
        ip *= H
        mfma_issued = {
            "historical_pairs": ih, "own_pairs": io, "prefix_pairs": ip,
            "flops": 4.0 * d * (ih + io + ip),
            "tflops_over_attention_time": 4.0 * d * (ih + io + ip) / (t_attn * 1e-3) / 1e12,
            "algorithmic_share": (hist_p + own_p + pre_p) / (ih + io + ip),
        }
    n_g, ms_g = kern.get("gate_topk", (0, 0.0))
    gate_bytes = (geom.total_tokens * H * d * q.element_size() + geom.total_tokens * H * w.topk * 4
                  + geom.total_blocks * H * d * 4)
    gate_gbps = gate_bytes / (ms_g / max(n_g, 1) * 1e-3) / 1e9 if ms_g > 0 else None
    n_p, ms_p = kern.get("pool_keys", (0, 0.0))
    pool_bytes = geom.total_tokens * H * d * q.element_size() + geom.total_blocks * H * d * 4
    pool_gbps = pool_bytes / (ms_p / max(n_p, 1) * 1e-3) / 1e9 if ms_p > 0 else None

    rec = {
        "metric": METRIC,
        "value": eff_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V generated on the GPU)",
        "config": {"workload": w.name, "seqlens": list(w.seqlens), "heads": H, "head_dim": d,
                   "block_size": w.block_size, "topk": w.topk,
                   "sparsity_last_query": 1 - w.topk * w.block_size / max(w.seqlens)},
        "ms_per_layer": ms_step,
        "step_ms": step_stats,
        "attended_pairs": pairs,
        "dense_ms": dense_ms,
        "dense_tflops": (4.0 * d * dense_pairs(w.seqlens, H) / (dense_ms * 1e-3) / 1e12
                         if dense_ms else None),
        "speedup_vs_dense": (dense_ms / ms_step) if dense_ms else None,
        "stages": stages,
        "dense_stages": {n: {"launches": c, "ms": t} for n, (c, t) in rec_dense_stages.items()},
        "own_block_tflops": own_tflops,
        # rows of the first k blocks through the dense kernel (attn_prefix)
        "dense_prefix_route": route,
        "prefix_tflops": prefix_tflops,
        "attention_mfma_frac": attn_frac,
        "pool_gbps": pool_gbps,
        "pool_hbm_frac": pool_gbps / PEAK_HBM_GBPS if pool_gbps else None,
        # gate + top-k: algorithmic bytes (Q read, block_idx written, kbar read once)
        "gate_gbps": gate_gbps,
        "gate_hbm_frac": gate_gbps / PEAK_HBM_GBPS if gate_gbps else None,
        # what the attention kernels put through the MFMA units, tile padding included
        "mfma_issued": mfma_issued,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(x, w, args.cpu_rows, args.cpu_seconds)
    del x, q
    torch.cuda.empty_cache()
    others = {}
    for name in [n for n in args.also.split(",") if n and n != w.name]:
        wname, _, gate = name.partition(":")
        gate = gate or "mean"
        wo = inputs.WORKLOADS[wname]
        if wo.head_group > 0:
            ms_s, wall_s, per_group, kern_s = measure_streamed(torch, inputs, moba, wo, dev,
                                                               head_chunk=wo.head_group // 2)
            pairs_s, _, _ = attended_pairs(wo.seqlens, wo.block_size, wo.topk, wo.heads)
            hist_s = attended_pairs_by_kernel(
                wo.seqlens, wo.block_size, wo.topk, wo.heads,
                prefix_route(list(wo.seqlens), wo.block_size, wo.topk, wo.head_group, wo.dtype))[0]
            n_hs, ms_hs = kern_s.get("attn_hist", (0, 0.0))
            dense_x = (dense_ms * dense_pairs(wo.seqlens, wo.heads) / dense_pairs(w.seqlens, H)
                       if dense_ms else None)
            others[name] = {
                "config": {"workload": wname, "gate": "mean", "seqlens": list(wo.seqlens),
                           "heads": wo.heads, "head_dim": wo.head_dim,
                           "block_size": wo.block_size, "topk": wo.topk,
                           "head_group": wo.head_group, "head_chunk": wo.head_group // 2},
                "steps": 1,
                "ms_per_layer": ms_s,
                "wall_ms_with_input_draws": wall_s,
                "group_ms": per_group,
                "effective_tflops": 4.0 * wo.head_dim * pairs_s / (ms_s * 1e-3) / 1e12,
                "attn_hist_tflops": (4.0 * wo.head_dim * hist_s / (ms_hs * 1e-3) / 1e12
                                     if ms_hs else None),
                # the dense kernel at 10M x 32 heads would run for minutes: its time
                # is the headline workload's measured dense rate per causal pair,
                # scaled by the causal pairs of this layer
                "dense_ms_extrapolated": dense_x,
                "speedup_vs_dense_extrapolated": (dense_x / ms_s) if dense_x else None,
                "stages_ms": {n: t for n, (c, t) in kern_s.items()},
            }
            continue
        if gate == "bwd":
            steps_b = min(args.also_steps, 3) if wo.total_tokens > (1 << 18) else args.also_steps
            ms_b, kern_b = measure_bwd(torch, inputs, moba, wo, dev, steps_b, max(1, args.warmup))
            pairs_b = attended_pairs(wo.seqlens, wo.block_size, wo.topk, wo.heads)[0]
            d_b = wo.head_dim
            st_b = {n: t / steps_b for n, (c, t) in kern_b.items()}
            others[name] = {
                "config": {"workload": wname, "pass": "backward (dq, dk, dv)",
                           "seqlens": list(wo.seqlens), "heads": wo.heads, "head_dim": d_b,
                           "block_size": wo.block_size, "topk": wo.topk},
                "steps": steps_b,
                "ms_per_layer": ms_b,
                # algorithmic: 5 products of 2d flops per attended pair
                "effective_tflops": 10.0 * d_b * pairs_b / (ms_b * 1e-3) / 1e12,
                # issued: S and dP are formed in both kernels (7 products)
                "issued_tflops": 14.0 * d_b * pairs_b / (ms_b * 1e-3) / 1e12,
                "bwd_kv_tflops": (8.0 * d_b * pairs_b / (st_b["bwd_kv"] * 1e-3) / 1e12
                                  if st_b.get("bwd_kv") else None),
                "bwd_q_tflops": (6.0 * d_b * pairs_b / (st_b["bwd_q"] * 1e-3) / 1e12
                                 if st_b.get("bwd_q") else None),
                "stages_ms": st_b,
            }
            continue
        steps_o = args.also_steps if wo.total_tokens <= (1 << 18) else min(args.also_steps, 3)
        # gate variants of the headline workload reuse its dense time; above
        # 4M tokens the dense kernel (minutes) is not run: its time is
        # extrapolated from the headline's measured dense rate per causal pair
        big = wo.total_tokens > (1 << 22)
        dense_reps_o = 2 if (args.dense_reps and wname != w.name and not big) else 0
        _, _, ms_o2, kern_o, dense_o, _, _, stats_o = measure(
            torch, inputs, moba, wo, dev, steps_o, max(1, args.warmup), dense_reps_o, gate=gate)
        if dense_o is None and wname == w.name:
            dense_o = dense_ms
        pairs_o, _, _ = attended_pairs(wo.seqlens, wo.block_size, wo.topk, wo.heads)
        dense_x = None
        if big and dense_ms:
            dense_x = dense_ms * dense_pairs(wo.seqlens, wo.heads) / dense_pairs(w.seqlens, H)
        n_ho, ms_ho = kern_o.get("attn_hist", (0, 0.0))
        hist_o = attended_pairs_by_kernel(
            wo.seqlens, wo.block_size, wo.topk, wo.heads,
            prefix_route(list(wo.seqlens), wo.block_size, wo.topk, wo.heads, wo.dtype))[0]
        others[name] = {
            "config": {"workload": wname, "gate": gate,
                       "seqlens": list(wo.seqlens), "heads": wo.heads, "head_dim": wo.head_dim,
                       "block_size": wo.block_size, "topk": wo.topk},
            "steps": steps_o,
            "attn_hist_tflops": (4.0 * wo.head_dim * hist_o / (ms_ho / n_ho * 1e-3) / 1e12
                                 if n_ho else None),
            "ms_per_layer": ms_o2,
            "step_ms": stats_o,
            "effective_tflops": 4.0 * wo.head_dim * pairs_o / (ms_o2 * 1e-3) / 1e12,
            "dense_ms": dense_o,
            "speedup_vs_dense": (dense_o / ms_o2) if dense_o else None,
            "dense_ms_extrapolated": dense_x,
            "speedup_vs_dense_extrapolated": (dense_x / ms_o2) if dense_x else None,
            "stages_ms": {n: t / steps_o for n, (c, t) in kern_o.items()},
        }
    rec["other_workloads"] = others
    if not args.no_peaks:
        print("[bench] measured peaks", file=sys.stderr, flush=True)
        pk = measured_peaks(torch, moba, dev)
        rec["measured_peaks"] = pk
        rec["roofline"]["frac_of_measured_peak"] = rec["roofline"]["achieved"] / pk["mfma_bf16_tflops"]
        rec["roofline"]["frac_of_measured_random_lds_peak"] = (
            rec["roofline"]["achieved"] / pk["mfma_bf16_random_lds_tflops"])
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
