"""Helpers that compare the HIP library's results with the CPU oracle.

Acceptance (bf16 inputs, fp32 accumulation): block selections bit-exact
except on rows the oracle flags as near-ties (k-1-th and k-th largest past
scores within 1e-5 relative), where the GPU's selection must be a valid
causal top-k under the oracle's fp64 scores and is then used for that row's
expected output; outputs max abs error <= 1e-2 and relative L2 <= 5e-3;
log-sum-exp within 1e-3 absolute.  fp32 inputs: 1e-4 on outputs and lse.
"""

from __future__ import annotations

import json
import os

import numpy as np
import torch

from oracle import moba_oracle as mo

BF16_TOL = dict(max_abs=1e-2, rel_l2=5e-3, lse_abs=1e-3)
F32_TOL = dict(max_abs=1e-4, rel_l2=1e-5, lse_abs=1e-4)


def host_head(x, h):
    """[T, H, d] device tensor -> [T, 1, d] fp32 numpy (exact for bf16)."""
    return x[:, h:h + 1, :].float().cpu().numpy()


def check_selection(q_h, k_h, cu, B, topk, rows_h, idx_gpu_rows):
    """Compares GPU selections of rows (token, 0) of one head with the oracle.
    Returns dict(ref=oracle dict, use_idx=idx to attend with, n_near, n_mismatch)."""
    ref = mo.gate_reference(q_h, k_h, cu, B, topk, rows=rows_h)
    mism = np.nonzero(np.any(ref["idx"] != idx_gpu_rows, axis=1))[0]
    use_idx = ref["idx"].copy()
    bad = []
    for r in mism:
        if ref["near_tie"][r] and mo.selection_is_valid(q_h, k_h, cu, B, topk, rows_h[r],
                                                        idx_gpu_rows[r]):
            use_idx[r] = idx_gpu_rows[r]
        else:
            bad.append(r)
    assert not bad, (f"{len(bad)} rows select different blocks without a near-tie, e.g. "
                     f"row {rows_h[bad[0]].tolist()}: gpu {idx_gpu_rows[bad[0]].tolist()} "
                     f"oracle {ref['idx'][bad[0]].tolist()} gap {ref['gap'][bad[0]]}")
    return dict(ref=ref, use_idx=use_idx, n_near=int(ref["near_tie"].sum()),
                n_mismatch=len(mism))


def error_stats(o_gpu, o_ref, lse_gpu, lse_ref):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    diff = o_gpu - o_ref
    return dict(max_abs=float(np.abs(diff).max()) if diff.size else 0.0,
                rel_l2=float(np.linalg.norm(diff) / max(np.linalg.norm(o_ref), 1e-300)),
                lse_abs=float(np.abs(np.asarray(lse_gpu, np.float64) - lse_ref).max())
                if diff.size else 0.0)


def emit(stats):
    """Prints the error statistics of the running test and, when the
    environment names a file in MOBA_PARITY_REPORT, appends them there as one
    JSON line."""
    name = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    line = json.dumps({"test": name, **stats})
    print("[stats]", line, flush=True)
    path = os.environ.get("MOBA_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


def assert_within(stats, tol, what=""):
    emit(stats)
    for key in ("max_abs", "rel_l2", "lse_abs"):
        assert stats[key] <= tol[key], f"{what}: {key} {stats[key]:.3e} > {tol[key]:.1e} ({stats})"


def check_moba_rows(q, k, v, cu, B, topk, scale, out, lse, idx, rows, tol):
    """Full check of MoBA output rows (global token, head) against the oracle.
    q, k, v, out, lse, idx are device tensors."""
    stats_all = []
    n_near = n_mis = 0
    for h in np.unique(rows[:, 1]):
        th = rows[rows[:, 1] == h, 0]
        rows_h = np.stack([th, np.zeros_like(th)], axis=1)
        q_h, k_h, v_h = host_head(q, h), host_head(k, h), host_head(v, h)
        tt = torch.as_tensor(th, device=out.device)
        idx_g = idx[tt, int(h), :].cpu().numpy().astype(np.int64)
        sel = check_selection(q_h, k_h, cu, B, topk, rows_h, idx_g)
        n_near += sel["n_near"]
        n_mis += sel["n_mismatch"]
        o_ref, lse_ref = mo.attend_given_selection(q_h, k_h, v_h, cu, B, sel["use_idx"], scale,
                                                   rows_h)
        o_g = out[tt, int(h), :].float().cpu().numpy()
        l_g = lse[tt, int(h)].cpu().numpy()
        stats_all.append((o_g, o_ref, l_g, lse_ref))
    o_g = np.concatenate([s[0] for s in stats_all])
    o_r = np.concatenate([s[1] for s in stats_all])
    l_g = np.concatenate([s[2] for s in stats_all])
    l_r = np.concatenate([s[3] for s in stats_all])
    st = error_stats(o_g, o_r, l_g, l_r)
    st.update(n_near=n_near, n_mismatch=n_mis, rows=len(rows))
    assert_within(st, tol, "moba")
    return st


def check_idx_all_rows(q, k, cu, B, topk, idx, heads=None):
    """Selections of every token of the given heads (default all)."""
    T, H, _ = q.shape
    n_near = n_mis = 0
    for h in (range(H) if heads is None else heads):
        q_h, k_h = host_head(q, h), host_head(k, h)
        rows_h = np.stack([np.arange(T), np.zeros(T, dtype=np.int64)], axis=1)
        idx_g = idx[:, h, :].cpu().numpy().astype(np.int64)
        sel = check_selection(q_h, k_h, cu, B, topk, rows_h, idx_g)
        n_near += sel["n_near"]
        n_mis += sel["n_mismatch"]
    st = dict(n_near=n_near, n_mismatch=n_mis, rows=int(T) * (H if heads is None else len(heads)))
    emit(st)
    return st


def check_idx_rows(q, k, cu, B, topk, idx, rows):
    """Selections of the given (global token, head) rows, head by head."""
    n_near = n_mis = 0
    for h in np.unique(rows[:, 1]):
        th = rows[rows[:, 1] == h, 0]
        rows_h = np.stack([th, np.zeros_like(th)], axis=1)
        q_h, k_h = host_head(q, int(h)), host_head(k, int(h))
        tt = torch.as_tensor(th, device=idx.device)
        idx_g = idx[tt, int(h), :].cpu().numpy().astype(np.int64)
        sel = check_selection(q_h, k_h, cu, B, topk, rows_h, idx_g)
        n_near += sel["n_near"]
        n_mis += sel["n_mismatch"]
    st = dict(n_near=n_near, n_mismatch=n_mis, rows=len(rows))
    emit(st)
    return st
