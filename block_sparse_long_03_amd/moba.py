"""Python binding of libmoba.so (ctypes).

Argument marshalling only: torch provides device memory and the current HIP
stream, every computation runs in the library's HIP kernels.  The entry points
carry the C names of ``include/moba.h``; ``forward`` and ``dense`` chain them.

Loading fails loudly when the library has not been built (there is no
fallback of any kind).
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import NamedTuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoba.so")

MOBA_OK = 0
MOBA_ERR_INVALID_ARG = -1
MOBA_ERR_UNSUPPORTED = -2
MOBA_ERR_WORKSPACE_TOO_SMALL = -3
MOBA_ERR_HIP = -4
MOBA_F32 = 0
MOBA_BF16 = 1
# the MOBA_API_VERSION of include/moba.h these bindings are written for
API_VERSION = 6

EXPORTS = ["moba_api_version", "moba_status_str", "moba_last_hip_error", "moba_pool_keys",
           "moba_gate_topk", "moba_pool_minmax", "moba_gate_topk_minmax", "moba_static_select",
           "moba_attn_workspace_bytes", "moba_attn_fwd", "moba_attn_fwd_static",
           "moba_attn_bwd_workspace_bytes", "moba_attn_bwd",
           "moba_dense_workspace_bytes", "moba_dense_causal_fwd", "moba_profiler_create",
           "moba_profiler_attach", "moba_profiler_reset", "moba_profiler_read",
           "moba_profiler_names", "moba_profiler_destroy", "moba_probe_mfma_rate"]

_lib = None


class MobaError(RuntimeError):
    def __init__(self, fn, status, hip_error=0):
        self.status = status
        self.hip_error = hip_error
        name = lib().moba_status_str(status).decode()
        extra = f" (hip error {hip_error})" if status == MOBA_ERR_HIP else ""
        super().__init__(f"{fn} failed: {name}{extra}")


def lib():
    """Loads libmoba.so once (after torch, so that both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_sparse_long_03_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    geo = [vp, vp, i32, i32, i32, i32, i32, i32, i32]  # cu_seqlens .. block_size
    L.moba_api_version.restype = i32
    L.moba_api_version.argtypes = []
    L.moba_status_str.restype = ctypes.c_char_p
    L.moba_status_str.argtypes = [i32]
    L.moba_last_hip_error.restype = i32
    L.moba_last_hip_error.argtypes = []
    L.moba_pool_keys.restype = i32
    L.moba_pool_keys.argtypes = [vp, i32] + geo + [vp, vp, vp]
    L.moba_gate_topk.restype = i32
    L.moba_gate_topk.argtypes = [vp, i32, vp, vp] + geo + [i32, vp, vp]
    L.moba_pool_minmax.restype = i32
    L.moba_pool_minmax.argtypes = [vp, i32] + geo + [vp, vp]
    L.moba_gate_topk_minmax.restype = i32
    L.moba_gate_topk_minmax.argtypes = [vp, i32, vp] + geo + [i32, vp, vp]
    L.moba_static_select.restype = i32
    L.moba_static_select.argtypes = [vp, vp] + [i32] * 8 + [vp, vp]
    L.moba_attn_workspace_bytes.restype = sz
    L.moba_attn_workspace_bytes.argtypes = [i32] * 8
    L.moba_attn_fwd.restype = i32
    L.moba_attn_fwd.argtypes = [vp, vp, vp, i32] + geo + [i32, vp, f32, vp, i32, vp, i32, vp, sz,
                                                          vp]
    L.moba_attn_fwd_static.restype = i32
    L.moba_attn_fwd_static.argtypes = [vp, vp, vp, i32] + geo + [i32, vp, f32, vp, i32, vp, vp]
    L.moba_attn_bwd_workspace_bytes.restype = sz
    L.moba_attn_bwd_workspace_bytes.argtypes = [i32] * 7
    L.moba_attn_bwd.restype = i32
    L.moba_attn_bwd.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32] + geo + [i32, vp, f32, vp, vp,
                                                                          vp, vp, sz, vp]
    L.moba_dense_workspace_bytes.restype = sz
    L.moba_dense_workspace_bytes.argtypes = [i32] * 6
    L.moba_dense_causal_fwd.restype = i32
    L.moba_dense_causal_fwd.argtypes = [vp, vp, vp, i32] + geo + [f32, vp, i32, vp, vp, sz, vp]
    L.moba_probe_mfma_rate.restype = i32
    L.moba_probe_mfma_rate.argtypes = [i32, i32, i32, vp, vp]
    L.moba_profiler_create.restype = i32
    L.moba_profiler_create.argtypes = [ctypes.POINTER(vp)]
    L.moba_profiler_attach.restype = i32
    L.moba_profiler_attach.argtypes = [vp]
    L.moba_profiler_reset.restype = i32
    L.moba_profiler_reset.argtypes = [vp]
    L.moba_profiler_read.restype = i32
    L.moba_profiler_read.argtypes = [vp, ctypes.c_char_p, ctypes.POINTER(i32),
                                     ctypes.POINTER(ctypes.c_double)]
    L.moba_profiler_names.restype = i32
    L.moba_profiler_names.argtypes = [vp, ctypes.c_char_p, sz]
    L.moba_profiler_destroy.restype = None
    L.moba_profiler_destroy.argtypes = [vp]
    if L.moba_api_version() != API_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI version {L.moba_api_version()}, the bindings "
                           f"expect {API_VERSION}: rebuild it with "
                           "`python -m block_sparse_long_03_amd.build`")
    _lib = L
    return L


def _check(fn, status):
    if status != MOBA_OK:
        raise MobaError(fn, status, lib().moba_last_hip_error())


def _dtype_code(t):
    if t == torch.bfloat16:
        return MOBA_BF16
    if t == torch.float32:
        return MOBA_F32
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


@dataclass
class Geometry:
    """Packed-batch geometry: host scalars plus the device cu_seqlens / cu_blocks."""
    cu_seqlens: torch.Tensor  # int32 [S+1] on the device
    cu_blocks: torch.Tensor   # int32 [S+1] on the device
    num_seqs: int
    total_tokens: int
    max_seqlen: int
    total_blocks: int
    block_size: int

    @staticmethod
    def make(seqlens_or_cu, block_size, device, is_cu=True):
        cu = [int(x) for x in seqlens_or_cu]
        if not is_cu:
            acc = [0]
            for L in cu:
                acc.append(acc[-1] + L)
            cu = acc
        lens = [b - a for a, b in zip(cu[:-1], cu[1:])]
        cb = [0]
        for L in lens:
            cb.append(cb[-1] + (L + block_size - 1) // block_size)
        dev = torch.device(device)
        return Geometry(torch.tensor(cu, dtype=torch.int32, device=dev),
                        torch.tensor(cb, dtype=torch.int32, device=dev),
                        len(lens), cu[-1], max(lens) if lens else 0, cb[-1], block_size)

    def args(self, num_heads, head_dim):
        return [_ptr(self.cu_seqlens), _ptr(self.cu_blocks), self.num_seqs, self.total_tokens,
                self.max_seqlen, self.total_blocks, num_heads, head_dim, self.block_size]


def _qkv_shape(x, geom):
    if x.dim() != 3 or not x.is_contiguous():
        raise ValueError("expected a contiguous [T, H, d] tensor")
    if x.shape[0] != geom.total_tokens:
        raise ValueError("token count does not match the geometry")
    return x.shape[1], x.shape[2]


class PooledKeys(NamedTuple):
    """Output of moba_pool_keys: kbar [NB, H, d] fp32 means and kbar3
    [H, 3, d / 16, NB, 16] bf16, the same means as exact hi + mid + lo terms
    (``kbar3_terms`` gives them as [NB, H, 3, d])."""
    kbar: torch.Tensor
    kbar3: torch.Tensor


def moba_pool_keys(k, geom, kbar=None, kbar3=None, stream=None):
    H, d = _qkv_shape(k, geom)
    if kbar is None:
        kbar = torch.empty((geom.total_blocks, H, d), dtype=torch.float32, device=k.device)
    if kbar3 is None:
        kbar3 = torch.empty((H, 3, d // 16, geom.total_blocks, 16), dtype=torch.bfloat16,
                            device=k.device)
    _check("moba_pool_keys", lib().moba_pool_keys(
        _ptr(k), _dtype_code(k.dtype), *geom.args(H, d), _ptr(kbar), _ptr(kbar3),
        _stream(stream)))
    return PooledKeys(kbar, kbar3)


def kbar3_terms(kbar3, num_heads, head_dim, total_blocks):
    """[NB, H, 3, d] view order of a kbar3 buffer (a copy)."""
    t = kbar3.reshape(num_heads, 3, head_dim // 16, total_blocks, 16)
    return t.permute(3, 0, 1, 2, 4).reshape(total_blocks, num_heads, 3, head_dim)


def moba_gate_topk(q, pooled, geom, topk, block_idx=None, stream=None):
    """pooled: the PooledKeys of moba_pool_keys."""
    H, d = _qkv_shape(q, geom)
    if block_idx is None:
        block_idx = torch.empty((geom.total_tokens, H, topk), dtype=torch.int32, device=q.device)
    _check("moba_gate_topk", lib().moba_gate_topk(
        _ptr(q), _dtype_code(q.dtype), _ptr(pooled.kbar), _ptr(pooled.kbar3),
        *geom.args(H, d), int(topk), _ptr(block_idx), _stream(stream)))
    return block_idx


def moba_pool_minmax(k, geom, kminmax=None, stream=None):
    """Elementwise block max and min of the keys, exact, in the library's
    group-major layout: kminmax [H, d / 2, NB, 4] fp32, where group g of a
    block's [kmax, kmin] row (2d values) holds its values 4g .. 4g + 3
    (``kminmax_rows`` gives them as [NB, H, 2, d])."""
    H, d = _qkv_shape(k, geom)
    if kminmax is None:
        kminmax = torch.empty((H, d // 2, geom.total_blocks, 4), dtype=torch.float32,
                              device=k.device)
    _check("moba_pool_minmax", lib().moba_pool_minmax(
        _ptr(k), _dtype_code(k.dtype), *geom.args(H, d), _ptr(kminmax), _stream(stream)))
    return kminmax


def kminmax_rows(kminmax, num_heads, head_dim, total_blocks):
    """[NB, H, 2, d] view order (max, then min) of a kminmax buffer (a copy)."""
    t = kminmax.reshape(num_heads, 2, head_dim // 4, total_blocks, 4)
    return t.permute(3, 0, 1, 2, 4).reshape(total_blocks, num_heads, 2, head_dim)


def moba_gate_topk_minmax(q, kminmax, geom, topk, block_idx=None, stream=None):
    """Causal top-k with the min/max pooled score (bf16 q)."""
    H, d = _qkv_shape(q, geom)
    if block_idx is None:
        block_idx = torch.empty((geom.total_tokens, H, topk), dtype=torch.int32, device=q.device)
    _check("moba_gate_topk_minmax", lib().moba_gate_topk_minmax(
        _ptr(q), _dtype_code(q.dtype), _ptr(kminmax), *geom.args(H, d), int(topk),
        _ptr(block_idx), _stream(stream)))
    return block_idx


def moba_static_select(geom, num_heads, topk, sink_blocks, block_idx=None, device=None,
                       stream=None):
    """Static routing rows (sliding window with sink_blocks = 0, sink + window
    otherwise, full attention when topk covers every block) in the
    moba_gate_topk format: block_idx [T, H, topk] int32."""
    if block_idx is None:
        block_idx = torch.empty((geom.total_tokens, num_heads, topk), dtype=torch.int32,
                                device=device if device is not None else geom.cu_seqlens.device)
    _check("moba_static_select", lib().moba_static_select(
        _ptr(geom.cu_seqlens), _ptr(geom.cu_blocks), geom.num_seqs, geom.total_tokens,
        geom.max_seqlen, geom.total_blocks, int(num_heads), geom.block_size, int(topk),
        int(sink_blocks), _ptr(block_idx), _stream(stream)))
    return block_idx


def moba_attn_workspace_bytes(dtype, total_tokens, total_blocks, num_heads, head_dim,
                              block_size, topk, head_chunk=0):
    """Workspace of moba_attn_fwd for passes of head_chunk heads (0: all)."""
    return int(lib().moba_attn_workspace_bytes(dtype, total_tokens, total_blocks, num_heads,
                                               head_dim, block_size, topk, int(head_chunk)))


def moba_attn_bwd_workspace_bytes(dtype, total_tokens, total_blocks, num_heads, head_dim,
                                  block_size, topk):
    return int(lib().moba_attn_bwd_workspace_bytes(dtype, total_tokens, total_blocks, num_heads,
                                                   head_dim, block_size, topk))


def moba_dense_workspace_bytes(dtype, total_tokens, total_blocks, num_heads, head_dim,
                               block_size):
    return int(lib().moba_dense_workspace_bytes(dtype, total_tokens, total_blocks, num_heads,
                                                head_dim, block_size))


def _workspace(nbytes, device):
    # torch allocations are at least 256-byte aligned
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def moba_attn_fwd(q, k, v, geom, topk, block_idx, scale, out=None, out_dtype=None, lse=None,
                  workspace=None, stream=None, head_chunk=0):
    """Sparse attention over the selected blocks; head_chunk heads per pass
    (0: all heads in one pass; the workspace scales with it)."""
    H, d = _qkv_shape(q, geom)
    dt = _dtype_code(q.dtype)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((geom.total_tokens, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _workspace(moba_attn_workspace_bytes(
            dt, geom.total_tokens, geom.total_blocks, H, d, geom.block_size, topk, head_chunk),
            q.device)
    _check("moba_attn_fwd", lib().moba_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), dt, *geom.args(H, d), int(topk), _ptr(block_idx),
        float(scale), _ptr(out), _dtype_code(out.dtype), _ptr(lse), int(head_chunk),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def moba_attn_fwd_static(q, k, v, geom, topk, block_idx, scale, out, lse, stream=None):
    """moba_attn_fwd with the library's fixed device workspace: the call
    allocates nothing (out and lse are the caller's tensors)."""
    H, d = _qkv_shape(q, geom)
    _check("moba_attn_fwd_static", lib().moba_attn_fwd_static(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), *geom.args(H, d), int(topk),
        _ptr(block_idx), float(scale), _ptr(out), _dtype_code(out.dtype), _ptr(lse),
        _stream(stream)))
    return out, lse


def moba_dense_causal_fwd(q, k, v, geom, scale, out=None, out_dtype=None, lse=None,
                          workspace=None, stream=None):
    H, d = _qkv_shape(q, geom)
    dt = _dtype_code(q.dtype)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((geom.total_tokens, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _workspace(moba_dense_workspace_bytes(
            dt, geom.total_tokens, geom.total_blocks, H, d, geom.block_size), q.device)
    _check("moba_dense_causal_fwd", lib().moba_dense_causal_fwd(
        _ptr(q), _ptr(k), _ptr(v), dt, *geom.args(H, d), float(scale), _ptr(out),
        _dtype_code(out.dtype), _ptr(lse), _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return out, lse


class Profiler:
    """Per-kernel HIP-event timing of the library's launches on this thread."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check("moba_profiler_create", lib().moba_profiler_create(ctypes.byref(h)))
        self.handle = h

    def attach(self):
        _check("moba_profiler_attach", lib().moba_profiler_attach(self.handle))
        return self

    def detach(self):
        _check("moba_profiler_attach", lib().moba_profiler_attach(None))

    def reset(self):
        _check("moba_profiler_reset", lib().moba_profiler_reset(self.handle))

    def read(self, name):
        n = ctypes.c_int()
        ms = ctypes.c_double()
        _check("moba_profiler_read", lib().moba_profiler_read(
            self.handle, name.encode(), ctypes.byref(n), ctypes.byref(ms)))
        return n.value, ms.value

    def names(self):
        buf = ctypes.create_string_buffer(4096)
        _check("moba_profiler_names", lib().moba_profiler_names(self.handle, buf, 4096))
        return [x for x in buf.value.decode().split(",") if x]

    def summary(self):
        return {nm: self.read(nm) for nm in self.names()}

    def close(self):
        if self.handle:
            lib().moba_profiler_destroy(self.handle)
            self.handle = None


def forward(q, k, v, geom, topk, scale, out_dtype=None, workspace=None, stream=None,
            head_chunk=0):
    """MoBA prefill forward: pool -> gate/top-k -> sparse attention.
    Returns (out, lse, block_idx)."""
    pooled = moba_pool_keys(k, geom, stream=stream)
    idx = moba_gate_topk(q, pooled, geom, topk, stream=stream)
    out, lse = moba_attn_fwd(q, k, v, geom, topk, idx, scale, out_dtype=out_dtype,
                             workspace=workspace, stream=stream, head_chunk=head_chunk)
    return out, lse, idx


def moba_attn_bwd(q, k, v, out, dout, lse, geom, topk, block_idx, scale, dq=None, dk=None,
                  dv=None, workspace=None, stream=None):
    """Gradients of moba_attn_fwd (fp32 dq, dk, dv) for the selections
    block_idx; out and lse are the forward's outputs."""
    H, d = _qkv_shape(q, geom)
    shape = (geom.total_tokens, H, d)
    dq = torch.empty(shape, dtype=torch.float32, device=q.device) if dq is None else dq
    dk = torch.empty(shape, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(shape, dtype=torch.float32, device=q.device) if dv is None else dv
    nbytes = moba_attn_bwd_workspace_bytes(_dtype_code(q.dtype), geom.total_tokens,
                                           geom.total_blocks, H, d, geom.block_size, int(topk))
    if workspace is None:
        workspace = _workspace(nbytes, q.device)
    _check("moba_attn_bwd", lib().moba_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _dtype_code(out.dtype), _ptr(dout), _ptr(lse),
        _dtype_code(q.dtype), *geom.args(H, d), int(topk), _ptr(block_idx), float(scale),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), _stream(stream)))
    return dq, dk, dv


def forward_head_streamed(source, geom, num_heads, group_heads, topk, scale, out_dtype=None,
                          head_chunk=0, groups=None, on_group=None, stream=None):
    """One MoBA layer whose heads are brought into device memory a group at a
    time, for layers too large to hold whole ("MoBA: Learned Block Sparsity
    for Long-Context Attention", "Efficiency and Implementation": the
    10M-token run splits work at the level of query heads).  Heads never
    interact in MoBA, so each group runs pool -> gate -> sparse attention on
    its own, in one workspace (sized for group_heads heads in passes of
    head_chunk) reused by every group.

    source(h0, h1) returns device tensors (q, k, v) [T, h1 - h0, d] for heads
    h0 .. h1 - 1 (a host-to-device copy, a projection, a generator).
    groups: indices of the groups to run (default all).  on_group(h0, out,
    lse, block_idx) receives each group's results; without it the (h0, out,
    lse) of every group are returned."""
    ngroups = (num_heads + group_heads - 1) // group_heads
    ws = None
    results = []
    for g in (range(ngroups) if groups is None else groups):
        h0 = g * group_heads
        h1 = min(num_heads, h0 + group_heads)
        q, k, v = source(h0, h1)
        H, d = _qkv_shape(q, geom)
        if H != h1 - h0:
            raise ValueError("source returned the wrong number of heads")
        if ws is None:
            ws = _workspace(moba_attn_workspace_bytes(
                _dtype_code(q.dtype), geom.total_tokens, geom.total_blocks, group_heads, d,
                geom.block_size, topk, head_chunk), q.device)
        out, lse, idx = forward(q, k, v, geom, topk, scale, out_dtype=out_dtype, workspace=ws,
                                stream=stream, head_chunk=head_chunk)
        del q, k, v
        if on_group is not None:
            on_group(h0, out, lse, idx)
        else:
            results.append((h0, out, lse))
        del idx
    return results


def forward_minmax(q, k, v, geom, topk, scale, out_dtype=None, workspace=None, stream=None):
    """MoBA with the min/max pooled gate: pool_minmax -> gate -> sparse
    attention.  Returns (out, lse, block_idx)."""
    kmm = moba_pool_minmax(k, geom, stream=stream)
    idx = moba_gate_topk_minmax(q, kmm, geom, topk, stream=stream)
    out, lse = moba_attn_fwd(q, k, v, geom, topk, idx, scale, out_dtype=out_dtype,
                             workspace=workspace, stream=stream)
    return out, lse, idx


def forward_static(q, k, v, geom, topk, sink_blocks, scale, out_dtype=None, workspace=None,
                   stream=None):
    """Attention through a static gate (sliding window / sink + window / full):
    static routing -> sparse attention.  Returns (out, lse, block_idx)."""
    H, d = _qkv_shape(q, geom)
    idx = moba_static_select(geom, H, topk, sink_blocks, device=q.device, stream=stream)
    out, lse = moba_attn_fwd(q, k, v, geom, topk, idx, scale, out_dtype=out_dtype,
                             workspace=workspace, stream=stream)
    return out, lse, idx


def dense(q, k, v, geom, scale, out_dtype=None, workspace=None, stream=None):
    """Dense causal attention with the library's own kernel.  Returns (out, lse)."""
    return moba_dense_causal_fwd(q, k, v, geom, scale, out_dtype=out_dtype,
                                 workspace=workspace, stream=stream)


def hybrid_schedule(num_layers, full_last):
    """Attention mode of each layer in the layer-wise hybrid: MoBA for the
    first num_layers - full_last layers, full attention for the last
    full_last ("MoBA: Learned Block Sparsity for Long-Context Attention",
    section "Why the Change Is Plausible": switching the last layers to full
    attention; the hybrid mode of the elamur.ai summary, "Key points")."""
    if not 0 <= full_last <= num_layers:
        raise ValueError("full_last must lie in [0, num_layers]")
    return ["moba"] * (num_layers - full_last) + ["full"] * full_last


def layer_forward(mode, q, k, v, geom, topk, scale, out_dtype=None, workspace=None,
                  stream=None):
    """One attention layer in the given hybrid mode: "moba" (pool, gate,
    sparse attention) or "full" (the dense causal kernel).  Returns
    (out, lse)."""
    if mode == "moba":
        out, lse, _ = forward(q, k, v, geom, topk, scale, out_dtype=out_dtype,
                              workspace=workspace, stream=stream)
        return out, lse
    if mode == "full":
        return dense(q, k, v, geom, scale, out_dtype=out_dtype, workspace=workspace,
                     stream=stream)
    raise ValueError(f"unknown attention mode {mode!r}")


def probe_mfma_rate(workgroups, iterations, sink, operands=0, stream=None):
    """Launches the bf16 MFMA rate probe (measurement support); operands 0 =
    fixed register operands, 1 = random register operands, 2 = random
    operands with B read from LDS; sink: float32 device tensor of at least
    workgroups * 256 elements.  Returns its flop count."""
    _check("moba_probe_mfma_rate", lib().moba_probe_mfma_rate(
        int(workgroups), int(iterations), int(operands), _ptr(sink), _stream(stream)))
    return workgroups * 4 * 4 * iterations * 2 * 32 * 32 * 16
