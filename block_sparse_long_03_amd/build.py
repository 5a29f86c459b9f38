"""Builds libmoba.so (the HIP kernels and the C ABI) for gfx950 in-tree.

    python -m block_sparse_long_03_amd.build

Sources are compiled in parallel with hipcc into ``_build/`` and linked into
``block_sparse_long_03_amd/libmoba.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoba.so")
SOURCES = ["api.cpp", "pool_gate.hip", "bucket_merge.hip", "attn_mfma.hip", "attn_f32.hip",
           "attn_bwd.hip", "probe.hip", "static_ws.hip"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


# per-source code generation options: the backward kernels keep MFMA
# operands and results in VGPRs (their register use fits without spills then);
# its resource report is checked below
SOURCE_FLAGS = {"attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1",
                                 "-Rpass-analysis=kernel-resource-usage"]}

# Kernels that must not use scratch memory: bwd_kv_pair_kernel's tile barrier
# lets exactly the wave's own LDS DMA of the iteration stay in flight
# (s_waitcnt vmcnt(n)), which is only right while no other vector-memory
# instruction, such as a register spill to scratch, sits in its loop.
NO_SCRATCH = {"attn_bwd.hip": ["bwd_kv_pair_kernel"]}


def _check_scratch(src, report):
    """Raises if a kernel listed in NO_SCRATCH reports scratch use."""
    current = None
    for line in report.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            current = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and current and any(k in current for k in NO_SCRATCH.get(src, [])):
            if int(m.group(1)) != 0:
                raise RuntimeError(f"{current} in {src} uses {m.group(1)} bytes of scratch per lane;"
                                   " its vmcnt accounting assumes none")


def _compile(src, build_dir=BUILD, defines=()):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = ([HIPCC, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + CFLAGS
           + SOURCE_FLAGS.get(src, []) + [f"-D{d}" for d in defines])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if src in NO_SCRATCH:
        _check_scratch(src, r.stderr)
    return obj


def build(verbose=True, out=LIB, defines=()):
    """Compiles every source (optionally with extra -D defines) and links `out`."""
    build_dir = BUILD if out == LIB else os.path.join(BUILD, os.path.basename(out) + ".d")
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build()
    sys.exit(0)
