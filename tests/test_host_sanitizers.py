"""The C-ABI layer (api.cpp) built for the host with AddressSanitizer and
UndefinedBehaviorSanitizer, against stub kernel launchers, and driven through
every entry point: invalid arguments, the supported limits, workspace sizes
for every head pass, geometries past the int32 limits and the largest token
counts the size arithmetic sees (tests/host_sanitize/driver.cpp).  Any
out-of-bounds access, signed overflow or other undefined behaviour aborts the
driver.  CPU only: g++ builds it, no GPU is touched."""

import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HIP_INCLUDE = "/opt/rocm/include"
HIP_LIB = "/opt/rocm/lib"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INCLUDE),
                    reason="needs g++ and the HIP headers")
def test_abi_under_host_sanitizers(tmp_path):
    exe = tmp_path / "abi_sanitized"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{HIP_INCLUDE}",
           str(ROOT / "block_sparse_long_03_amd/csrc/api.cpp"),
           str(ROOT / "tests/host_sanitize/stubs.cpp"),
           str(ROOT / "tests/host_sanitize/driver.cpp"),
           f"-L{HIP_LIB}", "-lamdhip64", f"-Wl,-rpath,{HIP_LIB}", "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "host sanitizer checks passed" in out
    print(out.strip().splitlines()[-1])
