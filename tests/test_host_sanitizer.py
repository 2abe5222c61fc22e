"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of libzb is compiled with the sanitizers on the host pass only
(the device code is built as usual and never instrumented), linked with
tests/native/host_check.cpp into one executable, and run on the CPU: the
schedule layer and the stage set-up path of every workload shape
(create, per-class sizes, the workspace plan for the real one-device order,
binding, slot claims, taps, a schedule refused before launch).  A sanitizer
report or a wrong status fails the test.  Runs without a GPU.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "split_backward_gemms_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _tool(name):
    for cand in (os.path.join(ROCM, "bin", name), os.path.join(ROCM, "llvm", "bin", name), shutil.which(name)):
        if cand and os.path.exists(cand):
            return cand
    return None


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{err[-4000:]}"
    return r


def test_host_code_is_sanitizer_clean(tmp_path):
    hipcc, clangxx = _tool("hipcc"), _tool("clang++")
    if not hipcc or not clangxx:
        pytest.skip("ROCm toolchain not available")
    # Sanitizers on the host pass only.
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    srcs = [s for s in sorted(os.listdir(CSRC)) if s.endswith((".hip", ".cpp"))]
    objs = [str(tmp_path / (s + ".o")) for s in srcs]
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        list(ex.map(lambda so: _run([hipcc] + common + san + ["-x", "hip", "-c", os.path.join(CSRC, so[0]),
                                                            "-o", so[1]]), zip(srcs, objs)))
    drv = str(tmp_path / "host_check.o")
    _run([clangxx, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-c", os.path.join(HERE, "native", "host_check.cpp"), "-o", drv])
    exe = str(tmp_path / "host_check")
    _run([clangxx, "-fsanitize=address,undefined", "-o", exe, drv] + objs +
         [f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "host checks: 0 failure(s)" in out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out
