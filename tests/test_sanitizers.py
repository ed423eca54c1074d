"""Host code under sanitizers, on the CPU only.

* The oracle's threaded entry points, driven by tests/native/oracle_threads.cpp,
  under ThreadSanitizer and under AddressSanitizer + UndefinedBehaviorSanitizer
  (g++), with one and several threads giving bitwise equal results.
* The library's host-side argument checks, tile-table parser and StairCut cut
  rule (the host-only tests of test_boundary.py and the StairCut tests) against
  a build of libnvfp4v.so whose host code carries AddressSanitizer and
  UndefinedBehaviorSanitizer (clang, via hipcc -Xarch_host), in a subprocess
  that preloads the matching runtime. The GPU code is built as usual and never
  launched.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "nvfp4_oracle.cpp")
DRIVER = os.path.join(ROOT, "tests", "native", "oracle_threads.cpp")


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.parametrize("san", ["thread", "address,undefined"])
def test_oracle_under_sanitizer(tmp_path, san):
    exe = str(tmp_path / "oracle_threads")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-pthread",
           "-fsanitize=" + san, "-fno-sanitize-recover=all", ORACLE_SRC, DRIVER, "-o", exe]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1", ASAN_OPTIONS="halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def _clang_runtime(name):
    base = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        p = os.path.join(base, ver, "lib", "linux", name)
        if os.path.exists(p):
            return p
    return None


@pytest.mark.skipif(_gpu_visible(), reason="host-only argument checks hand fake device addresses to the library")
@pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None, reason="needs hipcc")
@pytest.mark.parametrize("san,runtime,opts", [
    ("address", "libclang_rt.asan-x86_64.so", {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1"}),
    ("undefined", "libclang_rt.ubsan_standalone-x86_64.so", {"UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}),
])
def test_library_host_code_under_sanitizer(san, runtime, opts):
    rt = _clang_runtime(runtime)
    if rt is None:
        pytest.skip("no %s in the ROCm LLVM tree" % runtime)
    sys.path.insert(0, ROOT)
    from nvfp4_skinny_gemm_amd import build

    lib = build.build(sanitize=san)
    env = dict(os.environ, NVFP4V_LIBRARY=lib, LD_PRELOAD=rt, **opts)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_boundary.py"),
                        os.path.join(ROOT, "tests", "test_oracle_staircut_pins.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout
