"""Build libnvfp4v.so in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-FP32 instructions turned off
(-Xclang -target-feature -Xclang -packed-fp32-ops); hipcc's host pass warns that
it does not know that feature, which is harmless.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnvfp4v.so")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "format.hip", "gemm.hip", "staircase.hip", "pass.hip", "measure.hip", "head.hip", "staircut.cpp", "noalloc.hip", "attention.hip"]

CFLAGS = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-Wno-unknown-warning-option",
]


def _host_sanitizer_flags(sanitize: str) -> list:
    """Host-only sanitizer flags: each applies to the host pass alone (the GPU
    code is built as usual)."""
    flags = []
    for f in ("-fsanitize=" + sanitize, "-fno-sanitize-recover=all", "-g", "-fno-omit-frame-pointer"):
        flags += ["-Xarch_host", f]
    return flags


def _compile(src: str, sanitize: str = "") -> str:
    odir = os.path.join(OBJ, sanitize) if sanitize else OBJ
    obj = os.path.join(odir, os.path.splitext(src)[0] + ".o")
    extra = _host_sanitizer_flags(sanitize) if sanitize else []
    cmd = [HIPCC, *CFLAGS, *extra, "-I", OBJ, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


TABLE = os.path.join(HERE, "tables", "gfx950.txt")


def _embed_table() -> None:
    """The built-in tile table is tables/gfx950.txt, compiled into the library
    as a string (the file stays the one source of its rows)."""
    text = open(TABLE).read()
    assert ")TABLE\"" not in text
    out = os.path.join(OBJ, "tile_table_gfx950.inc")
    body = 'R"TABLE(' + text + ')TABLE"\n'
    if not os.path.exists(out) or open(out).read() != body:
        with open(out, "w") as f:
            f.write(body)


def build(verbose: bool = False, sanitize: str = "") -> str:
    """Build libnvfp4v.so. With `sanitize` ("address", "undefined" or "thread")
    the host code is instrumented and the library goes to
    _build/<sanitize>/libnvfp4v.so instead (load it with NVFP4V_LIBRARY and the
    matching clang runtime in LD_PRELOAD; for CPU-only runs)."""
    assert sanitize in ("", "address", "undefined", "thread"), sanitize
    os.makedirs(os.path.join(OBJ, sanitize) if sanitize else OBJ, exist_ok=True)
    _embed_table()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, sanitize), SOURCES))
    lib = os.path.join(OBJ, sanitize, "libnvfp4v.so") if sanitize else LIB
    tmp = lib + ".tmp"
    link = ["-Xarch_host", "-fsanitize=" + sanitize] if sanitize else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser()
    ap.add_argument("--sanitize", default="", choices=("", "address", "undefined", "thread"))
    build(verbose=True, sanitize=ap.parse_args().sanitize)
    sys.exit(0)
