"""CPU oracle for the NVFP4 verify GEMM (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports, links or calls it, and shares no code with
it. The arithmetic lives in ``nvfp4_oracle.cpp`` (plain C++17, fp64); this
module only marshals numpy arrays through ctypes.

Every function restates the definition it follows:
  w(j,k)  = E2M1(code) * E4M3(scale of the 16-block along k) * ts
  C[i][j] = sum_k a(i,k) w(j,k)     (fp64, k ascending)
  S[i][j] = sum_k |a(i,k) w(j,k)|
The parity bar used by the tests is |C_gpu - C| <= 1e-5 * S per element.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.cpp")
# ORACLE_SANITIZE=address|thread|undefined selects a build of the oracle with
# that g++ sanitizer (run with the matching runtime in LD_PRELOAD, e.g.
# LD_PRELOAD=$(g++ -print-file-name=libasan.so)).
_SANITIZE = os.environ.get("ORACLE_SANITIZE", "")
assert _SANITIZE in ("", "address", "thread", "undefined"), "ORACLE_SANITIZE=%r" % _SANITIZE
_LIB = os.path.join(_HERE, "liboracle%s.so" % ("_" + _SANITIZE if _SANITIZE else ""))

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with g++ (-O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["g++", "-std=c++17", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
               "-shared", "-pthread", _SRC, "-o", tmp]
        if _SANITIZE:
            cmd[1:1] = ["-fsanitize=" + _SANITIZE, "-fno-sanitize-recover=all", "-g", "-fno-omit-frame-pointer"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    c = ctypes
    p = c.c_void_p
    i64 = c.c_int64
    lib.oracle_thread_count.restype = c.c_int
    lib.oracle_e2m1_value.argtypes = [c.c_int]
    lib.oracle_e2m1_value.restype = c.c_double
    lib.oracle_e4m3_value.argtypes = [c.c_int]
    lib.oracle_e4m3_value.restype = c.c_double
    lib.oracle_e4m3_encode.argtypes = [c.c_double, p]
    lib.oracle_e4m3_encode.restype = c.c_int
    lib.oracle_e2m1_encode.argtypes = [c.c_double, p]
    lib.oracle_e2m1_encode.restype = c.c_int
    lib.oracle_quantize.argtypes = [p, i64, i64, p, p, c.c_int]
    lib.oracle_quantize.restype = c.c_int
    lib.oracle_decode.argtypes = [p, p, i64, i64, c.c_double, p]
    lib.oracle_decode.restype = None
    lib.oracle_gemm.argtypes = [p, i64, i64, p, p, i64, c.c_double, p, p, c.c_int]
    lib.oracle_gemm.restype = None
    lib.oracle_gemm_cols.argtypes = [p, i64, i64, p, p, p, i64, c.c_double, p, p, c.c_int]
    lib.oracle_gemm_cols.restype = None
    lib.oracle_bf16_from_f32.argtypes = [p, i64, p]
    lib.oracle_fp8_quantize.argtypes = [p, i64, i64, p, p, c.c_int]
    lib.oracle_fp8_quantize.restype = c.c_int
    lib.oracle_fp8_gemm_cols.argtypes = [p, i64, i64, p, p, p, i64, p, p, c.c_int]
    lib.oracle_fp8_gemm_cols.restype = None
    lib.oracle_bf16_from_f32.restype = None
    lib.oracle_glue_scale.argtypes = [p, i64, c.c_float, p]
    lib.oracle_glue_scale.restype = None
    lib.oracle_glue_sum.argtypes = [p, p, i64, c.c_float, p]
    lib.oracle_glue_sum.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def thread_count() -> int:
    """Threads the oracle uses by default: the size of the CPU affinity mask."""
    return int(_load().oracle_thread_count())


def e2m1_value(code: int) -> float:
    return float(_load().oracle_e2m1_value(int(code)))


def e4m3_value(byte: int) -> float:
    return float(_load().oracle_e4m3_value(int(byte)))


def e4m3_encode(x: float) -> int:
    out = np.zeros(1, np.uint8)
    if _load().oracle_e4m3_encode(float(x), _ptr(out)) != 0:
        raise ValueError("NaN has no E4M3 encoding here")
    return int(out[0])


def e2m1_encode(q: float) -> int:
    out = np.zeros(1, np.uint8)
    if _load().oracle_e2m1_encode(float(q), _ptr(out)) != 0:
        raise ValueError("NaN has no E2M1 encoding")
    return int(out[0])


def quantize(w: np.ndarray, threads: int = 0):
    """fp32 w[n, k] -> (codes u8[n, k/2], scales u8[n, k/16]) in the canonical format."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    codes = np.zeros((n, k // 2), np.uint8)
    scales = np.zeros((n, k // 16), np.uint8)
    rc = _load().oracle_quantize(_ptr(w), n, k, _ptr(codes), _ptr(scales), int(threads))
    if rc == -1:
        raise ValueError("non-finite weight")
    if rc != 0:
        raise ValueError("k must be a multiple of 16")
    return codes, scales


def decode(codes: np.ndarray, scales: np.ndarray, ts: float = 1.0) -> np.ndarray:
    """Canonical format -> dense fp64 weights [n, k] (times ts)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    n = codes.shape[0]
    k = codes.shape[1] * 2
    w = np.empty((n, k), np.float64)
    _load().oracle_decode(_ptr(codes), _ptr(scales), n, k, float(ts), _ptr(w))
    return w


def gemm(a_bf16: np.ndarray, codes: np.ndarray, scales: np.ndarray, ts: float = 1.0,
         cols=None, threads: int = 0):
    """(C, S) in fp64 for A[m, k] (bf16 bit patterns, uint16) against the weights.

    With ``cols`` given, only those weight rows are evaluated and the outputs are
    [m, len(cols)]; ``codes``/``scales`` still hold the full matrix.
    """
    a = np.ascontiguousarray(a_bf16, dtype=np.uint16)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    m, k = a.shape
    if codes.shape[1] * 2 != k or scales.shape[1] * 16 != k:
        raise ValueError("shape mismatch between A and the weights")
    lib = _load()
    if cols is None:
        n = codes.shape[0]
        c = np.empty((m, n), np.float64)
        s = np.empty((m, n), np.float64)
        lib.oracle_gemm(_ptr(a), m, k, _ptr(codes), _ptr(scales), n, float(ts), _ptr(c),
                        _ptr(s), int(threads))
        return c, s
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if cols.size and (cols.min() < 0 or cols.max() >= codes.shape[0]):
        raise ValueError("column index out of range")
    c = np.empty((m, cols.size), np.float64)
    s = np.empty((m, cols.size), np.float64)
    lib.oracle_gemm_cols(_ptr(a), m, k, _ptr(codes), _ptr(scales), _ptr(cols), cols.size,
                         float(ts), _ptr(c), _ptr(s), int(threads))
    return c, s


def fp8_quantize(w: np.ndarray, threads: int = 0):
    """fp32 w[n, k] -> (E4M3 codes u8[n, k], fp32 row scales[n]) for the FP8 head."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    codes = np.zeros((n, k), np.uint8)
    scales = np.zeros(n, np.float32)
    rc = _load().oracle_fp8_quantize(_ptr(w), n, k, _ptr(codes), _ptr(scales), int(threads))
    if rc == -1:
        raise ValueError("non-finite weight")
    if rc != 0:
        raise ValueError("bad shape")
    return codes, scales


def fp8_gemm(a_bf16: np.ndarray, codes: np.ndarray, row_scales: np.ndarray, cols=None,
             threads: int = 0):
    """(C, S) in fp64 for A[m, k] (bf16 bits) against the FP8 head codes[n, k], row_scales[n].

    With ``cols`` given, only those weight rows are evaluated ([m, len(cols)]).
    """
    a = np.ascontiguousarray(a_bf16, dtype=np.uint16)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    row_scales = np.ascontiguousarray(row_scales, dtype=np.float32)
    m, k = a.shape
    if codes.shape[1] != k or row_scales.shape[0] != codes.shape[0]:
        raise ValueError("shape mismatch between A and the weights")
    cols = np.arange(codes.shape[0], dtype=np.int64) if cols is None else \
        np.ascontiguousarray(cols, dtype=np.int64)
    if cols.size and (cols.min() < 0 or cols.max() >= codes.shape[0]):
        raise ValueError("column index out of range")
    c = np.empty((m, cols.size), np.float64)
    s = np.empty((m, cols.size), np.float64)
    _load().oracle_fp8_gemm_cols(_ptr(a), m, k, _ptr(codes), _ptr(row_scales), _ptr(cols),
                                 cols.size, _ptr(c), _ptr(s), int(threads))
    return c, s


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_bf16_from_f32(_ptr(x), x.size, _ptr(out))
    return out


def glue_scale(x: np.ndarray, cst: float) -> np.ndarray:
    """bf16(x * c) elementwise, fp32 product then round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_glue_scale(_ptr(x), x.size, float(np.float32(cst)), _ptr(out))
    return out


def glue_sum(x: np.ndarray, y: np.ndarray, cst: float) -> np.ndarray:
    """bf16(x * c + y * c) elementwise: two fp32 products, one fp32 sum (no FMA)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.ascontiguousarray(y, dtype=np.float32)
    if x.shape != y.shape:
        raise ValueError("shape mismatch")
    out = np.empty(x.shape, np.uint16)
    _load().oracle_glue_sum(_ptr(x), _ptr(y), x.size, float(np.float32(cst)), _ptr(out))
    return out


def within_tolerance(c_gpu: np.ndarray, c: np.ndarray, s: np.ndarray, rel: float = 1e-5):
    """Boolean mask of elements meeting |c_gpu - c| <= rel * S.

    S == 0 requires an exact zero (+0 and -0 compare equal); a NaN reference
    requires a NaN result. Infinite results never pass.
    """
    g = np.asarray(c_gpu, dtype=np.float64)
    ok = np.abs(g - c) <= rel * s
    nan_ref = np.isnan(c)
    ok = np.where(nan_ref, np.isnan(g), ok)
    ok &= ~np.isinf(g)
    return ok
