"""Python binding of libnvfp4v (the NVFP4 skinny verify-GEMM for MI355X).

Argument marshalling only: every step runs in the HIP library behind the C ABI
declared in include/nvfp4v.h. PyTorch provides device memory and streams. The
library must be built (``python nvfp4_skinny_gemm_amd/build.py`` or
``__graft_entry__.build()``); without it, importing the binding's entry points
raises, there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4v.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "nvfp4v.h")

OK = 0
E_INVALID_ARG = -1
E_SHAPE = -2
E_M_RANGE = -3
E_ALIGN = -4
E_HIP = -5
E_FAULT = -6
E_NONFINITE = -7
E_WORKSPACE = -8
MAX_M = 64

_lib = None


class Nvfp4vError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, strerror(status), status))


def load():
    """Load libnvfp4v.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libnvfp4v.so is not built: run __graft_entry__.build() "
                          "(python nvfp4_skinny_gemm_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    c = ctypes
    p = c.c_void_p
    i64 = c.c_int64
    lib.nvfp4v_create.argtypes = [c.POINTER(p), c.c_int]
    lib.nvfp4v_destroy.argtypes = [p]
    lib.nvfp4v_destroy.restype = None
    lib.nvfp4v_strerror.argtypes = [c.c_int]
    lib.nvfp4v_strerror.restype = c.c_char_p
    lib.nvfp4v_last_hip_error.argtypes = [p]
    lib.nvfp4v_quantize_host.argtypes = [p, i64, i64, p, p]
    lib.nvfp4v_quantize.argtypes = [p, p, i64, i64, p, p, p]
    lib.nvfp4v_encode_e4m3_host.argtypes = [p, i64, p]
    lib.nvfp4v_packed_bytes.argtypes = [i64, i64]
    lib.nvfp4v_packed_bytes.restype = c.c_size_t
    lib.nvfp4v_pack.argtypes = [p, p, p, i64, i64, p, p]
    lib.nvfp4v_unpack.argtypes = [p, p, i64, i64, p, p, p]
    lib.nvfp4v_verify_gemm.argtypes = [p, p, i64, i64, p, i64, c.c_float, p, p]
    lib.nvfp4v_describe_plan.argtypes = [p, i64, i64, i64, c.c_char_p, c.c_size_t]
    lib.nvfp4v_staircase.argtypes = [p, i64, i64, c.c_int, c.c_int, c.c_int, c.c_int,
                                     c.c_size_t, p]
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().nvfp4v_strerror(int(status)).decode()


def _check(status: int, where: str):
    if status != OK:
        raise Nvfp4vError(status, where)


def _np_ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _t_ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def packed_bytes(n: int, k: int) -> int:
    return int(load().nvfp4v_packed_bytes(int(n), int(k)))


def quantize_host(w):
    """fp32 numpy w[n, k] -> (codes u8[n, k/2], scales u8[n, k/16])."""
    import numpy as np

    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    codes = np.zeros((n, k // 2), np.uint8)
    scales = np.zeros((n, max(k // 16, 1)), np.uint8)
    _check(load().nvfp4v_quantize_host(_np_ptr(w), n, k, _np_ptr(codes), _np_ptr(scales)),
           "nvfp4v_quantize_host")
    return codes, scales


def encode_e4m3_host(x):
    import numpy as np

    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(x.shape, np.uint8)
    _check(load().nvfp4v_encode_e4m3_host(_np_ptr(x), x.size, _np_ptr(out)),
           "nvfp4v_encode_e4m3_host")
    return out


class Context:
    """An nvfp4v context on one GPU (owns the split-K workspace)."""

    def __init__(self, device: int = 0):
        lib = load()
        h = ctypes.c_void_p()
        _check(lib.nvfp4v_create(ctypes.byref(h), int(device)), "nvfp4v_create")
        self._h = h
        self.device = device

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            load().nvfp4v_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    def last_hip_error(self) -> int:
        return int(load().nvfp4v_last_hip_error(self._h))

    # -- format --------------------------------------------------------------
    def quantize(self, w, stream=None):
        """fp32 cuda tensor w[n, k] -> (codes u8[n, k/2], scales u8[n, k/16]) on the device."""
        import torch

        n, k = w.shape
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
        scales = torch.empty((n, k // 16), dtype=torch.uint8, device=w.device)
        _check(load().nvfp4v_quantize(self._h, _t_ptr(w), n, k, _t_ptr(codes), _t_ptr(scales),
                                      _stream_handle(stream)), "nvfp4v_quantize")
        return codes, scales

    def pack(self, codes, scales, n: int, k: int, out=None, stream=None):
        import torch

        nb = packed_bytes(n, k)
        if out is None:
            out = torch.empty(nb, dtype=torch.uint8, device=codes.device)
        _check(load().nvfp4v_pack(self._h, _t_ptr(codes), _t_ptr(scales), n, k, _t_ptr(out),
                                  _stream_handle(stream)), "nvfp4v_pack")
        return out

    def unpack(self, packed, n: int, k: int, stream=None):
        import torch

        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=packed.device)
        scales = torch.empty((n, k // 16), dtype=torch.uint8, device=packed.device)
        _check(load().nvfp4v_unpack(self._h, _t_ptr(packed), n, k, _t_ptr(codes), _t_ptr(scales),
                                    _stream_handle(stream)), "nvfp4v_unpack")
        return codes, scales

    # -- GEMM ----------------------------------------------------------------
    def verify_gemm(self, a, packed, n: int, k: int, ts: float = 1.0, out=None, stream=None):
        """C[m, n] fp32 = ts * A[m, k] (bf16 cuda tensor) * W^T."""
        import torch

        m = a.shape[0]
        if out is None:
            out = torch.empty((m, n), dtype=torch.float32, device=a.device)
        _check(load().nvfp4v_verify_gemm(self._h, _t_ptr(a), m, k, _t_ptr(packed), n,
                                         float(ts), _t_ptr(out), _stream_handle(stream)),
               "nvfp4v_verify_gemm")
        return out

    def describe_plan(self, n: int, k: int, m: int) -> str:
        buf = ctypes.create_string_buffer(256)
        _check(load().nvfp4v_describe_plan(self._h, n, k, m, buf, 256), "nvfp4v_describe_plan")
        return buf.value.decode()

    def staircase(self, n: int, k: int, m_lo: int, m_hi: int, warmup: int = 3, reps: int = 20,
                  rotate_bytes: int = 2 << 30):
        import numpy as np

        out = np.zeros(m_hi - m_lo + 1, np.float64)
        _check(load().nvfp4v_staircase(self._h, n, k, m_lo, m_hi, warmup, reps, rotate_bytes,
                                       _np_ptr(out)), "nvfp4v_staircase")
        return out


def exported_names():
    """Function names declared in include/nvfp4v.h."""
    import re

    src = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"\b(nvfp4v_[a-z0-9_]+)\s*\(", src)))
