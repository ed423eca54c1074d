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
# NVFP4V_LIBRARY names another build of the same library (the host-sanitizer
# builds of build.py --sanitize); by default the in-tree libnvfp4v.so.
LIB_PATH = os.environ.get("NVFP4V_LIBRARY") or os.path.join(HERE, "libnvfp4v.so")
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
E_TIMEOUT = -9
E_DISPATCH = -10
E_TABLE = -11
PASS_CHAIN = 0
PASS_PERSISTENT = 1
MAX_M = 128

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
    lib.nvfp4v_create.argtypes = [c.POINTER(p), c.c_int, c.c_char_p]
    lib.nvfp4v_load_tile_table.argtypes = [p, c.c_char_p]
    lib.nvfp4v_destroy.argtypes = [p]
    lib.nvfp4v_destroy.restype = None
    lib.nvfp4v_strerror.argtypes = [c.c_int]
    lib.nvfp4v_strerror.restype = c.c_char_p
    lib.nvfp4v_last_hip_error.argtypes = [p]
    lib.nvfp4v_ctx_size.argtypes = []
    lib.nvfp4v_ctx_size.restype = c.c_size_t
    lib.nvfp4v_device_status.argtypes = [p]
    lib.nvfp4v_f16_redone.argtypes = [p, c.POINTER(c.c_uint64)]
    lib.nvfp4v_quantize_host.argtypes = [p, i64, i64, p, p]
    lib.nvfp4v_quantize.argtypes = [p, p, i64, i64, p, p, p]
    lib.nvfp4v_encode_e4m3_host.argtypes = [p, i64, p]
    lib.nvfp4v_packed_bytes.argtypes = [i64, i64]
    lib.nvfp4v_packed_bytes.restype = c.c_size_t
    lib.nvfp4v_pack.argtypes = [p, p, p, i64, i64, p, p]
    lib.nvfp4v_unpack.argtypes = [p, p, i64, i64, p, p, p]
    lib.nvfp4v_verify_gemm.argtypes = [p, p, i64, i64, p, i64, c.c_float, p, p]
    lib.nvfp4v_act_packed_bytes.argtypes = [i64, i64]
    lib.nvfp4v_act_packed_bytes.restype = c.c_size_t
    lib.nvfp4v_pack_activations.argtypes = [p, p, i64, i64, p, p]
    lib.nvfp4v_verify_gemm_pa.argtypes = [p, p, i64, i64, p, i64, c.c_float, p, p]
    lib.nvfp4v_verify_gemm_static.argtypes = [p, i64, i64, p, i64, c.c_float, p, p]
    lib.nvfp4v_describe_plan.argtypes = [p, i64, i64, i64, c.c_char_p, c.c_size_t]
    lib.nvfp4v_staircase.argtypes = [p, i64, i64, c.c_int, c.c_int, c.c_int, c.c_int,
                                     c.c_size_t, p]
    lib.nvfp4v_glue_scale.argtypes = [p, p, i64, i64, i64, c.c_float, p, p]
    lib.nvfp4v_glue_sum.argtypes = [p, p, i64, p, i64, i64, i64, c.c_float, p, p]
    lib.nvfp4v_pass_workspace_bytes.argtypes = [i64, i64, i64, c.c_int]
    lib.nvfp4v_pass_status.argtypes = [p]
    lib.nvfp4v_pass_error_site.argtypes = [p]
    lib.nvfp4v_last_pass_grid.argtypes = [p]
    lib.nvfp4v_set_pass_mode.argtypes = [p, c.c_int]
    lib.nvfp4v_get_pass_mode.argtypes = [p]
    lib.nvfp4v_pass_timeline.argtypes = [p, p, c.c_size_t, p, p]
    lib.nvfp4v_pass_workspace_bytes.restype = c.c_size_t
    lib.nvfp4v_verify_pass.argtypes = [p, p, c.c_int, i64, i64, p, i64, p, c.c_size_t, p, p, p]
    lib.nvfp4v_read_probe_sink_words.argtypes = [p]
    lib.nvfp4v_read_probe_sink_words.restype = c.c_size_t
    lib.nvfp4v_read_probe.argtypes = [p, p, c.c_size_t, p, p]
    lib.nvfp4v_copy_probe.argtypes = [p, p, p, c.c_size_t, p]
    lib.nvfp4v_fp8_packed_bytes.argtypes = [i64, i64]
    lib.nvfp4v_fp8_packed_bytes.restype = c.c_size_t
    lib.nvfp4v_fp8_quantize_host.argtypes = [p, i64, i64, p, p]
    lib.nvfp4v_fp8_pack_host.argtypes = [p, p, i64, i64, p]
    lib.nvfp4v_fp8_head_gemm.argtypes = [p, p, i64, i64, p, i64, p, p]
    lib.nvfp4v_fp8_head_gemm_pa.argtypes = [p, p, i64, i64, p, i64, p, p]
    lib.nvfp4v_staircut.argtypes = [p, c.c_int, p, p, c.c_int, p, c.c_int, p, p, p, p]
    lib.nvfp4v_kv_cache_bytes.argtypes = [i64, c.c_int, c.c_int]
    lib.nvfp4v_kv_cache_bytes.restype = c.c_size_t
    lib.nvfp4v_kv_write.argtypes = [p, p, p, i64, i64, c.c_int, c.c_int, i64, p, p, p]
    lib.nvfp4v_tree_attention_workspace_bytes.argtypes = [i64, i64, c.c_int, c.c_int, c.c_int]
    lib.nvfp4v_tree_attention_workspace_bytes.restype = c.c_size_t
    lib.nvfp4v_tree_attention.argtypes = [p, p, p, p, i64, i64, i64, c.c_int, c.c_int, c.c_int, p,
                                          c.c_float, p, p, c.c_size_t, p]
    lib.nvfp4v_tree_attention_plan.argtypes = [p, i64, i64, c.c_int, c.c_int, c.c_int, p, p]
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


def _nbytes(t):
    return t.numel() * t.element_size()


def _require(t, name, dtypes=None, shape=None, min_bytes=None):
    """Check a device tensor before its address crosses the C ABI: a CUDA
    tensor, contiguous, of one of `dtypes`, of exactly `shape`, and holding at
    least `min_bytes` bytes. The library checks pointers and sizes it is given;
    this checks that the tensor really is what those sizes describe."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor, got %s" % (name, type(t).__name__))
    if not t.is_cuda:
        raise ValueError("%s must be a device (cuda) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError("%s must have dtype %s, got %s" % (name, " or ".join(map(str, dtypes)), t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if min_bytes is not None and _nbytes(t) < min_bytes:
        raise ValueError("%s holds %d bytes, needs at least %d" % (name, _nbytes(t), min_bytes))
    return t


def _bf16_types():
    import torch

    return (torch.bfloat16, torch.int16, torch.uint16) if hasattr(torch, "uint16") else (torch.bfloat16, torch.int16)


def _f32():
    import torch

    return (torch.float32,)


def _u8():
    import torch

    return (torch.uint8,)


def packed_bytes(n: int, k: int) -> int:
    return int(load().nvfp4v_packed_bytes(int(n), int(k)))


def act_packed_bytes(m: int, k: int) -> int:
    return int(load().nvfp4v_act_packed_bytes(int(m), int(k)))


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


def fp8_packed_bytes(n: int, k: int) -> int:
    return int(load().nvfp4v_fp8_packed_bytes(int(n), int(k)))


def fp8_quantize_host(w):
    """fp32 numpy w[n, k] -> (E4M3 codes u8[n, k], fp32 row scales[n]) for the FP8 head."""
    import numpy as np

    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    codes = np.zeros((n, k), np.uint8)
    scales = np.zeros(n, np.float32)
    _check(load().nvfp4v_fp8_quantize_host(_np_ptr(w), n, k, _np_ptr(codes), _np_ptr(scales)),
           "nvfp4v_fp8_quantize_host")
    return codes, scales


def fp8_pack_host(codes, row_scales):
    """E4M3 codes u8[n, k] + fp32 row scales[n] -> packed head (host uint8 array)."""
    import numpy as np

    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    row_scales = np.ascontiguousarray(row_scales, dtype=np.float32)
    n, k = codes.shape
    nb = fp8_packed_bytes(n, k)
    if nb == 0 or row_scales.shape != (n,):
        raise Nvfp4vError(E_SHAPE, "fp8_pack_host")
    out = np.empty(nb, np.uint8)
    _check(load().nvfp4v_fp8_pack_host(_np_ptr(codes), _np_ptr(row_scales), n, k, _np_ptr(out)),
           "nvfp4v_fp8_pack_host")
    return out


def verify_gemm_static(a, packed, n: int, k: int, ts: float = 1.0, out=None, stream=None):
    """nvfp4v_verify_gemm_static: the verify GEMM without a context, for callers
    that cannot allocate (its scratch is a fixed device array of the library;
    calls must not overlap on one GPU). ``out`` must be given by callers that
    cannot allocate; without it a tensor is allocated here for convenience."""
    import torch

    m = a.shape[0]
    _require(a, "a", _bf16_types(), shape=(m, k))
    _require(packed, "packed", min_bytes=packed_bytes(n, k))
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=a.device)
    _require(out, "out", _f32(), shape=(m, n))
    _check(load().nvfp4v_verify_gemm_static(_t_ptr(a), m, k, _t_ptr(packed), n, float(ts), _t_ptr(out),
                                            _stream_handle(stream)), "nvfp4v_verify_gemm_static")
    return out


ATTN_HEAD_DIM = 128
ATTN_MAX_ROWS = 32


def kv_cache_bytes(cap: int, hkv: int, d: int = ATTN_HEAD_DIM) -> int:
    """Bytes of one key or value cache of `cap` positions (a multiple of 32)."""
    return int(load().nvfp4v_kv_cache_bytes(cap, hkv, d))


def tree_attention_workspace_bytes(ctx_len: int, m: int, hq: int, hkv: int, d: int = ATTN_HEAD_DIM) -> int:
    return int(load().nvfp4v_tree_attention_workspace_bytes(ctx_len, m, hq, hkv, d))


def staircut(us_by_rows, parent, p_accept, sizes=None):
    """StairCut's cut of a draft tree on a measured staircase (host code).

    us_by_rows[r - 1]: verify-pass microseconds at r rows; parent[v]: the
    parent of node v (-1: the root), parents before children; p_accept[v]: the
    probability that node v's token is accepted given its parent was; sizes:
    candidate node counts (None: 7, 15, 23, 31). Returns (n_keep, keep mask
    (uint8 per node), expected committed tokens, tokens per millisecond)."""
    import numpy as np

    us = np.ascontiguousarray(us_by_rows, dtype=np.float64)
    par = np.ascontiguousarray(parent, dtype=np.int32)
    p = np.ascontiguousarray(p_accept, dtype=np.float64)
    if par.shape != p.shape or par.ndim != 1:
        raise ValueError("parent and p_accept must be 1-D of one length")
    sz = None if sizes is None else np.ascontiguousarray(sizes, dtype=np.int32)
    keep = np.zeros(par.size, np.uint8)
    n_keep = ctypes.c_int32()
    e = ctypes.c_double()
    rate = ctypes.c_double()
    _check(load().nvfp4v_staircut(_np_ptr(us), us.size, _np_ptr(par), _np_ptr(p), par.size,
                                  None if sz is None else _np_ptr(sz), 0 if sz is None else sz.size,
                                  ctypes.byref(n_keep), _np_ptr(keep), ctypes.byref(e),
                                  ctypes.byref(rate)), "nvfp4v_staircut")
    return int(n_keep.value), keep, float(e.value), float(rate.value)


class Context:
    """An nvfp4v context on one GPU (owns the split-K workspace)."""

    def __init__(self, device: int = 0, tile_table: str = None):
        """tile_table: a tile-table file (None: the built-in gfx950 table)."""
        lib = load()
        h = ctypes.c_void_p()
        path = None if tile_table is None else os.fsencode(tile_table)
        _check(lib.nvfp4v_create(ctypes.byref(h), int(device), path), "nvfp4v_create")
        self._h = h
        self.device = device

    def load_tile_table(self, path: str = None) -> None:
        """Load a tile-table file (None: back to the built-in table alone)."""
        _check(load().nvfp4v_load_tile_table(self._h, None if path is None else os.fsencode(path)),
               "nvfp4v_load_tile_table")

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

    def device_status(self) -> int:
        """Synchronise; E_DISPATCH if some split-K row block's pieces ran on two XCDs, else 0."""
        return int(load().nvfp4v_device_status(self._h))

    def f16_redone(self) -> int:
        """Synchronise; GEMM work units computed again from the bf16 copy of their activations."""
        n = ctypes.c_uint64(0)
        _check(load().nvfp4v_f16_redone(self._h, ctypes.byref(n)), "nvfp4v_f16_redone")
        return int(n.value)

    def last_hip_error(self) -> int:
        return int(load().nvfp4v_last_hip_error(self._h))

    # -- format --------------------------------------------------------------
    def quantize(self, w, stream=None):
        """fp32 cuda tensor w[n, k] -> (codes u8[n, k/2], scales u8[n, k/16]) on the device."""
        import torch

        _require(w, "w", _f32())
        n, k = w.shape
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
        scales = torch.empty((n, k // 16), dtype=torch.uint8, device=w.device)
        _check(load().nvfp4v_quantize(self._h, _t_ptr(w), n, k, _t_ptr(codes), _t_ptr(scales),
                                      _stream_handle(stream)), "nvfp4v_quantize")
        return codes, scales

    def pack(self, codes, scales, n: int, k: int, out=None, stream=None):
        import torch

        nb = packed_bytes(n, k)
        _require(codes, "codes", _u8(), min_bytes=n * (k // 2))
        _require(scales, "scales", _u8(), min_bytes=n * (k // 16))
        if out is None:
            out = torch.empty(nb, dtype=torch.uint8, device=codes.device)
        _require(out, "out", min_bytes=nb)
        _check(load().nvfp4v_pack(self._h, _t_ptr(codes), _t_ptr(scales), n, k, _t_ptr(out),
                                  _stream_handle(stream)), "nvfp4v_pack")
        return out

    def unpack(self, packed, n: int, k: int, stream=None):
        import torch

        _require(packed, "packed", min_bytes=packed_bytes(n, k))
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
        _require(a, "a", _bf16_types(), shape=(m, k))
        _require(packed, "packed", min_bytes=packed_bytes(n, k))
        if out is None:
            out = torch.empty((m, n), dtype=torch.float32, device=a.device)
        _require(out, "out", _f32(), shape=(m, n))
        _check(load().nvfp4v_verify_gemm(self._h, _t_ptr(a), m, k, _t_ptr(packed), n,
                                         float(ts), _t_ptr(out), _stream_handle(stream)),
               "nvfp4v_verify_gemm")
        return out

    def pack_activations(self, a, k: int = None, out=None, stream=None):
        """bf16 cuda tensor a[m, k] -> packed activations (uint8 cuda tensor)."""
        import torch

        _require(a, "a", _bf16_types())
        m, k = a.shape
        if out is None:
            out = torch.empty(act_packed_bytes(m, k), dtype=torch.uint8, device=a.device)
        _require(out, "out", min_bytes=act_packed_bytes(m, k))
        _check(load().nvfp4v_pack_activations(self._h, _t_ptr(a), m, k, _t_ptr(out),
                                              _stream_handle(stream)), "nvfp4v_pack_activations")
        return out

    def verify_gemm_pa(self, act, m: int, k: int, packed, n: int, ts: float = 1.0, out=None,
                       stream=None):
        """verify_gemm with activations already packed by pack_activations."""
        import torch

        _require(act, "act", min_bytes=act_packed_bytes(m, k))
        _require(packed, "packed", min_bytes=packed_bytes(n, k))
        if out is None:
            out = torch.empty((m, n), dtype=torch.float32, device=act.device)
        _require(out, "out", _f32(), shape=(m, n))
        _check(load().nvfp4v_verify_gemm_pa(self._h, _t_ptr(act), m, k, _t_ptr(packed), n,
                                            float(ts), _t_ptr(out), _stream_handle(stream)),
               "nvfp4v_verify_gemm_pa")
        return out

    def fp8_head_gemm(self, a, packed, n: int, k: int, out=None, stream=None):
        """C[m, n] fp32 = A[m, k] (bf16 cuda tensor) * (s . W8)^T for the packed FP8 head."""
        import torch

        m = a.shape[0]
        _require(a, "a", _bf16_types(), shape=(m, k))
        _require(packed, "packed", min_bytes=fp8_packed_bytes(n, k))
        if out is None:
            out = torch.empty((m, n), dtype=torch.float32, device=a.device)
        _require(out, "out", _f32(), shape=(m, n))
        _check(load().nvfp4v_fp8_head_gemm(self._h, _t_ptr(a), m, k, _t_ptr(packed), n,
                                           _t_ptr(out), _stream_handle(stream)),
               "nvfp4v_fp8_head_gemm")
        return out

    def fp8_head_gemm_pa(self, act, m: int, k: int, packed, n: int, out=None, stream=None):
        """fp8_head_gemm with activations already packed by pack_activations."""
        import torch

        _require(act, "act", min_bytes=act_packed_bytes(m, k))
        _require(packed, "packed", min_bytes=fp8_packed_bytes(n, k))
        if out is None:
            out = torch.empty((m, n), dtype=torch.float32, device=act.device)
        _require(out, "out", _f32(), shape=(m, n))
        _check(load().nvfp4v_fp8_head_gemm_pa(self._h, _t_ptr(act), m, k, _t_ptr(packed), n,
                                              _t_ptr(out), _stream_handle(stream)),
               "nvfp4v_fp8_head_gemm_pa")
        return out

    # -- tree-verify attention ----------------------------------------------
    def tree_attention_plan(self, ctx_len: int, m: int, hq: int, hkv: int, d: int = ATTN_HEAD_DIM):
        """(chunks per key/value head, positions per chunk) of tree_attention on this GPU."""
        nch, chunk = ctypes.c_int(0), ctypes.c_int(0)
        _check(load().nvfp4v_tree_attention_plan(self._h, ctx_len, m, hq, hkv, d, ctypes.byref(nch),
                                                 ctypes.byref(chunk)), "nvfp4v_tree_attention_plan")
        return nch.value, chunk.value

    def kv_write(self, k_rows, v_rows, pos0: int, cap: int, k_cache, v_cache, stream=None):
        """Write keys / values bf16 [n, Hkv, 128] to cache positions pos0 .. pos0 + n - 1."""
        n, hkv, d = k_rows.shape
        _require(k_rows, "k_rows", _bf16_types(), shape=(n, hkv, d))
        _require(v_rows, "v_rows", _bf16_types(), shape=(n, hkv, d))
        nb = kv_cache_bytes(cap, hkv, d)
        if nb == 0:
            raise ValueError("bad cache shape: cap=%d (a positive multiple of 32), hkv=%d, d=%d (128)" % (cap, hkv, d))
        _require(k_cache, "k_cache", min_bytes=nb)
        _require(v_cache, "v_cache", min_bytes=nb)
        _check(load().nvfp4v_kv_write(self._h, _t_ptr(k_rows), _t_ptr(v_rows), n, pos0, hkv, d, cap,
                                      _t_ptr(k_cache), _t_ptr(v_cache), _stream_handle(stream)), "nvfp4v_kv_write")

    def tree_attention(self, q, k_cache, v_cache, cap: int, ctx_len: int, hkv: int, parent_rows,
                       scale: float = None, out=None, ws=None, stream=None):
        """O fp32 [M, Hq, 128] of the tree rows q (bf16 [M, Hq, 128]) against the cached
        context (positions 0..ctx_len-1) and their own root paths (parent_rows: M ints,
        -1 for row 0). `ws` (uint8, tree_attention_workspace_bytes, its first 1024 bytes
        zero before the first use) is allocated zeroed when not given."""
        import numpy as np
        import torch

        m, hq, d = q.shape
        _require(q, "q", _bf16_types(), shape=(m, hq, d))
        nb = kv_cache_bytes(cap, hkv, d)
        if nb == 0:
            raise ValueError("bad cache shape: cap=%d, hkv=%d, d=%d" % (cap, hkv, d))
        _require(k_cache, "k_cache", min_bytes=nb)
        _require(v_cache, "v_cache", min_bytes=nb)
        par = np.ascontiguousarray(np.asarray(parent_rows, dtype=np.int32))
        if par.shape != (m,):
            raise ValueError("parent_rows must hold one entry per tree row")
        wsb = tree_attention_workspace_bytes(ctx_len, m, hq, hkv, d)
        if wsb == 0:
            raise ValueError("bad attention shape: ctx_len=%d m=%d hq=%d hkv=%d d=%d" % (ctx_len, m, hq, hkv, d))
        if ws is None:
            ws = torch.zeros(wsb, dtype=torch.uint8, device=q.device)
        _require(ws, "ws", min_bytes=wsb)
        if out is None:
            out = torch.empty((m, hq, d), dtype=torch.float32, device=q.device)
        _require(out, "out", _f32(), shape=(m, hq, d))
        if scale is None:
            scale = 1.0 / float(np.sqrt(d))
        _check(load().nvfp4v_tree_attention(self._h, _t_ptr(q), _t_ptr(k_cache), _t_ptr(v_cache), cap, ctx_len, m,
                                            hq, hkv, d, _np_ptr(par), float(scale), _t_ptr(out), _t_ptr(ws),
                                            ws.numel() * ws.element_size(), _stream_handle(stream)),
               "nvfp4v_tree_attention")
        return out

    # -- chain glue and the full pass ---------------------------------------
    def glue_scale(self, x, c: float, out=None, stream=None):
        """bf16(x * c) for an fp32 cuda tensor x[rows, cols] (row stride x.stride(0))."""
        import torch

        if x.dtype != torch.float32 or x.dim() != 2 or x.stride(1) != 1 or not x.is_cuda:
            raise ValueError("x must be a 2-D fp32 cuda tensor with unit column stride")
        rows, cols = x.shape
        if out is None:
            out = torch.empty((rows, cols), dtype=torch.bfloat16, device=x.device)
        _require(out, "out", _bf16_types(), shape=(rows, cols))
        _check(load().nvfp4v_glue_scale(self._h, _t_ptr(x), x.stride(0), rows, cols, float(c),
                                        _t_ptr(out), _stream_handle(stream)), "nvfp4v_glue_scale")
        return out

    def glue_sum(self, x, y, c: float, out=None, stream=None):
        """bf16(x * c + y * c) for fp32 cuda tensors of one shape (no fused multiply-add)."""
        import torch

        for t, nm in ((x, "x"), (y, "y")):
            if t.dtype != torch.float32 or t.dim() != 2 or t.stride(1) != 1 or not t.is_cuda:
                raise ValueError("%s must be a 2-D fp32 cuda tensor with unit column stride" % nm)
        if tuple(y.shape) != tuple(x.shape):
            raise ValueError("x and y must have one shape")
        rows, cols = x.shape
        if out is None:
            out = torch.empty((rows, cols), dtype=torch.bfloat16, device=x.device)
        _require(out, "out", _bf16_types(), shape=(rows, cols))
        _check(load().nvfp4v_glue_sum(self._h, _t_ptr(x), x.stride(0), _t_ptr(y), y.stride(0),
                                      rows, cols, float(c), _t_ptr(out), _stream_handle(stream)),
               "nvfp4v_glue_sum")
        return out

    def verify_pass(self, layers, hidden: int, inter: int, h0, ws, h_out, trace=None,
                    stream=None):
        """Enqueue the chained pass; layers is a ctypes array of Layer."""
        m = h0.shape[0]
        _require(h0, "h0", _bf16_types(), shape=(m, hidden))
        _require(h_out, "h_out", _bf16_types(), shape=(m, hidden))
        _require(ws, "ws", min_bytes=pass_workspace_bytes(m, hidden, inter, len(layers)))
        if trace is not None:
            _require(trace, "trace", _bf16_types(), shape=(len(layers), m, hidden))
        _check(load().nvfp4v_verify_pass(
            self._h, ctypes.cast(layers, ctypes.c_void_p), len(layers), hidden, inter,
            _t_ptr(h0), m, _t_ptr(ws), ws.numel() * ws.element_size(), _t_ptr(h_out),
            _t_ptr(trace) if trace is not None else None, _stream_handle(stream)),
            "nvfp4v_verify_pass")
        return h_out

    def pass_status(self) -> int:
        """Synchronise; NVFP4V_OK, or E_TIMEOUT if the last pass gave up at a barrier."""
        return int(load().nvfp4v_pass_status(self._h))

    def pass_error_site(self) -> int:
        """Synchronise; where the last persistent pass gave up (0: it did not)."""
        return int(load().nvfp4v_pass_error_site(self._h))

    def set_pass_mode(self, mode: int) -> None:
        """PASS_CHAIN (four GEMM launches per layer) or PASS_PERSISTENT."""
        _check(load().nvfp4v_set_pass_mode(self._h, int(mode)), "set_pass_mode")

    def get_pass_mode(self) -> int:
        return int(load().nvfp4v_get_pass_mode(self._h))

    def last_pass_grid(self) -> int:
        return int(load().nvfp4v_last_pass_grid(self._h))

    def pass_timeline(self):
        """(start, done) real-time-clock stamps [phases, groups] of the last pass
        (context created with NVFP4V_PASS_TRACE=1)."""
        import numpy as np

        buf = np.zeros(2 * 1024 * 512, np.uint64)
        ph, gr = ctypes.c_int(), ctypes.c_int()
        _check(load().nvfp4v_pass_timeline(self._h, _np_ptr(buf), buf.size, ctypes.byref(ph),
                                           ctypes.byref(gr)), "nvfp4v_pass_timeline")
        t = buf.reshape(512, 1024, 2)[: ph.value, : gr.value]
        return t[:, :, 0], t[:, :, 1]

    # -- measurement helpers ------------------------------------------------
    def read_probe(self, buf, sink, stream=None):
        _check(load().nvfp4v_read_probe(self._h, _t_ptr(buf), buf.numel() * buf.element_size(),
                                        _t_ptr(sink), _stream_handle(stream)), "nvfp4v_read_probe")

    def read_probe_sink_words(self) -> int:
        return int(load().nvfp4v_read_probe_sink_words(self._h))

    def copy_probe(self, src, dst, stream=None):
        nb = src.numel() * src.element_size()
        _check(load().nvfp4v_copy_probe(self._h, _t_ptr(src), _t_ptr(dst), nb,
                                        _stream_handle(stream)), "nvfp4v_copy_probe")

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


class Layer(ctypes.Structure):
    """struct nvfp4v_layer: packed device pointers of one layer and their tensor scales."""

    _fields_ = [("qkv", ctypes.c_void_p), ("o", ctypes.c_void_p), ("gate_up", ctypes.c_void_p),
                ("down", ctypes.c_void_p), ("ts_qkv", ctypes.c_float), ("ts_o", ctypes.c_float),
                ("ts_gate_up", ctypes.c_float), ("ts_down", ctypes.c_float)]


def pass_workspace_bytes(m: int, hidden: int, inter: int, n_layers: int) -> int:
    return int(load().nvfp4v_pass_workspace_bytes(m, hidden, inter, n_layers))


def exported_names():
    """Function names declared in include/nvfp4v.h."""
    import re

    src = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"\b(nvfp4v_[a-z0-9_]+)\s*\(", src)))
