"""ctypes wrapper over the C oracle (libpnref.so), numpy in / numpy out.

Test infrastructure only: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.
"""
import ctypes
import os

import numpy as np

from . import build as _build

PN3T = 0
PN4T = 1
ROTATE_BLOCK = 1024  # Hadamard block of the activation rotation (reading in pnref.c)
BLOCK_BYTES = 34
_TYPES = {"pn3t": PN3T, "pn4t": PN4T, PN3T: PN3T, PN4T: PN4T}


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _t(pn_type):
    return _TYPES[pn_type]


def _check(st, what):
    if st != 0:
        raise ValueError("%s failed with status %d" % (what, st))


def _as_bytes(w):
    w = np.ascontiguousarray(w)
    if w.dtype != np.uint8:
        w = w.view(np.uint8)
    return w.reshape(-1)


class Oracle:
    """One loaded copy of the C oracle.  ``path`` selects the shared object."""

    def __init__(self, path=None):
        path = path or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        lib = ctypes.CDLL(path)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.pnref_half_to_float.restype = ctypes.c_float
        lib.pnref_half_to_float.argtypes = [ctypes.c_uint16]
        lib.pnref_double_to_half.restype = ctypes.c_uint16
        lib.pnref_double_to_half.argtypes = [ctypes.c_double]
        lib.pnref_decode_block.argtypes = [ctypes.c_int, u8p, f32p]
        lib.pnref_dequantize.argtypes = [ctypes.c_int, u8p, i64, i64, f32p]
        lib.pnref_gemv_f64.argtypes = [ctypes.c_int, u8p, i64, i64, u16p, f64p, f64p]
        lib.pnref_gemm_f64.argtypes = [ctypes.c_int, u8p, i64, i64, u16p, i64,
                                       ctypes.c_int, f64p, i64, f64p]
        lib.pnref_quantize.argtypes = [ctypes.c_int, f32p, i64, i64, u8p]
        lib.pnref_set_threads.argtypes = [ctypes.c_int]
        lib.pnref_rotate.argtypes = [u16p, i64, i64, u16p]
        lib.pnref_weights_per_block.argtypes = [ctypes.c_int]
        lib.pnref_zero_point.argtypes = [ctypes.c_int]
        self.lib = lib
        self.path = path

    def weights_per_block(self, pn_type):
        return self.lib.pnref_weights_per_block(_t(pn_type))

    def zero_point(self, pn_type):
        return self.lib.pnref_zero_point(_t(pn_type))

    def row_bytes(self, pn_type, k):
        return (k // self.weights_per_block(pn_type)) * BLOCK_BYTES

    def set_threads(self, n):
        """Set the OpenMP thread count of the fp64 GEMV; returns the count in use."""
        return self.lib.pnref_set_threads(int(n))

    def half_to_float(self, bits):
        return self.lib.pnref_half_to_float(int(bits))

    def double_to_half(self, v):
        return self.lib.pnref_double_to_half(float(v))

    def decode_block(self, pn_type, blk):
        blk = _as_bytes(blk)
        if blk.size < BLOCK_BYTES:
            raise ValueError("block needs 34 bytes")
        out = np.empty(self.weights_per_block(pn_type), np.float32)
        _check(self.lib.pnref_decode_block(_t(pn_type), _ptr(blk, ctypes.c_uint8),
                                           _ptr(out, ctypes.c_float)), "decode_block")
        return out

    def dequantize(self, pn_type, w, n, k):
        w = _as_bytes(w)
        if w.size < n * self.row_bytes(pn_type, k):
            raise ValueError("weight buffer too small")
        out = np.empty((n, k), np.float32)
        _check(self.lib.pnref_dequantize(_t(pn_type), _ptr(w, ctypes.c_uint8), n, k,
                                         _ptr(out, ctypes.c_float)), "dequantize")
        return out

    def gemv_f64(self, pn_type, w, n, k, x):
        """Return (y64, abs_sum) for y = W x with W packed and x fp16."""
        w = _as_bytes(w)
        x = np.ascontiguousarray(x, dtype=np.float16).view(np.uint16)
        if w.size < n * self.row_bytes(pn_type, k) or x.size < k:
            raise ValueError("buffer too small")
        y = np.empty(n, np.float64)
        a = np.empty(n, np.float64)
        _check(self.lib.pnref_gemv_f64(_t(pn_type), _ptr(w, ctypes.c_uint8), n, k,
                                       _ptr(x, ctypes.c_uint16), _ptr(y, ctypes.c_double),
                                       _ptr(a, ctypes.c_double)), "gemv_f64")
        return y, a

    def gemm_f64(self, pn_type, w, n, k, xm):
        """Return (Y64 [M,N], abs_sum [M,N]) for Y = X W^T with X fp16 [M,K]."""
        w = _as_bytes(w)
        xm = np.ascontiguousarray(xm, dtype=np.float16)
        m = xm.shape[0]
        if xm.shape[1] != k:
            raise ValueError("X must be [M, K]")
        if w.size < n * self.row_bytes(pn_type, k):
            raise ValueError("weight buffer too small")
        xb = xm.view(np.uint16)
        y = np.empty((m, n), np.float64)
        a = np.empty((m, n), np.float64)
        _check(self.lib.pnref_gemm_f64(_t(pn_type), _ptr(w, ctypes.c_uint8), n, k,
                                       _ptr(xb, ctypes.c_uint16), k, m,
                                       _ptr(y, ctypes.c_double), n,
                                       _ptr(a, ctypes.c_double)), "gemm_f64")
        return y, a

    def rotate(self, x, block=ROTATE_BLOCK):
        """Blockwise Hadamard rotation of fp16 rows: x fp16 [..., K] -> fp16
        [..., K] (pnref_rotate on each row)."""
        x = np.ascontiguousarray(x, dtype=np.float16)
        k = x.shape[-1]
        flat = x.reshape(-1, k).view(np.uint16)
        out = np.empty_like(flat)
        for r in range(flat.shape[0]):
            _check(self.lib.pnref_rotate(_ptr(flat[r], ctypes.c_uint16), k, block,
                                         _ptr(out[r], ctypes.c_uint16)), "rotate")
        return out.view(np.float16).reshape(x.shape)

    def quantize(self, pn_type, wf, n, k):
        """Quantize fp32 [N, K] into packed PN rows (uint8 [N, row_bytes])."""
        wf = np.ascontiguousarray(wf, dtype=np.float32).reshape(n, k)
        out = np.zeros((n, self.row_bytes(pn_type, k)), np.uint8)
        _check(self.lib.pnref_quantize(_t(pn_type), _ptr(wf, ctypes.c_float), n, k,
                                       _ptr(out, ctypes.c_uint8)), "quantize")
        return out


_default = None


def default():
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def weights_per_block(pn_type):
    return default().weights_per_block(pn_type)


def zero_point(pn_type):
    return default().zero_point(pn_type)


def row_bytes(pn_type, k):
    return default().row_bytes(pn_type, k)


def set_threads(n):
    return default().set_threads(n)


def half_to_float(bits):
    return default().half_to_float(bits)


def double_to_half(v):
    return default().double_to_half(v)


def decode_block(pn_type, blk):
    return default().decode_block(pn_type, blk)


def dequantize(pn_type, w, n, k):
    return default().dequantize(pn_type, w, n, k)


def gemv_f64(pn_type, w, n, k, x):
    return default().gemv_f64(pn_type, w, n, k, x)


def gemm_f64(pn_type, w, n, k, xm):
    return default().gemm_f64(pn_type, w, n, k, xm)


def quantize(pn_type, wf, n, k):
    return default().quantize(pn_type, wf, n, k)


def rotate(x, block=ROTATE_BLOCK):
    return default().rotate(x, block)
