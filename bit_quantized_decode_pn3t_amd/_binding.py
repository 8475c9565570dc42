"""ctypes binding of libpn.so (the C ABI in include/pn.h).

Argument marshalling only: every step of the product runs in the HIP
kernels.  Functions keep the C names.  Arrays may be torch tensors (their
data_ptr() is passed) or plain integer device addresses; ``stream`` defaults
to torch's current stream on the current device.

There is no fallback: if libpn.so is missing or fails to load, every call
raises.
"""
import ctypes
import os

PN_PN3T = 0
PN_PN4T = 1
TYPES = {"pn3t": PN_PN3T, "pn4t": PN_PN4T, PN_PN3T: PN_PN3T, PN_PN4T: PN_PN4T}

SMALLM_MATH = {"mfma": 0, "valu": 1, 0: 0, 1: 1}
GEMV_KERNEL = {"auto": 0, "stream": 1, "rows": 2, 0: 0, 1: 1, 2: 2}

STATUS = {0: "PN_OK", -1: "PN_EINVAL", -2: "PN_ESHAPE", -3: "PN_EALIGN",
          -4: "PN_EUNSUPPORTED", -5: "PN_ELAUNCH", -6: "PN_ENOMEM"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpn.so")

# Every symbol include/pn.h declares.
EXPORTS = ("pn_weights_per_block", "pn_row_bytes", "pn_gemv", "pn_gemv2",
           "pn_gemm_smallm", "pn_set_smallm_math", "pn_get_smallm_math", "pn_set_gemv_kernel",
           "pn_get_gemv_kernel", "pn_dequantize", "pn_rotate", "pn_gemm_prefill", "pn_gemm_prefill_group",
           "pn_group_create", "pn_group_create_smallm", "pn_group_run", "pn_group_destroy", "pn_gemv_batch",
           "pn_read_probe_scratch_bytes", "pn_read_probe", "pn_status_str", "pn_last_variant",
           "pn_variant_name")


class PNError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s returned %s (%d): %s" % (what, STATUS.get(status, "?"), status,
                                                     status_str(status)))


class pn_gemv_desc(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("type", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


DESC_ROTATE = 1  # PN_DESC_ROTATE
ROTATE_BLOCK = 1024  # PN_ROTATE_BLOCK


class pn_gemm_desc(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("X", ctypes.c_void_p), ("Y", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("ldx", ctypes.c_int64),
                ("ldy", ctypes.c_int64), ("type", ctypes.c_int32), ("M", ctypes.c_int32)]


_lib = None


def lib():
    """Load libpn.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libpn.so is not built (%s); run __graft_entry__.build() or "
                           "python bit_quantized_decode_pn3t_amd/build.py" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.pn_weights_per_block.argtypes = [i32]
    L.pn_weights_per_block.restype = i32
    L.pn_row_bytes.argtypes = [i32, i64]
    L.pn_row_bytes.restype = ctypes.c_size_t
    L.pn_gemv.argtypes = [i32, vp, i64, i64, vp, vp, vp]
    L.pn_gemv.restype = i32
    L.pn_gemv2.argtypes = [i32, vp, vp, i64, i64, vp, vp, vp, vp]
    L.pn_gemv2.restype = i32
    L.pn_gemm_smallm.argtypes = [i32, vp, i64, i64, vp, i64, i32, vp, i64, vp]
    L.pn_gemm_smallm.restype = i32
    L.pn_set_gemv_kernel.argtypes = [i32]
    L.pn_set_gemv_kernel.restype = i32
    L.pn_get_gemv_kernel.argtypes = []
    L.pn_get_gemv_kernel.restype = i32
    L.pn_set_smallm_math.argtypes = [i32]
    L.pn_set_smallm_math.restype = i32
    L.pn_get_smallm_math.argtypes = []
    L.pn_get_smallm_math.restype = i32
    L.pn_group_create_smallm.argtypes = [ctypes.POINTER(pn_gemm_desc), i32, ctypes.POINTER(vp)]
    L.pn_group_create_smallm.restype = i32
    L.pn_gemm_prefill_group.argtypes = [ctypes.POINTER(pn_gemm_desc), i32, vp]
    L.pn_gemm_prefill_group.restype = i32
    L.pn_dequantize.argtypes = [i32, vp, i64, i64, vp, vp]
    L.pn_dequantize.restype = i32
    L.pn_rotate.argtypes = [vp, i64, i32, i64, vp, i64, vp]
    L.pn_rotate.restype = i32
    L.pn_gemm_prefill.argtypes = [i32, vp, i64, i64, vp, i64, i64, vp, i64, vp]
    L.pn_gemm_prefill.restype = i32
    L.pn_group_create.argtypes = [ctypes.POINTER(pn_gemv_desc), i32, ctypes.POINTER(vp)]
    L.pn_group_create.restype = i32
    L.pn_group_run.argtypes = [vp, vp]
    L.pn_group_run.restype = i32
    L.pn_group_destroy.argtypes = [vp]
    L.pn_group_destroy.restype = None
    L.pn_gemv_batch.argtypes = [ctypes.POINTER(pn_gemv_desc), i32, vp]
    L.pn_gemv_batch.restype = i32
    L.pn_read_probe_scratch_bytes.argtypes = []
    L.pn_read_probe_scratch_bytes.restype = ctypes.c_size_t
    L.pn_read_probe.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t), vp]
    L.pn_read_probe.restype = i32
    L.pn_status_str.argtypes = [i32]
    L.pn_status_str.restype = ctypes.c_char_p
    L.pn_last_variant.argtypes = []
    L.pn_last_variant.restype = i32
    L.pn_variant_name.argtypes = [i32]
    L.pn_variant_name.restype = ctypes.c_char_p
    _lib = L
    return L


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _t(pn_type):
    return TYPES.get(pn_type, pn_type)


def _check(status, what):
    if status != 0:
        raise PNError(status, what)


def status_str(status):
    return lib().pn_status_str(status).decode()


def pn_weights_per_block(pn_type):
    return lib().pn_weights_per_block(_t(pn_type))


def pn_row_bytes(pn_type, K):
    return lib().pn_row_bytes(_t(pn_type), K)


def pn_gemv(pn_type, W, N, K, x, y, stream=None, check=True):
    st = lib().pn_gemv(_t(pn_type), _ptr(W), N, K, _ptr(x), _ptr(y), _stream(stream))
    if check:
        _check(st, "pn_gemv")
    return st


def pn_gemv2(pn_type, W0, W1, N, K, x, y0, y1, stream=None, check=True):
    st = lib().pn_gemv2(_t(pn_type), _ptr(W0), _ptr(W1), N, K, _ptr(x), _ptr(y0), _ptr(y1),
                        _stream(stream))
    if check:
        _check(st, "pn_gemv2")
    return st


def pn_gemm_smallm(pn_type, W, N, K, X, ldx, M, Y, ldy, stream=None, check=True):
    st = lib().pn_gemm_smallm(_t(pn_type), _ptr(W), N, K, _ptr(X), ldx, M, _ptr(Y), ldy,
                              _stream(stream))
    if check:
        _check(st, "pn_gemm_smallm")
    return st


def pn_set_smallm_math(math, check=True):
    """Select the small-M arithmetic: "mfma" (default) or "valu"."""
    st = lib().pn_set_smallm_math(SMALLM_MATH.get(math, math if isinstance(math, int) else -1))
    if check:
        _check(st, "pn_set_smallm_math")
    return st


def pn_get_smallm_math():
    return {0: "mfma", 1: "valu"}[lib().pn_get_smallm_math()]


def pn_set_gemv_kernel(kernel, check=True):
    """Select the M = 1 kernel: "auto" (row tiles for large launches),
    "stream" (register pipeline) or "rows" (row tiles wherever they apply).
    "stream" also keeps the small-M MFMA products on register loads; otherwise
    those whose rows are whole periods are staged through LDS by DMA."""
    st = lib().pn_set_gemv_kernel(GEMV_KERNEL.get(kernel, kernel if isinstance(kernel, int) else -1))
    if check:
        _check(st, "pn_set_gemv_kernel")
    return st


def pn_get_gemv_kernel():
    return {0: "auto", 1: "stream", 2: "rows"}[lib().pn_get_gemv_kernel()]


def pn_dequantize(pn_type, W, N, K, out, stream=None, check=True):
    st = lib().pn_dequantize(_t(pn_type), _ptr(W), N, K, _ptr(out), _stream(stream))
    if check:
        _check(st, "pn_dequantize")
    return st


def pn_gemm_prefill(pn_type, W, N, K, X, ldx, M, Y, ldy, stream=None, check=True):
    st = lib().pn_gemm_prefill(_t(pn_type), _ptr(W), N, K, _ptr(X), ldx, M, _ptr(Y), ldy, _stream(stream))
    if check:
        _check(st, "pn_gemm_prefill")
    return st


PREFILL_GROUP_MAX = 8  # PN_PREFILL_GROUP_MAX


def pn_gemm_prefill_group(problems, stream=None, check=True):
    """Run (pn_type, W, N, K, X, ldx, M, Y, ldy) prefill problems as one launch."""
    arr = (pn_gemm_desc * max(len(problems), 1))()
    for i, (t, W, N, K, X, ldx, M, Y, ldy) in enumerate(problems):
        arr[i] = pn_gemm_desc(_ptr(W), _ptr(X), _ptr(Y), N, K, ldx, ldy, _t(t), M)
    st = lib().pn_gemm_prefill_group(arr, len(problems), _stream(stream))
    if check:
        _check(st, "pn_gemm_prefill_group")
    return st


def pn_rotate(x, K, M, ldx, out, ldo, stream=None, check=True):
    st = lib().pn_rotate(_ptr(x), K, M, ldx, _ptr(out), ldo, _stream(stream))
    if check:
        _check(st, "pn_rotate")
    return st


class Group:
    """A pn_group plan over (pn_type, W, N, K, x, y) problems; frees itself.
    With smallm=True the problems are (pn_type, W, N, K, X, ldx, M, Y, ldy)
    and the plan comes from pn_group_create_smallm.  `rotate` (GEMV plans):
    one flag per problem, or one for all, for PN_DESC_ROTATE."""

    def __init__(self, problems, smallm=False, rotate=False):
        h = ctypes.c_void_p()
        if smallm:
            arr = (pn_gemm_desc * len(problems))()
            for i, (t, W, N, K, X, ldx, M, Y, ldy) in enumerate(problems):
                arr[i] = pn_gemm_desc(_ptr(W), _ptr(X), _ptr(Y), N, K, ldx, ldy, _t(t), M)
            _check(lib().pn_group_create_smallm(arr, len(problems), ctypes.byref(h)),
                   "pn_group_create_smallm")
        else:
            arr = (pn_gemv_desc * len(problems))()
            flags = list(rotate) if isinstance(rotate, (list, tuple)) else [rotate] * len(problems)
            for i, (t, W, N, K, x, y) in enumerate(problems):
                arr[i] = pn_gemv_desc(_ptr(W), _ptr(x), _ptr(y), N, K, _t(t),
                                      DESC_ROTATE if flags[i] else 0)
            _check(lib().pn_group_create(arr, len(problems), ctypes.byref(h)), "pn_group_create")
        self.handle = h
        self.keep = problems  # the plan holds raw device pointers

    def run(self, stream=None):
        _check(lib().pn_group_run(self.handle, _stream(stream)), "pn_group_run")

    def close(self):
        if self.handle:
            lib().pn_group_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def pn_group_create(problems):
    return Group(problems)


def pn_group_create_smallm(problems):
    return Group(problems, smallm=True)


BATCH_MAX_PROBLEMS = 32  # PN_BATCH_MAX_PROBLEMS
BATCH_MAX_ROWS = 65536 * 16  # PN_BATCH_MAX_ROWS


def pn_gemv_batch(problems, stream=None, check=True):
    """Run (pn_type, W, N, K, x, y) problems as one launch with no plan and no
    allocation (the library's static per-device batch buffer holds the plan)."""
    arr = (pn_gemv_desc * max(len(problems), 1))()
    for i, (t, W, N, K, x, y) in enumerate(problems):
        arr[i] = pn_gemv_desc(_ptr(W), _ptr(x), _ptr(y), N, K, _t(t), 0)
    st = lib().pn_gemv_batch(arr, len(problems), _stream(stream))
    if check:
        _check(st, "pn_gemv_batch")
    return st


def pn_read_probe_scratch_bytes():
    return lib().pn_read_probe_scratch_bytes()


def pn_read_probe(buf, nbytes, scratch, scratch_bytes, stream=None, check=True):
    """Launch the streaming-read probe; returns the number of bytes it reads."""
    got = ctypes.c_size_t(0)
    st = lib().pn_read_probe(_ptr(buf), nbytes, _ptr(scratch), scratch_bytes, ctypes.byref(got),
                             _stream(stream))
    if check:
        _check(st, "pn_read_probe")
    return got.value


def pn_last_variant():
    return lib().pn_last_variant()


def pn_variant_name(v):
    return lib().pn_variant_name(v).decode()
