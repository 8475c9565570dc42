"""The C-ABI library loads and exports every symbol include/pn.h declares;
host-side argument checks fail with the documented status before any launch.
CPU only: no call here reaches the GPU."""
import ctypes
import os
import re

import pytest

from bit_quantized_decode_pn3t_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pn.h")

PN_EINVAL, PN_ESHAPE, PN_EALIGN = -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_binding_exports():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        ctypes.cast(getattr(lib, name), ctypes.c_void_p)


def test_host_helpers():
    assert B.pn_weights_per_block("pn3t") == 80
    assert B.pn_weights_per_block("pn4t") == 64
    assert B.pn_weights_per_block(7) == 0
    assert B.pn_row_bytes("pn3t", 5120) == 64 * 34
    assert B.pn_row_bytes("pn4t", 17408) == 272 * 34
    assert B.pn_row_bytes("pn4t", 6144) == 96 * 34
    assert B.pn_row_bytes("pn3t", 6144) == 0
    assert B.pn_row_bytes("pn3t", 0) == 0
    assert "ok" in B.status_str(0)
    assert B.pn_variant_name(B.pn_last_variant()) == "none"


def test_variant_names():
    """Every kernel the library can report has its own name; unknown ids are
    reported as such rather than as a kernel."""
    names = [B.pn_variant_name(v) for v in range(18)]
    assert names[0] == "none"
    assert len(set(names)) == len(names), names
    for expect in ("gemv_rows", "gemv_rows_group", "gemv_stream", "gemv_stream_group", "gemv_generic",
                   "gemm_stream_mfma", "gemm_stream_valu", "gemm_stream_mfma_group", "gemm_stream_valu_group",
                   "gemm_rows_mfma", "gemm_rows_mfma_group", "gemm_prefill", "hadamard_rotate", "dequant",
                   "gemv_rows_batch", "gemv_stream_batch", "gemm_prefill_group"):
        assert expect in names, expect
    assert B.pn_variant_name(18) not in names[1:]
    assert B.pn_variant_name(-1) not in names[1:]


FAKE = 0x10000  # never dereferenced: every call below fails its host checks


@pytest.mark.parametrize("args,status", [
    (("pn3t", None, 4, 80, FAKE, FAKE), PN_EINVAL),
    ((9, FAKE, 4, 80, FAKE, FAKE), PN_EINVAL),
    (("pn3t", FAKE, 0, 80, FAKE, FAKE), PN_ESHAPE),
    (("pn3t", FAKE, 4, 81, FAKE, FAKE), PN_ESHAPE),
    (("pn3t", FAKE, 4, 64, FAKE, FAKE), PN_ESHAPE),
    (("pn4t", FAKE, 4, 0, FAKE, FAKE), PN_ESHAPE),
    (("pn3t", FAKE + 1, 4, 80, FAKE, FAKE), PN_EALIGN),
    (("pn3t", FAKE, 4, 80, FAKE + 2, FAKE), PN_EALIGN),
    (("pn3t", FAKE, 4, 80, FAKE, FAKE + 2), PN_EALIGN),
    (("pn3t", FAKE, 4, 80, None, FAKE), PN_EINVAL),
])
def test_gemv_host_checks(args, status):
    assert B.pn_gemv(*args, stream=0, check=False) == status


def test_other_entry_points_host_checks():
    assert B.pn_gemv2("pn3t", FAKE, None, 4, 80, FAKE, FAKE, FAKE, stream=0, check=False) == PN_EINVAL
    assert B.pn_gemv2("pn4t", FAKE, FAKE, 4, 80, FAKE, FAKE, FAKE, stream=0, check=False) == PN_ESHAPE
    assert B.pn_gemm_smallm("pn3t", FAKE, 4, 80, FAKE, 80, 17, FAKE, 4, stream=0, check=False) == PN_ESHAPE
    assert B.pn_gemm_smallm("pn3t", FAKE, 4, 80, FAKE, 80, 0, FAKE, 4, stream=0, check=False) == PN_ESHAPE
    assert B.pn_gemm_smallm("pn3t", FAKE, 4, 80, FAKE, 79, 2, FAKE, 4, stream=0, check=False) == PN_ESHAPE
    assert B.pn_gemm_smallm("pn3t", FAKE, 4, 80, FAKE, 81, 2, FAKE, 4, stream=0, check=False) == PN_ESHAPE
    assert B.pn_gemm_smallm("pn3t", FAKE, 4, 80, FAKE, 80, 2, FAKE, 3, stream=0, check=False) == PN_ESHAPE
    assert B.pn_dequantize("pn4t", FAKE, 4, 64, FAKE + 1, stream=0, check=False) == PN_EALIGN
    assert B.pn_dequantize("pn4t", FAKE, 4, 100, FAKE, stream=0, check=False) == PN_ESHAPE
    with pytest.raises(B.PNError):
        B.pn_gemv("pn3t", FAKE, 4, 81, FAKE, FAKE, stream=0)


def test_group_host_checks():
    with pytest.raises(B.PNError) as e:
        B.Group([("pn3t", FAKE, 4, 81, FAKE, FAKE)])
    assert e.value.status == PN_ESHAPE
    with pytest.raises(B.PNError) as e:
        B.Group([("pn3t", FAKE, 4, 640, FAKE, FAKE), ("pn4t", FAKE + 1, 4, 512, FAKE, FAKE)])
    assert e.value.status == PN_EALIGN
    with pytest.raises(B.PNError) as e:  # rows of 3 blocks: not whole 8-block passes
        B.Group([("pn3t", FAKE, 4, 240, FAKE, FAKE)])
    assert e.value.status == -4
    lib = B.lib()
    h = ctypes.c_void_p()
    assert lib.pn_group_create(None, 1, ctypes.byref(h)) == PN_EINVAL
    assert lib.pn_group_run(None, None) == PN_EINVAL
    lib.pn_group_destroy(None)


def test_batch_host_checks():
    """pn_gemv_batch refuses, before anything reaches the GPU, a bad count,
    more problems than its buffer holds, rotated inputs and the checks of
    pn_group_create."""
    lib = B.lib()
    ok = ("pn3t", FAKE, 4, 640, FAKE, FAKE)
    assert lib.pn_gemv_batch(None, 1, None) == PN_EINVAL
    assert B.pn_gemv_batch([], stream=0, check=False) == PN_EINVAL
    assert B.pn_gemv_batch([ok] * (B.BATCH_MAX_PROBLEMS + 1), stream=0, check=False) == -4
    assert B.pn_gemv_batch([ok, ("pn3t", FAKE, 4, 81, FAKE, FAKE)], stream=0, check=False) == PN_ESHAPE
    assert B.pn_gemv_batch([ok, ("pn4t", FAKE + 1, 4, 512, FAKE, FAKE)], stream=0, check=False) == PN_EALIGN
    assert B.pn_gemv_batch([ok, ("pn3t", FAKE, 4, 640, None, FAKE)], stream=0, check=False) == PN_EINVAL
    assert B.pn_gemv_batch([("pn3t", FAKE, 4, 240, FAKE, FAKE)], stream=0, check=False) == -4
    arr = (B.pn_gemv_desc * 1)()
    arr[0] = B.pn_gemv_desc(FAKE, FAKE, FAKE, 4, 5120, 0, B.DESC_ROTATE)
    assert lib.pn_gemv_batch(arr, 1, None) == -4
    arr[0] = B.pn_gemv_desc(FAKE, FAKE, FAKE, 4, 5120, 0, 2)
    assert lib.pn_gemv_batch(arr, 1, None) == PN_EINVAL


def test_prefill_host_checks():
    lib = B.lib()
    X16 = 0x10000  # 16-byte aligned, never dereferenced
    ok = dict(t=0, W=FAKE, N=4, K=640, X=X16, ldx=640, M=3, Y=FAKE, ldy=4)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.pn_gemm_prefill(a["t"], a["W"], a["N"], a["K"], a["X"], a["ldx"], a["M"], a["Y"], a["ldy"], None)
    assert call(t=7) == PN_EINVAL
    assert call(W=None) == PN_EINVAL
    assert call(X=None) == PN_EINVAL
    assert call(Y=None) == PN_EINVAL
    assert call(K=81) == PN_ESHAPE
    assert call(M=0) == PN_ESHAPE
    assert call(ldx=320) == PN_ESHAPE
    assert call(ldy=3) == PN_ESHAPE
    assert call(K=80 * 3, ldx=240) == -4  # an odd number of blocks
    assert call(t=1, K=64 * 5, ldx=320) == -4
    assert call(W=FAKE + 2) == PN_EALIGN
    assert call(X=X16 + 8) == PN_EALIGN
    assert call(ldx=644) == PN_EALIGN
    assert call(Y=FAKE + 2) == PN_EALIGN
    # rows whose 256-row tile spans 2 GiB or more would overflow the kernel's
    # 32-bit offsets: refused before any launch, never wrapped
    big = 80 * 2 * 126_400  # pn3t, an even number of blocks, 256 rows x 8.6 MB
    assert call(K=big, ldx=big) == -4
    assert call(t=1, K=64 * 2 * 126_400, ldx=64 * 2 * 126_400) == -4


def test_prefill_group_host_checks():
    """pn_gemm_prefill_group: the count bounds, and each entry checked as
    pn_gemm_prefill checks it, before anything is enqueued."""
    lib = B.lib()
    X16 = 0x10000
    ok = ("pn3t", FAKE, 4, 640, X16, 640, 3, FAKE, 4)
    assert lib.pn_gemm_prefill_group(None, 1, None) == PN_EINVAL
    assert B.pn_gemm_prefill_group([], stream=0, check=False) == PN_EINVAL
    assert B.pn_gemm_prefill_group([ok] * (B.PREFILL_GROUP_MAX + 1), stream=0, check=False) == PN_EINVAL
    bad = [(("pn3t", FAKE, 4, 81, X16, 81, 3, FAKE, 4), PN_ESHAPE),
           (("pn3t", FAKE, 4, 640, X16, 640, 0, FAKE, 4), PN_ESHAPE),
           (("pn3t", FAKE, 4, 240, X16, 240, 3, FAKE, 4), -4),
           (("pn3t", FAKE, 4, 640, X16 + 8, 640, 3, FAKE, 4), PN_EALIGN),
           (("pn3t", FAKE, 4, 640, X16, 640, 3, None, 4), PN_EINVAL)]
    for entry, status in bad:
        # the failing entry last, after valid ones: still nothing runs
        assert B.pn_gemm_prefill_group([ok, ok, entry], stream=0, check=False) == status, entry
        assert B.pn_gemm_prefill_group([entry], stream=0, check=False) == status, entry


def test_rotate_host_checks():
    lib = B.lib()
    assert lib.pn_rotate(None, 1024, 1, 1024, FAKE, 1024, None) == PN_EINVAL
    assert lib.pn_rotate(FAKE, 1024, 1, 1024, None, 1024, None) == PN_EINVAL
    for k, m, ldx, ldo in ((1000, 1, 1000, 1000), (512, 1, 512, 512), (0, 1, 0, 0), (1024, 0, 1024, 1024),
                           (1024, 1, 1023, 1024), (2048, 2, 2048, 1024)):
        assert lib.pn_rotate(FAKE, k, m, ldx, FAKE, ldo, None) == PN_ESHAPE, (k, m, ldx, ldo)
    assert lib.pn_rotate(FAKE + 2, 1024, 1, 1024, FAKE, 1024, None) == PN_EALIGN
    assert lib.pn_rotate(FAKE, 1024, 2, 1026, FAKE + 2, 1025, None) == PN_EALIGN
    # group entries: unknown flag bits, and rotation of K not a multiple of 1024
    arr = (B.pn_gemv_desc * 1)()
    arr[0] = B.pn_gemv_desc(FAKE, FAKE, FAKE, 4, 5120, 0, 2)
    h = ctypes.c_void_p()
    assert lib.pn_group_create(arr, 1, ctypes.byref(h)) == PN_EINVAL
    with pytest.raises(B.PNError) as e:
        B.Group([("pn3t", FAKE, 4, 640, FAKE, FAKE)], rotate=True)
    assert e.value.status == PN_ESHAPE
    with pytest.raises(B.PNError) as e:
        B.Group([("pn3t", FAKE, 4, 5120, FAKE + 2, FAKE)], rotate=True)
    assert e.value.status == PN_EALIGN


def test_smallm_group_host_checks():
    ok = ("pn3t", FAKE, 4, 80, FAKE, 80, 2, FAKE, 4)
    bad = [
        (("pn3t", FAKE, 4, 80, FAKE, 80, 17, FAKE, 4), PN_ESHAPE),     # M > 16
        (("pn3t", FAKE, 4, 80, FAKE, 81, 2, FAKE, 4), PN_ESHAPE),      # odd ldx
        (("pn4t", FAKE, 4, 80, FAKE, 80, 2, FAKE, 4), PN_ESHAPE),      # K not whole pn4t blocks
        (("pn3t", FAKE, 4, 80, FAKE + 2, 80, 2, FAKE, 4), PN_EALIGN),  # X
        (("pn3t", FAKE, 4, 80, FAKE, 80, 2, None, 4), PN_EINVAL),
    ]
    for args, status in bad:
        with pytest.raises(B.PNError) as e:
            B.Group([ok, args], smallm=True)
        assert e.value.status == status, args
    lib = B.lib()
    h = ctypes.c_void_p()
    assert lib.pn_group_create_smallm(None, 1, ctypes.byref(h)) == PN_EINVAL


def _in_thread(fn):
    import threading
    out = {}
    t = threading.Thread(target=lambda: out.setdefault("v", fn()))
    t.start()
    t.join()
    return out["v"]


def test_smallm_math_setting():
    """The arithmetic selection belongs to the calling host thread."""
    assert B.pn_get_smallm_math() == "mfma"
    assert B.pn_set_smallm_math(7, check=False) == PN_EINVAL
    assert B.pn_get_smallm_math() == "mfma"
    B.pn_set_smallm_math("valu")
    try:
        assert B.pn_get_smallm_math() == "valu"
        # another thread starts from the default and its choice stays its own
        assert _in_thread(B.pn_get_smallm_math) == "mfma"
        assert _in_thread(lambda: (B.pn_set_smallm_math("mfma"), B.pn_get_smallm_math())[1]) == "mfma"
        assert B.pn_get_smallm_math() == "valu"
    finally:
        B.pn_set_smallm_math("mfma")
    assert B.pn_get_smallm_math() == "mfma"


def test_gemv_kernel_setting():
    """The M = 1 kernel selection belongs to the calling host thread."""
    assert B.pn_get_gemv_kernel() == "auto"
    assert B.pn_set_gemv_kernel(5, check=False) == PN_EINVAL
    assert B.pn_get_gemv_kernel() == "auto"
    B.pn_set_gemv_kernel("stream")
    try:
        assert B.pn_get_gemv_kernel() == "stream"
        assert _in_thread(B.pn_get_gemv_kernel) == "auto"
        assert _in_thread(lambda: (B.pn_set_gemv_kernel("rows"), B.pn_get_gemv_kernel())[1]) == "rows"
        assert B.pn_get_gemv_kernel() == "stream"
        B.pn_set_gemv_kernel("rows")
        assert B.pn_get_gemv_kernel() == "rows"
    finally:
        B.pn_set_gemv_kernel("auto")
    assert B.pn_get_gemv_kernel() == "auto"
