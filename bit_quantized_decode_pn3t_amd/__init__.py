"""PN (pn3t / pn4t) decode GEMV for AMD Instinct MI355X (gfx950).

The compute lives in libpn.so (hand-written HIP kernels behind the C ABI of
include/pn.h); ``_binding`` marshals arguments to it.  Importing this package
does not load the library; the first call does, and raises if it is missing.
"""
from ._binding import (PN_PN3T, PN_PN4T, PNError, Group, lib, pn_dequantize,  # noqa: F401
                       pn_gemm_smallm, pn_get_smallm_math, pn_gemv, pn_gemv2, pn_group_create,
                       pn_group_create_smallm, pn_last_variant, pn_row_bytes, pn_set_smallm_math,
                       pn_variant_name, pn_weights_per_block, status_str)
