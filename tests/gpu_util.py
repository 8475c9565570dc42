"""Helpers for the GPU parity tests (test helper)."""
import sys

import numpy as np

TOL = 1e-5  # max |y - y_ref| <= TOL * sum_k |w x|, row by row


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def sync():
    import torch
    torch.cuda.synchronize()


def f32_bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def assert_bits_equal(got, want, what=""):
    got = np.asarray(got, np.float32).reshape(-1)
    want = np.asarray(want, np.float32).reshape(-1)
    nan = np.isnan(got) & np.isnan(want)
    bad = ~nan & (f32_bits(got) != f32_bits(want))
    if bad.any():
        i = int(np.nonzero(bad)[0][0])
        raise AssertionError("%s: %d of %d values differ in bits; first at %d: %r (%08x) vs %r (%08x)" % (
            what, int(bad.sum()), bad.size, i, got[i], f32_bits(got)[i], want[i], f32_bits(want)[i]))


def assert_gemv_close(y, y64, a, what="", tol=TOL):
    """Row by row: |y - y64| <= tol * a; a row with a = 0 must be exactly +-0."""
    y = np.asarray(y, np.float64)
    err = np.abs(y - y64)
    bound = tol * a
    bad = ~(err <= bound)
    zero_rows = a == 0
    bad |= zero_rows & (y != 0)
    if bad.any():
        i = int(np.nonzero(bad.reshape(-1))[0][0])
        raise AssertionError("%s: %d of %d rows outside %g*sum|wx|; first flat index %d: y=%r ref=%r a=%r" % (
            what, int(bad.sum()), bad.size, tol, i, y.reshape(-1)[i], y64.reshape(-1)[i], a.reshape(-1)[i]))
    return float((err / np.where(a > 0, a, 1)).max()) if err.size else 0.0
