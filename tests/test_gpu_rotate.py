"""Parity of the activation rotation against the CPU oracle: pn_rotate's
fp16 outputs bit for bit (the rotation is exact up to one fp16 rounding, so
every correct implementation gives the same bits), and group plans with
PN_DESC_ROTATE inputs within 1e-5 * sum|w x| row by row, on every kernel
choice."""
import numpy as np
import pytest

from gpu_util import assert_gemv_close, dev, say, sync

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from bit_quantized_decode_pn3t_amd import _binding as B  # noqa: E402
from bit_quantized_decode_pn3t_amd import synth  # noqa: E402
from oracle import pnref  # noqa: E402


def assert_half_bits_equal(got, want, what):
    got = np.asarray(got, np.float16).reshape(-1)
    want = np.asarray(want, np.float16).reshape(-1)
    nan = np.isnan(got) & np.isnan(want)
    bad = ~nan & (got.view(np.uint16) != want.view(np.uint16))
    if bad.any():
        i = int(np.nonzero(bad)[0][0])
        raise AssertionError("%s: %d of %d values differ; first at %d: %r (%04x) vs %r (%04x)" % (
            what, int(bad.sum()), bad.size, i, got[i], got.view(np.uint16)[i], want[i], want.view(np.uint16)[i]))


def gpu_rotate(x, ldx=None, ldo=None, inplace=False):
    """x: fp16 [M, K] on the host.  Rows ldx / ldo elements apart on the GPU."""
    m, k = x.shape
    ldx = ldx or k
    ldo = ldo or k
    xb = torch.zeros(m * ldx, dtype=torch.float16, device="cuda")
    xb.view(m, ldx)[:, :k] = dev(x)
    if inplace:
        out, ldo = xb, ldx
    else:
        out = torch.full((m * ldo,), float("nan"), dtype=torch.float16, device="cuda")
    B.pn_rotate(xb, k, m, ldx, out, ldo)
    sync()
    assert B.pn_variant_name(B.pn_last_variant()) == "hadamard_rotate"
    return out.view(m, ldo)[:, :k].cpu().numpy()


def activations(kind, rs, m, k):
    if kind == "normal":
        x = rs.standard_normal((m, k))
    elif kind == "wide":  # every fp16 binade, subnormals included
        x = rs.standard_normal((m, k)) * np.exp2(rs.integers(-24, 15, (m, k)))
    elif kind == "tiny":  # results that are fp16 subnormals or round to +-0
        x = rs.standard_normal((m, k)) * 2.0 ** -19
    elif kind == "huge":  # results that overflow fp16
        x = rs.uniform(40000, 65504, (m, k)) * rs.choice([-1, 1], (m, k)) ** (np.arange(k) % 7 == 0)
    elif kind == "ties":  # sums near the middle of two fp16 values
        x = np.round(rs.standard_normal((m, k)) * 32) / 32 + 2.0 ** -11
    else:
        raise ValueError(kind)
    return x.astype(np.float16)


@pytest.mark.parametrize("k,m", [(1024, 1), (5120, 1), (6144, 2), (17408, 1), (2048, 5)])
@pytest.mark.parametrize("kind", ["normal", "wide", "tiny", "huge", "ties"])
def test_rotate_bits(k, m, kind):
    rs = np.random.default_rng([k, m, len(kind)])
    x = activations(kind, rs, m, k)
    say("rotate %s K=%d M=%d" % (kind, k, m))
    assert_half_bits_equal(gpu_rotate(x), pnref.rotate(x), "rotate %s K=%d M=%d" % (kind, k, m))


def test_rotate_strided_and_in_place():
    rs = np.random.default_rng(3)
    x = activations("normal", rs, 3, 5120)
    want = pnref.rotate(x)
    say("rotate strided rows")
    assert_half_bits_equal(gpu_rotate(x, ldx=5122, ldo=6000), want, "strided")
    say("rotate in place")
    assert_half_bits_equal(gpu_rotate(x, ldx=5130, inplace=True), want, "in place")


def test_rotate_special_values():
    """Zeros of either sign give +0; inf and NaN inputs give what the exact
    definition gives (an inf where no opposite inf meets it, else NaN)."""
    x = np.zeros((4, 1024), np.float16)
    x[0] = -0.0
    x[1, 7] = np.inf
    x[2, 3] = np.inf
    x[2, 900] = -np.inf
    x[3, 11] = np.nan
    x[3, 12] = 1.0
    say("rotate special values")
    got = gpu_rotate(x)
    assert_half_bits_equal(got, pnref.rotate(x), "special")
    assert not np.signbit(got[0]).any()


def _problems(rs):
    """(type, N, K, rotated): rotated inputs need K a multiple of 1024."""
    return [("pn3t", 48, 5120, True), ("pn4t", 40, 6144, True), ("pn3t", 16, 1280, False),
            ("pn4t", 24, 17408, True), ("pn4t", 33, 5120, False), ("pn3t", 20, 2048 * 5, True)]


@pytest.mark.parametrize("kernel", ["auto", "stream", "rows"])
def test_rotated_group(kernel):
    """A plan mixing rotated and plain inputs: y = W (H x) for the flagged
    ones, y = W x for the others; x itself is left as it was, and a second
    run gives the same bits."""
    rs = np.random.default_rng(17)
    specs = _problems(rs)
    host, probs, flags = [], [], []
    for i, (t, n, k, rot) in enumerate(specs):
        g = np.random.default_rng([17, i])
        w = synth.random_blocks(g, t, n, k, unused_bits=True)
        x = synth.activation(g, k)
        y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        xd = dev(x)
        host.append((t, w, n, k, x, rot))
        probs.append((t, dev(w.reshape(-1)), n, k, xd, y))
        flags.append(rot)
    B.pn_set_gemv_kernel(kernel)
    try:
        say("rotated group (%s)" % kernel)
        plan = B.Group(probs, rotate=flags)
        plan.run()
        sync()
        first = [p[5].cpu().numpy() for p in probs]
        for p in probs:
            p[5].fill_(float("nan"))
        plan.run()
        sync()
        plan.close()
    finally:
        B.pn_set_gemv_kernel("auto")
    for (t, w, n, k, x, rot), p, y0 in zip(host, probs, first):
        assert np.array_equal(p[4].cpu().numpy().view(np.uint16), x.view(np.uint16)), "x changed"
        y = p[5].cpu().numpy()
        assert np.array_equal(y.view(np.uint32), y0.view(np.uint32)), "second run differs"
        xe = pnref.rotate(x) if rot else x
        y64, a = pnref.gemv_f64(t, w, n, k, xe)
        assert_gemv_close(y, y64, a, "rotated group %s %dx%d rot=%s" % (t, n, k, rot))
