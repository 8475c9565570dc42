"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Decoded weights must match bit for bit (NaN equal to NaN); GEMV outputs must
satisfy |y - y_ref| <= 1e-5 * sum_k |w x| row by row, y_ref the oracle's fp64
sum.  Every case prints what it runs before touching the GPU."""
import numpy as np
import pytest

from gpu_util import TOL, assert_bits_equal, assert_gemv_close, dev, say, sync
from golden_io import load_blocks

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from bit_quantized_decode_pn3t_amd import _binding as B  # noqa: E402
from bit_quantized_decode_pn3t_amd import synth  # noqa: E402
from oracle import pnref  # noqa: E402

WPB = {"pn3t": 80, "pn4t": 64}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield


def gpu_dequant(t, w, n, k, offset=0):
    """Dequantize on the GPU; `offset` shifts the weight base by that many bytes."""
    raw = np.ascontiguousarray(w).reshape(-1)
    buf = torch.zeros(raw.size + offset + 16, dtype=torch.uint8, device="cuda")
    buf[offset:offset + raw.size] = dev(raw)
    out = torch.empty((n, k), dtype=torch.float32, device="cuda")
    B.pn_dequantize(t, buf.data_ptr() + offset, n, k, out)
    sync()
    assert B.pn_variant_name(B.pn_last_variant()) == "dequant"
    return out.cpu().numpy()


def gpu_gemv(t, w, n, k, x, offset=0, expect_variant=None):
    raw = np.ascontiguousarray(w).reshape(-1)
    buf = torch.zeros(raw.size + offset + 16, dtype=torch.uint8, device="cuda")
    buf[offset:offset + raw.size] = dev(raw)
    xd = dev(np.asarray(x, np.float16))
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    B.pn_gemv(t, buf.data_ptr() + offset, n, k, xd, y)
    sync()
    if expect_variant:
        assert B.pn_variant_name(B.pn_last_variant()) == expect_variant
    return y.cpu().numpy()


def random_matrix(seed, t, n, k, unused_bits=True):
    """Random packed rows; pn3t words carry junk in their unused bits 15 and
    31 unless `unused_bits` is False (readers must ignore those bits)."""
    g = np.random.default_rng(seed)
    return synth.random_blocks(g, t, n, k, unused_bits=unused_bits), g


# ---------------------------------------------------------------------------
# decode, bit-exact
# ---------------------------------------------------------------------------
def test_dequant_goldens():
    for gid, (t, blk, expect) in load_blocks().items():
        for off in (0, 2):
            say("dequant golden %s offset %d" % (gid, off))
            got = gpu_dequant(t, blk, 1, WPB[t], off)
            assert_bits_equal(got, expect.view(np.float32), gid)


@pytest.mark.parametrize("t", ["pn3t", "pn4t"])
@pytest.mark.parametrize("offset", [0, 2, 6])
def test_dequant_random_blocks(t, offset):
    """200k blocks of random bytes: every scale pattern (subnormal, +-0,
    +-inf, NaN) and, for pn3t, junk in the unused bits."""
    say("dequant random %s offset %d" % (t, offset))
    rs = np.random.default_rng(5 + offset)
    nb = 8
    n = 25000
    raw = rs.integers(0, 256, size=n * nb * 34, dtype=np.uint8)
    k = nb * WPB[t]
    got = gpu_dequant(t, raw, n, k, offset)
    want = pnref.dequantize(t, raw, n, k)
    assert_bits_equal(got, want, "random %s" % t)


@pytest.mark.parametrize("t,n,k", [("pn3t", 256, 5120), ("pn4t", 5120, 17408), ("pn4t", 1024, 5120),
                                   ("pn4t", 5120, 6144), ("pn3t", 37, 80 * 3), ("pn4t", 5, 64)])
def test_dequant_shapes(t, n, k):
    say("dequant %s %dx%d" % (t, n, k))
    w, _ = random_matrix(101, t, n, k)
    assert_bits_equal(gpu_dequant(t, w, n, k), pnref.dequantize(t, w, n, k), "%s %dx%d" % (t, n, k))


# ---------------------------------------------------------------------------
# M = 1, on every kernel choice: "auto" (the library's own pick), "stream"
# (register pipeline) and "rows" (row tiles wherever they apply)
# ---------------------------------------------------------------------------
KERNELS = ["auto", "stream", "rows"]


@pytest.fixture
def gemv_kernel(request):
    B.pn_set_gemv_kernel(request.param)
    yield request.param
    B.pn_set_gemv_kernel("auto")


def rows_min_tiles():
    return torch.cuda.get_device_properties(0).multi_processor_count * 32


def rows_ok(t, k, offset=0):
    nb = k // WPB[t]
    return offset % 16 == 0 and nb % 8 == 0 and nb * 34 <= 1 << 24


def m1_variant(kernel, t, k, offset=0, tiles=0):
    """The kernel pn_gemv should report for this shape (the library's rules,
    restated from include/pn.h); `tiles` = 16-row tiles of the launch."""
    if kernel != "stream" and rows_ok(t, k, offset) and (kernel == "rows" or tiles >= rows_min_tiles()):
        return "gemv_rows"
    nw = k // WPB[t] * 8
    if nw % 64 == 0 and nw * (20 if t == "pn3t" else 16) <= 65536:
        return "gemv_stream"
    return "gemv_generic"


def tiles_of(*ns):
    return sum((n + 15) // 16 for n in ns)


@pytest.mark.parametrize("gemv_kernel", KERNELS, indirect=True)
def test_gemv_config0(gemv_kernel):
    c = synth.config0()
    say("gemv config 0 pn3t 256x5120 (%s)" % gemv_kernel)
    y = gpu_gemv(c["type"], c["W"], c["N"], c["K"], c["x"], expect_variant=m1_variant(gemv_kernel, "pn3t", 5120, 0, tiles_of(256)))
    y64, a = pnref.gemv_f64(c["type"], c["W"], c["N"], c["K"], c["x"])
    assert_gemv_close(y, y64, a, "config 0")


@pytest.mark.parametrize("gemv_kernel", KERNELS, indirect=True)
def test_gemv_config1(gemv_kernel):
    c = synth.config1()
    say("gemv config 1 pn4t 5120x17408 (%s)" % gemv_kernel)
    y = gpu_gemv(c["type"], c["W"], c["N"], c["K"], c["x"], expect_variant=m1_variant(gemv_kernel, "pn4t", 17408, 0, tiles_of(5120)))
    y64, a = pnref.gemv_f64(c["type"], c["W"], c["N"], c["K"], c["x"])
    assert_gemv_close(y, y64, a, "config 1")


@pytest.mark.parametrize("gemv_kernel", KERNELS, indirect=True)
def test_gemv2_config2(gemv_kernel):
    """Fused gate+up: weights N(0, 0.02) quantized by the oracle's quantizer."""
    say("gemv2 config 2: quantize 2 x 17408x5120 on the CPU (%s)" % gemv_kernel)
    wg, wu, x = synth.config2_weights()
    qg = pnref.quantize("pn3t", wg, 17408, 5120)
    qu = pnref.quantize("pn3t", wu, 17408, 5120)
    say("gemv2 config 2 on the GPU")
    W0, W1, xd = dev(qg), dev(qu), dev(x)
    y0 = torch.empty(17408, dtype=torch.float32, device="cuda")
    y1 = torch.empty(17408, dtype=torch.float32, device="cuda")
    B.pn_gemv2("pn3t", W0, W1, 17408, 5120, xd, y0, y1)
    sync()
    assert B.pn_variant_name(B.pn_last_variant()) == m1_variant(gemv_kernel, "pn3t", 5120, 0, tiles_of(17408, 17408))
    for q, y, name in ((qg, y0, "gate"), (qu, y1, "up")):
        y64, a = pnref.gemv_f64("pn3t", q, 17408, 5120, x)
        assert_gemv_close(y.cpu().numpy(), y64, a, "config 2 " + name)
    # decoded weights of the quantized matrices are bit-exact too (first and last rows)
    for q in (qg, qu):
        rows = np.ascontiguousarray(q[[0, 17407]])
        assert_bits_equal(gpu_dequant("pn3t", rows, 2, 5120), pnref.dequantize("pn3t", rows, 2, 5120))


EDGE_SHAPES = [
    # (type, N, K, W byte offset)
    ("pn3t", 1, 640, 0),          # one pass per row
    ("pn3t", 13, 1280, 0),        # N not a multiple of the tile
    ("pn3t", 257, 5120, 2),       # 2-aligned base
    ("pn4t", 3, 512, 0),
    ("pn4t", 1023, 6144, 2),
    ("pn4t", 200000, 512, 0),     # many rows per wave
    ("pn4t", 64, 17408, 6),
    ("pn3t", 5, 80, 0),           # one block per row
    ("pn3t", 9, 240, 2),          # ragged: 3 blocks
    ("pn4t", 7, 576, 0),          # ragged: 9 blocks
    ("pn4t", 33, 64 * 600, 0),    # activation larger than LDS
    ("pn3t", 4, 80 * 500, 2),
    # shapes of the row-tile kernel: P = periods (8 blocks) per row, 4 per window
    ("pn3t", 1, 5120, 0),         # one row: a tile of 1 valid row
    ("pn3t", 17, 80 * 24, 0),     # P = 3: one window, three of four lane rows
    ("pn4t", 33, 64 * 40, 0),     # P = 5: the second window has one period
    ("pn4t", 16, 5120, 0),        # P = 10: one whole tile, last window half used
    ("pn4t", 31, 64 * 8 * 7, 0),  # P = 7, a ragged second tile
    ("pn3t", 2000, 80 * 128, 0),  # P = 16: four whole windows
    ("pn3t", 100, 5120, 16),      # 16-aligned, not 256-aligned base
    ("pn3t", 100, 5120, 4),       # 4-aligned base: not for row tiles
    ("pn4t", 1000, 17408, 0),     # P = 34: nine windows
    ("pn3t", 3, 80 * 800, 0),     # P = 100: x of 128 KB (register kernel: generic)
    ("pn3t", 200000, 5120, 0),    # 435 MB: many tiles per wave
    ("pn4t", 4099, 6144, 0),      # P = 12, 257 tiles
]


@pytest.mark.parametrize("gemv_kernel", KERNELS, indirect=True)
@pytest.mark.parametrize("t,n,k,offset", EDGE_SHAPES)
def test_gemv_edge_shapes(gemv_kernel, t, n, k, offset):
    say("gemv edge %s N=%d K=%d offset=%d (%s)" % (t, n, k, offset, gemv_kernel))
    w, g = random_matrix(n * 7 + k, t, n, k, unused_bits=True)
    x = synth.activation(g, k)
    y = gpu_gemv(t, w, n, k, x, offset, expect_variant=m1_variant(gemv_kernel, t, k, offset, tiles_of(n)))
    y64, a = pnref.gemv_f64(t, w, n, k, x)
    assert_gemv_close(y, y64, a, "%s %dx%d" % (t, n, k))


@pytest.mark.parametrize("gemv_kernel", KERNELS, indirect=True)
@pytest.mark.parametrize("t", ["pn3t", "pn4t"])
def test_gemv_one_hot_is_exact(gemv_kernel, t):
    """x = e_k gives the decoded column exactly, on every kernel."""
    wpb = WPB[t]
    cases = [(40, wpb * 8, (0, 1, wpb * 4 + 1, wpb * 8 - 1)), (6, wpb * 3, (0, 1, wpb + 1, wpb * 3 - 1)),
             (9, wpb * 66, tuple(range(0, 2 * wpb)) + (wpb * 33, wpb * 33 + 1, wpb * 66 - 1))]
    for n, k, kks in cases:
        w, g = random_matrix(3 + n, t, n, k)
        dense = pnref.dequantize(t, w, n, k)
        say("gemv one-hot %s %dx%d, %d columns (%s)" % (t, n, k, len(kks), gemv_kernel))
        for kk in kks:
            x = np.zeros(k, np.float16)
            x[kk] = 1.0
            got = gpu_gemv(t, w, n, k, x, expect_variant=m1_variant(gemv_kernel, t, k, 0, tiles_of(n)))
            assert_bits_equal(got + 0.0, dense[:, kk] + 0.0, "one-hot k=%d" % kk)


@pytest.mark.parametrize("t", ["pn3t", "pn4t"])
def test_rows_one_hot_every_column(t):
    """Row tiles, every column of a four-period window (both blocks of each
    block pair, each lane's broadcast activation pairs) and of a partial
    window: x = e_k gives the decoded column exactly."""
    wpb = WPB[t]
    n, k = 21, wpb * 8 * 5  # two tiles (the second ragged), windows of 4 and 1 periods
    w, g = random_matrix(17, t, n, k)
    dense = pnref.dequantize(t, w, n, k)
    B.pn_set_gemv_kernel("rows")
    try:
        say("rows one-hot %s %dx%d, all %d columns" % (t, n, k, k))
        raw = dev(np.ascontiguousarray(w).reshape(-1))
        y = torch.empty(n, dtype=torch.float32, device="cuda")
        x = torch.zeros(k, dtype=torch.float16, device="cuda")
        got = np.empty((k, n), np.float32)
        for kk in range(k):
            x.zero_()
            x[kk] = 1.0
            B.pn_gemv(t, raw, n, k, x, y)
            got[kk] = y.cpu().numpy()
        assert B.pn_variant_name(B.pn_last_variant()) == "gemv_rows"
        assert_bits_equal(got.T + 0.0, dense + 0.0, "one-hot every column")
    finally:
        B.pn_set_gemv_kernel("auto")


@pytest.mark.parametrize("gemv_kernel", KERNELS, indirect=True)
@pytest.mark.parametrize("t", ["pn3t", "pn4t"])
def test_gemv_zero_codes(gemv_kernel, t):
    """All codes at z: every output is +-0 whatever x is."""
    blk = load_blocks()["G2" if t == "pn3t" else "G6"][1]
    for nblk in (16, 64):
        k = WPB[t] * nblk
        w = np.tile(blk, nblk * 9).reshape(9, -1)
        x = np.random.default_rng(4).standard_normal(k).astype(np.float16)
        say("gemv zero codes %s K=%d (%s)" % (t, k, gemv_kernel))
        y = gpu_gemv(t, w, 9, k, x, expect_variant=m1_variant(gemv_kernel, t, k, 0, 1))
        assert np.all(y == 0)


@pytest.mark.parametrize("gemv_kernel", KERNELS, indirect=True)
@pytest.mark.parametrize("t", ["pn3t", "pn4t"])
def test_gemv_outlier_activations(gemv_kernel, t):
    """fp16 activations up to +-65504 (no fp16 accumulation anywhere)."""
    for nblk in (16, 64):
        n, k = 64, WPB[t] * nblk
        w, g = random_matrix(77, t, n, k)
        x = synth.activation(g, k)
        x[::97] = np.float16(65504.0)
        x[5::89] = np.float16(-65504.0)
        say("gemv outliers %s K=%d (%s)" % (t, k, gemv_kernel))
        y = gpu_gemv(t, w, n, k, x, expect_variant=m1_variant(gemv_kernel, t, k, 0, tiles_of(n)))
        y64, a = pnref.gemv_f64(t, w, n, k, x)
        assert_gemv_close(y, y64, a, "outliers")


def subnormal_activations(g, k, mix=False):
    """fp16 activations that are all subnormal (|x| < 2^-14: a random nonzero
    10-bit fraction, random sign), or with `mix` every third one normal."""
    bits = g.integers(1, 1024, size=k).astype(np.uint16) | (g.integers(0, 2, size=k).astype(np.uint16) << 15)
    x = bits.view(np.float16).copy()
    if mix:
        x[::3] = synth.activation(g, k)[::3]
    return x


@pytest.mark.parametrize("gemv_kernel", KERNELS, indirect=True)
@pytest.mark.parametrize("t", ["pn3t", "pn4t"])
def test_gemv_subnormal_activations(gemv_kernel, t):
    """fp16-subnormal activations are values like any other: x = 2^-24 e_k
    (the smallest subnormal) gives w[:, k] * 2^-24 exactly, and all-subnormal
    or mixed activations stay within the bound.  A kernel that flushed
    subnormal inputs to zero would return zeros here."""
    wpb = WPB[t]
    n, k = 40, wpb * 8 * 5  # two tiles (the second ragged); windows of 4 and 1 periods
    w, g = random_matrix(31, t, n, k)
    dense = pnref.dequantize(t, w, n, k).astype(np.float64)
    variant = m1_variant(gemv_kernel, t, k, 0, tiles_of(n))
    say("gemv subnormal activations %s (%s)" % (t, gemv_kernel))
    for kk in (0, 1, wpb - 1, wpb + 2, 4 * wpb + 7, k - 1):
        x = np.zeros(k, np.float16)
        x[kk] = np.uint16(1).view(np.float16)  # 2^-24
        y = gpu_gemv(t, w, n, k, x, expect_variant=variant)
        want = (dense[:, kk] * 2.0 ** -24).astype(np.float32)  # exact: at most 14 significant bits
        assert_bits_equal(y + 0.0, want + 0.0, "one-hot 2^-24 at k=%d" % kk)
    for mix in (False, True):
        x = subnormal_activations(g, k, mix)
        y = gpu_gemv(t, w, n, k, x, expect_variant=variant)
        y64, a = pnref.gemv_f64(t, w, n, k, x)
        assert np.all(a > 0)
        assert_gemv_close(y, y64, a, "subnormal activations (mixed=%s)" % mix)


@pytest.mark.parametrize("gemv_kernel", KERNELS, indirect=True)
def test_gemv_deterministic(gemv_kernel):
    c = synth.config0()
    say("gemv determinism (%s)" % gemv_kernel)
    ys = [gpu_gemv(c["type"], c["W"], c["N"], c["K"], c["x"]) for _ in range(5)]
    for y in ys[1:]:
        assert_bits_equal(y, ys[0], "repeat")


GROUP_SPECS = {
    # mixed: includes a row of one 8-block pass, so "auto" keeps the register kernel
    "mixed": [("pn3t", 100, 5120), ("pn4t", 37, 5120), ("pn4t", 300, 6144), ("pn3t", 1, 640),
              ("pn4t", 65, 17408), ("pn3t", 2000, 1280)],
    # every problem fits the row-tile kernel (periods per row 8, 10, 12, 1, 34, 3, 7)
    "rows": [("pn3t", 100, 5120), ("pn4t", 37, 5120), ("pn4t", 300, 6144), ("pn3t", 1, 640),
             ("pn4t", 65, 17408), ("pn3t", 2000, 80 * 24), ("pn4t", 3, 64 * 56)],
}


@pytest.mark.parametrize("gemv_kernel", KERNELS, indirect=True)
@pytest.mark.parametrize("which", ["mixed", "rows"])
def test_group(gemv_kernel, which):
    """One grouped launch over problems of both types and several shapes."""
    specs = GROUP_SPECS[which]
    host, probs = [], []
    for i, (t, n, k) in enumerate(specs):
        w, g = random_matrix(500 + i, t, n, k)
        x = synth.activation(g, k)
        wd, xd = dev(w), dev(x)
        y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        host.append((t, w, n, k, x, y))
        probs.append((t, wd, n, k, xd, y))
    say("group %s of %d problems (%s)" % (which, len(specs), gemv_kernel))
    tiles = tiles_of(*[n for _, n, _ in specs])
    rows = all(m1_variant(gemv_kernel, t, k, 0, tiles) == "gemv_rows" for t, _, k in specs)
    if not rows and not all(m1_variant("stream", t, k) == "gemv_stream" for t, _, k in specs):
        with pytest.raises(B.PNError) as e:  # the register kernel takes whole 8-block passes only
            B.Group(probs)
        assert e.value.status == -4
        return
    grp = B.Group(probs)
    grp.run()
    sync()
    assert B.pn_variant_name(B.pn_last_variant()) == ("gemv_rows_group" if rows else "gemv_stream_group")
    for t, w, n, k, x, y in host:
        y64, a = pnref.gemv_f64(t, w, n, k, x)
        assert_gemv_close(y.cpu().numpy(), y64, a, "group %s %dx%d" % (t, n, k))
    grp.close()


# ---------------------------------------------------------------------------
# small M (both arithmetic units over the same loads)
# ---------------------------------------------------------------------------
# The three small-M paths: MFMA arithmetic with the kernel choice left to the
# library (gemm_rows, weights staged through LDS by DMA, wherever the rows
# are whole 8-block periods; gemm_stream elsewhere), MFMA on gemm_stream
# forced, and the VALU arithmetic (gemm_stream).
MATHS = ["mfma", "mfma_stream", "valu"]
# (type, N, K): several 32-row (gemm_stream) and 16-row (gemm_rows) wave tiles
# with ragged tails; rows shorter than the 2U-block pipeline (1 and 7
# blocks), rows for the in-order U-slot pipeline (9 and 11 blocks: at least
# 2U, fewer than the grouped pipeline's 4U); rows of one period (8 blocks);
# and activations that take several LDS chunks at M = 8 (pn3t K = 5120: 2
# chunks for gemm_stream at M = 16, 2 for gemm_rows from M = 9; pn4t K = 17408:
# several for both).
SMALLM_SHAPES = [("pn3t", 256, 5120), ("pn4t", 300, 17408), ("pn4t", 33, 6144), ("pn3t", 7, 80),
                 ("pn4t", 19, 64 * 9), ("pn3t", 45, 80 * 7), ("pn3t", 40, 80 * 11), ("pn4t", 1000, 5120),
                 ("pn3t", 130, 640), ("pn4t", 17, 512), ("pn3t", 129, 640 * 3)]


def smallm_variant(path, t, k, group=False):
    """The kernel the library picks for a problem on this path."""
    rows = path == "mfma" and (k // WPB[t]) % 8 == 0
    name = "gemm_rows_mfma" if rows else "gemm_stream_" + ("valu" if path == "valu" else "mfma")
    return name + ("_group" if group else "")


@pytest.fixture
def smallm_math(request):
    B.pn_set_smallm_math("valu" if request.param == "valu" else "mfma")
    B.pn_set_gemv_kernel("stream" if request.param == "mfma_stream" else "auto")
    yield request.param
    B.pn_set_smallm_math("mfma")
    B.pn_set_gemv_kernel("auto")


def gpu_smallm(t, w, n, k, X, m, ldx, ldy):
    Y = torch.full((m, ldy), 7.0, dtype=torch.float32, device="cuda")
    B.pn_gemm_smallm(t, dev(w), n, k, dev(X), ldx, m, Y, ldy)
    sync()
    return Y.cpu().numpy()


@pytest.mark.parametrize("smallm_math", MATHS, indirect=True)
@pytest.mark.parametrize("t,n,k", SMALLM_SHAPES)
@pytest.mark.parametrize("m", [1, 2, 5, 8, 9, 16])
def test_gemm_smallm(smallm_math, t, n, k, m):
    w, g = random_matrix(n + k + m, t, n, k)
    ldx, ldy = k + 2 * (m % 2), n + 3
    X = np.zeros((m, ldx), np.float16)
    X[:, :k] = synth.activation(g, k, m)
    say("gemm_smallm %s %s %dx%d M=%d" % (smallm_math, t, n, k, m))
    Y = gpu_smallm(t, w, n, k, X, m, ldx, ldy)
    assert B.pn_variant_name(B.pn_last_variant()) == smallm_variant(smallm_math, t, k)
    assert np.all(Y[:, n:] == 7.0), "wrote past N in a row of Y"
    y64, a = pnref.gemm_f64(t, w, n, k, X[:, :k])
    assert_gemv_close(Y[:, :n], y64, a, "smallm %s %s M=%d" % (smallm_math, t, m))
    if m == 1:
        y1 = gpu_gemv(t, w, n, k, X[0, :k])
        # both within TOL of the fp64 sum, so within 2 * TOL of each other
        assert_gemv_close(Y[0, :n], y1.astype(np.float64), a[0], "smallm vs gemv", tol=2 * TOL)


@pytest.mark.parametrize("smallm_math", MATHS, indirect=True)
@pytest.mark.parametrize("t", ["pn3t", "pn4t"])
@pytest.mark.parametrize("nblk", [6, 16])
def test_smallm_one_hot_exact(smallm_math, t, nblk):
    """Row m of X is one-hot at k_m: Y[m, r] = w[r, k_m] exactly (one exact
    product, the rest zeros).  Pins the k <-> (block, word, slot) map of the
    operand layouts, including both words of a lane, the block edges and all
    16 batch rows; with 16 blocks (two periods) also both blocks of a pair in
    gemm_rows's stage (the first block's words lie off the dword grid)."""
    wpb = WPB[t]
    n, k = 70, wpb * nblk
    w, _ = random_matrix(17, t, n, k)
    ks = [0, 1, wpb // 4 - 1, wpb // 4, wpb // 2 + 3, wpb - 1, wpb, 5 * wpb + wpb - 2,
          2, wpb // 8, wpb // 4 + 7, wpb // 2 - 1, wpb // 2, 3 * wpb // 4, 2 * wpb + 9, 4 * wpb - 1]
    if nblk == 16:
        ks[8:] = [3 * wpb + 11, 7 * wpb + wpb - 1, 8 * wpb, 9 * wpb + 21, 11 * wpb + 40, 12 * wpb + 5,
                  14 * wpb + 63, 16 * wpb - 1]
    X = np.zeros((16, k), np.float16)
    for m, km in enumerate(ks):
        X[m, km] = 1.0
    say("smallm one-hot %s %s %d blocks" % (smallm_math, t, nblk))
    Y = gpu_smallm(t, w, n, k, X, 16, k, n)
    assert B.pn_variant_name(B.pn_last_variant()) == smallm_variant(smallm_math, t, k)
    dense = pnref.dequantize(t, w, n, k)
    for m, km in enumerate(ks):
        assert_bits_equal(Y[m] + 0.0, dense[:, km] + 0.0, "one-hot m=%d k=%d" % (m, km))


@pytest.mark.parametrize("smallm_math", MATHS, indirect=True)
@pytest.mark.parametrize("t", ["pn3t", "pn4t"])
@pytest.mark.parametrize("m", [8, 16])
def test_smallm_subnormal_activations(smallm_math, t, m):
    """Batch rows of fp16-subnormal activations: row 0 is 2^-24 e_k (exact:
    Y[0, :] = w[:, k] * 2^-24), row 1 all subnormal, row 2 mixed, the rest
    N(0, 1); 16 blocks (two periods) so that both small-M kernels run."""
    wpb = WPB[t]
    n, k = 70, wpb * 16
    w, g = random_matrix(41 + m, t, n, k)
    X = synth.activation(g, k, m)
    kk = 5 * wpb + 3
    X[0] = 0
    X[0, kk] = np.uint16(1).view(np.float16)
    X[1] = subnormal_activations(g, k)
    X[2] = subnormal_activations(g, k, mix=True)
    say("smallm subnormal activations %s %s M=%d" % (smallm_math, t, m))
    Y = gpu_smallm(t, w, n, k, X, m, k, n)
    assert B.pn_variant_name(B.pn_last_variant()) == smallm_variant(smallm_math, t, k)
    dense = pnref.dequantize(t, w, n, k).astype(np.float64)
    assert_bits_equal(Y[0] + 0.0, (dense[:, kk] * 2.0 ** -24).astype(np.float32) + 0.0, "one-hot 2^-24")
    y64, a = pnref.gemm_f64(t, w, n, k, X)
    assert np.all(a[1:3] > 0)
    assert_gemv_close(Y, y64, a, "smallm subnormal activations")


@pytest.mark.parametrize("smallm_math", MATHS, indirect=True)
def test_smallm_deterministic(smallm_math):
    t, n, k, m = "pn4t", 300, 17408, 8
    w, g = random_matrix(3, t, n, k)
    X = synth.activation(g, k, m)
    say("smallm determinism %s" % smallm_math)
    y1 = gpu_smallm(t, w, n, k, X, m, k, n)
    y2 = gpu_smallm(t, w, n, k, X, m, k, n)
    assert_bits_equal(y1, y2, "two runs")


@pytest.mark.parametrize("smallm_math", MATHS, indirect=True)
def test_smallm_group(smallm_math):
    """One launch over problems of mixed type, shape, M and leading
    dimensions; each against the oracle."""
    specs = [("pn3t", 100, 5120, 8), ("pn4t", 70, 17408, 3), ("pn4t", 300, 6144, 8),
             ("pn3t", 5, 80, 1), ("pn4t", 260, 5120, 16), ("pn3t", 33, 80 * 9, 6), ("pn3t", 64, 5120, 13)]
    host, probs, keep = [], [], []
    for i, (t, n, k, m) in enumerate(specs):
        w, g = random_matrix(1000 + i, t, n, k)
        ldx, ldy = k + 2 * (i % 2), n + 1
        X = np.zeros((m, ldx), np.float16)
        X[:, :k] = synth.activation(g, k, m)
        Y = torch.full((m, ldy), 7.0, dtype=torch.float32, device="cuda")
        wd, xd = dev(w), dev(X)
        keep += [wd, xd]
        probs.append((t, wd, n, k, xd, ldx, m, Y, ldy))
        host.append((t, w, n, k, X[:, :k], Y))
    say("smallm group %s: %d problems" % (smallm_math, len(specs)))
    grp = B.Group(probs, smallm=True)
    grp.run()
    sync()
    # one problem (K = 80, 720) is not whole periods: the plan runs on gemm_stream
    assert B.pn_variant_name(B.pn_last_variant()) == smallm_variant(smallm_math, "pn3t", 80, group=True)
    for t, w, n, k, X, Y in host:
        Yh = Y.cpu().numpy()
        assert np.all(Yh[:, n:] == 7.0)
        y64, a = pnref.gemm_f64(t, w, n, k, X)
        assert_gemv_close(Yh[:, :n], y64, a, "smallm group %s %dx%d M=%d" % (t, n, k, X.shape[0]))
    grp.close()


@pytest.mark.parametrize("t", ["pn3t", "pn4t"])
def test_smallm_unaligned_weights(t):
    """Rows of whole periods whose W is 2-byte but not 16-byte aligned: the
    DMA kernel needs 16-byte chunks, so the library runs gemm_stream."""
    n, k, m = 70, WPB[t] * 16, 8
    w, g = random_matrix(61, t, n, k)
    X = synth.activation(g, k, m)
    raw = dev(np.concatenate([np.zeros(2, np.uint8), np.ascontiguousarray(w).reshape(-1)]))
    wd = raw[2:]
    assert wd.data_ptr() % 16 == 2
    Y = torch.full((m, n), 7.0, dtype=torch.float32, device="cuda")
    say("smallm unaligned W %s" % t)
    B.pn_gemm_smallm(t, wd, n, k, dev(X), k, m, Y, n)
    sync()
    assert B.pn_variant_name(B.pn_last_variant()) == "gemm_stream_mfma"
    y64, a = pnref.gemm_f64(t, w, n, k, X)
    assert_gemv_close(Y.cpu().numpy(), y64, a, "smallm unaligned W")


@pytest.mark.parametrize("smallm_math", ["mfma", "mfma_stream"], indirect=True)
@pytest.mark.parametrize("t,n,k", [("pn3t", 17408, 5120), ("pn4t", 5120, 17408)])
def test_smallm_full_size_m16(smallm_math, t, n, k):
    """M = 16 (k = 15 drafts) on the gate and down projections at full size:
    the activations take several LDS chunks per tile on both kernels.  Every
    output against the oracle."""
    m = 16
    w, g = random_matrix(n + m, t, n, k)
    X = synth.activation(g, k, m)
    say("smallm full size M=16 %s %s %dx%d" % (smallm_math, t, n, k))
    Y = gpu_smallm(t, w, n, k, X, m, k, n)
    assert B.pn_variant_name(B.pn_last_variant()) == smallm_variant(smallm_math, t, k)
    y64, a = pnref.gemm_f64(t, w, n, k, X)
    assert_gemv_close(Y, y64, a, "smallm full size M=16")


@pytest.mark.parametrize("smallm_math", MATHS, indirect=True)
def test_smallm_group_periods(smallm_math):
    """A plan whose problems are all whole periods (gemm_rows runs it with the
    MFMA arithmetic): mixed types, M, leading dimensions, ragged N against the
    16-row waves and 128-row tiles, one- and many-chunk activations."""
    specs = [("pn3t", 6144 // 16 + 5, 5120, 8), ("pn4t", 1024 + 3, 5120, 16), ("pn4t", 200, 17408, 8),
             ("pn3t", 17, 640, 1), ("pn4t", 130, 6144, 5), ("pn3t", 2, 1280, 12)]
    host, probs, keep = [], [], []
    for i, (t, n, k, m) in enumerate(specs):
        w, g = random_matrix(2000 + i, t, n, k)
        ldx, ldy = k + 8 * (i % 2), n + 2 * (i % 3)
        X = np.zeros((m, ldx), np.float16)
        X[:, :k] = synth.activation(g, k, m)
        Y = torch.full((m, ldy), 7.0, dtype=torch.float32, device="cuda")
        wd, xd = dev(w), dev(X)
        keep += [wd, xd]
        probs.append((t, wd, n, k, xd, ldx, m, Y, ldy))
        host.append((t, w, n, k, X[:, :k], Y))
    say("smallm group of whole periods %s: %d problems" % (smallm_math, len(specs)))
    grp = B.Group(probs, smallm=True)
    grp.run()
    sync()
    assert B.pn_variant_name(B.pn_last_variant()) == smallm_variant(smallm_math, "pn3t", 640, group=True)
    for t, w, n, k, X, Y in host:
        Yh = Y.cpu().numpy()
        assert np.all(Yh[:, n:] == 7.0)
        y64, a = pnref.gemm_f64(t, w, n, k, X)
        assert_gemv_close(Yh[:, :n], y64, a, "smallm group %s %dx%d M=%d" % (t, n, k, X.shape[0]))
    grp.close()


@pytest.mark.parametrize("n", [64 << 20, 16711680])
def test_read_probe(n):
    """The streaming-read probe reads what it reports and folds it exactly:
    the XOR of all per-lane checksums equals the XOR of every word read
    (16,711,680 bytes: each wave's share ends inside a 16 KiB stage)."""
    say("read probe %d bytes" % n)
    rs = np.random.default_rng(9)
    host = rs.integers(0, 2 ** 32, size=n // 4, dtype=np.uint32)
    buf = dev(host.view(np.uint8))
    scratch = torch.zeros(B.pn_read_probe_scratch_bytes() // 4, dtype=torch.int32, device="cuda")
    got = B.pn_read_probe(buf, n, scratch, scratch.numel() * 4)
    sync()
    assert 0 < got <= n and got % 1024 == 0
    want = np.bitwise_xor.reduce(host[: got // 4])
    assert np.bitwise_xor.reduce(scratch.cpu().numpy().view(np.uint32)) == want
