"""Parity of the prefill GEMM (pn_gemm_prefill: any number of activation
rows, weights decoded inside an MFMA GEMM) against the CPU oracle's fp64
product, within 1e-5 * sum|w x| for every (row of X, weight row)."""
import numpy as np
import pytest

from gpu_util import assert_bits_equal, assert_gemv_close, dev, say, sync

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from bit_quantized_decode_pn3t_amd import _binding as B  # noqa: E402
from bit_quantized_decode_pn3t_amd import synth  # noqa: E402
from golden_io import load_blocks  # noqa: E402
from oracle import pnref  # noqa: E402

WPB = {"pn3t": 80, "pn4t": 64}


def gpu_prefill(t, w, n, k, xm, ldx=None, ldy=None):
    m = xm.shape[0]
    ldx = ldx or k
    ldy = ldy or n
    wd = dev(np.ascontiguousarray(w).reshape(-1))
    xb = torch.zeros(m * ldx, dtype=torch.float16, device="cuda")
    xb.view(m, ldx)[:, :k] = dev(xm)
    y = torch.full((m * ldy,), float("nan"), dtype=torch.float32, device="cuda")
    B.pn_gemm_prefill(t, wd, n, k, xb, ldx, m, y, ldy)
    sync()
    assert B.pn_variant_name(B.pn_last_variant()) == "gemm_prefill"
    yh = y.view(m, ldy).cpu().numpy()
    assert np.all(np.isnan(yh[:, n:])), "wrote past N"
    return yh[:, :n]


# (type, N, K, M): tiles of 128 x 128, ragged in both; K from one block pair per
# period to the down projection's 17408, with rows of two and three block
# pairs (the weights run two pairs ahead of the pair computed: pieces of one,
# two and three pairs take different paths through the pipeline)
SHAPES = [("pn3t", 256, 5120, 1), ("pn3t", 256, 5120, 17), ("pn3t", 256, 5120, 300), ("pn4t", 320, 6144, 129),
          ("pn4t", 130, 17408, 64), ("pn3t", 1000, 640, 257), ("pn4t", 96, 128, 200), ("pn3t", 33, 160, 5),
          ("pn4t", 300, 256, 140), ("pn3t", 270, 480, 33)]


@pytest.mark.parametrize("t,n,k,m", SHAPES)
def test_prefill_matches_oracle(t, n, k, m):
    g = np.random.default_rng([n, k, m])
    w = synth.random_blocks(g, t, n, k, unused_bits=True)
    xm = synth.activation(g, k, m)
    say("prefill %s N=%d K=%d M=%d" % (t, n, k, m))
    y = gpu_prefill(t, w, n, k, xm)
    y64, a = pnref.gemm_f64(t, w, n, k, xm)
    assert_gemv_close(y, y64, a, "prefill %s %dx%d M=%d" % (t, n, k, m))


def test_prefill_leading_dimensions():
    g = np.random.default_rng(5)
    t, n, k, m = "pn4t", 200, 1024, 150
    w = synth.random_blocks(g, t, n, k, unused_bits=True)
    xm = synth.activation(g, k, m)
    say("prefill ldx/ldy")
    y = gpu_prefill(t, w, n, k, xm, ldx=1048, ldy=203)
    y64, a = pnref.gemm_f64(t, w, n, k, xm)
    assert_gemv_close(y, y64, a, "prefill ld")


@pytest.mark.parametrize("t", ["pn3t", "pn4t"])
def test_prefill_zero_codes_and_outliers(t):
    """All codes at z give exact zeros whatever X is; fp16 activations up to
    +-65504 stay within the bound (no fp16 accumulation anywhere)."""
    blk = load_blocks()["G2" if t == "pn3t" else "G6"][1]
    nblk = 64
    k = WPB[t] * nblk
    w = np.tile(blk, nblk * 40).reshape(40, -1)
    g = np.random.default_rng(9)
    xm = synth.activation(g, k, 70)
    xm[:, ::97] = np.float16(65504.0)
    xm[3, 5::89] = np.float16(-65504.0)
    say("prefill zero codes %s" % t)
    assert np.all(gpu_prefill(t, w, 40, k, xm) == 0)
    w2 = synth.random_blocks(g, t, 140, k, unused_bits=True)
    say("prefill outliers %s" % t)
    y64, a = pnref.gemm_f64(t, w2, 140, k, xm)
    assert_gemv_close(gpu_prefill(t, w2, 140, k, xm), y64, a, "prefill outliers")


@pytest.mark.parametrize("t", ["pn3t", "pn4t"])
def test_prefill_subnormal_activations(t):
    """fp16-subnormal activations: row 0 of X is 2^-24 e_k (exact: the decoded
    column times 2^-24), row 1 all subnormal, row 2 mixed, the rest N(0, 1).
    A kernel that flushed subnormal inputs to zero would return zeros."""
    g = np.random.default_rng(44)
    n, k, m = 300, WPB[t] * 64, 130
    w = synth.random_blocks(g, t, n, k, unused_bits=True)
    xm = synth.activation(g, k, m)
    kk = 17 * WPB[t] + 5
    xm[0] = 0
    xm[0, kk] = np.uint16(1).view(np.float16)
    for r, mix in ((1, False), (2, True)):
        bits = g.integers(1, 1024, size=k).astype(np.uint16) | (g.integers(0, 2, size=k).astype(np.uint16) << 15)
        xm[r] = bits.view(np.float16)
        if mix:
            xm[r, ::3] = synth.activation(g, k)[::3]
    say("prefill subnormal activations %s" % t)
    y = gpu_prefill(t, w, n, k, xm)
    dense = pnref.dequantize(t, w, n, k).astype(np.float64)
    want = (dense[:, kk] * 2.0 ** -24).astype(np.float32)
    assert np.array_equal((y[0] + 0.0).view(np.uint32), (want + 0.0).view(np.uint32)), "one-hot 2^-24"
    y64, a = pnref.gemm_f64(t, w, n, k, xm)
    assert np.all(a[1:3] > 0)
    assert_gemv_close(y, y64, a, "prefill subnormal activations")


def test_prefill_layer_full_size():
    """Every product of one 27B-shaped layer (q, k, v, o, gate, up, down) with
    a 512-token prompt chunk, as the benchmark runs it (on 256 CUs: gate and
    up 272 tiles, one round dealt whole and 16 tiles' block pairs shared; q
    96 tiles, o and down 80, k and v 16, all shared): every output against
    the oracle."""
    m = 512
    g = np.random.default_rng(21)
    for name, t, n, k in synth.SWEEP_LAYER:
        w = synth.random_blocks(g, t, n, k, unused_bits=True)
        xm = synth.activation(g, k, m)
        say("prefill full size %s %s %dx%d M=%d" % (name, t, n, k, m))
        y = gpu_prefill(t, w, n, k, xm)
        y64, a = pnref.gemm_f64(t, w, n, k, xm)
        assert_gemv_close(y, y64, a, "prefill full size %s" % name)


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("case", ["one_over", "two_rounds_and_three", "two_m_tiles", "below"])
def test_prefill_dealing(case):
    """The tiles of whole rounds dealt whole and the rest's block pairs
    shared (by two workgroups here: 8 or 10 pairs a tile, at least 4 a
    piece): launches with one tile more than a round, two rounds and three
    tiles, tiles over two M tiles, and fewer tiles than CUs; ragged last
    tiles in N and M.  Every output against the oracle; the rows of tiles
    dealt whole come out the same on a second run."""
    G = cus()
    t, n, k, m = {"one_over": ("pn3t", (G + 1) * 256 - 100, 1280, 1),
                  "two_rounds_and_three": ("pn4t", (2 * G + 3) * 256, 1280, 1),
                  "two_m_tiles": ("pn3t", (G // 2 + 1) * 256 - 7, 1280, 200),
                  "below": ("pn4t", (G // 8) * 256 + 33, 1280, 130)}[case]
    g = np.random.default_rng([77, n, k, m])
    w = synth.random_blocks(g, t, n, k, unused_bits=True)
    xm = synth.activation(g, k, m)
    say("prefill dealing %s: %s N=%d K=%d M=%d on %d CUs" % (case, t, n, k, m, G))
    y = gpu_prefill(t, w, n, k, xm)
    y64, a = pnref.gemm_f64(t, w, n, k, xm)
    assert_gemv_close(y, y64, a, "prefill dealing %s" % case)
    tiles = ((n + 255) // 256) * ((m + 127) // 128)
    whole = tiles // G * G
    if whole:  # tiles [0, whole) in (M tile, N tile) order, N fastest
        tn = (n + 255) // 256
        y2 = gpu_prefill(t, w, n, k, xm)
        for tile in range(whole):
            r0, c0 = (tile // tn) * 128, (tile % tn) * 256
            assert_bits_equal(y2[r0:r0 + 128, c0:c0 + 256], y[r0:r0 + 128, c0:c0 + 256], "tile %d dealt whole" % tile)


def gpu_prefill_group(specs):
    """Run (type, w, N, K, xm, ldx, ldy) products as one pn_gemm_prefill_group
    launch; each product's outputs, checked for writes past N."""
    probs, outs = [], []
    for t, w, n, k, xm, ldx, ldy in specs:
        m = xm.shape[0]
        wd = dev(np.ascontiguousarray(w).reshape(-1))
        xb = torch.zeros(m * ldx, dtype=torch.float16, device="cuda")
        xb.view(m, ldx)[:, :k] = dev(xm)
        y = torch.full((m * ldy,), float("nan"), dtype=torch.float32, device="cuda")
        probs.append((t, wd, n, k, xb, ldx, m, y, ldy))
        outs.append((y, m, n, ldy))
    B.pn_gemm_prefill_group(probs)
    sync()
    assert B.pn_variant_name(B.pn_last_variant()) == "gemm_prefill_group"
    res = []
    for y, m, n, ldy in outs:
        yh = y.view(m, ldy).cpu().numpy()
        assert np.all(np.isnan(yh[:, n:])), "wrote past N"
        res.append(yh[:, :n])
    return res


def check_group(specs, what):
    for (t, w, n, k, xm, _, _), y in zip(specs, gpu_prefill_group(specs)):
        y64, a = pnref.gemm_f64(t, w, n, k, xm)
        assert_gemv_close(y, y64, a, "%s: %s %dx%d M=%d" % (what, t, n, k, xm.shape[0]))


def group_specs(shapes, seed):
    g = np.random.default_rng(seed)
    specs = []
    for t, n, k, m, ldx, ldy in shapes:
        specs.append((t, synth.random_blocks(g, t, n, k, unused_bits=True), n, k, synth.activation(g, k, m),
                      ldx or k, ldy or n))
    return specs


def test_prefill_group_mixed():
    """One launch over products of both types, ragged N and M, different M
    and K per product and padded leading dimensions: each against the
    oracle."""
    shapes = [("pn3t", 300, 640, 129, None, None), ("pn4t", 97, 1024, 129, 1032, 101),
              ("pn4t", 260, 384, 40, None, None), ("pn3t", 33, 160, 5, 168, 40), ("pn3t", 513, 1280, 256, None, None)]
    say("prefill group mixed: %d products" % len(shapes))
    check_group(group_specs(shapes, 31), "prefill group mixed")


@pytest.mark.parametrize("case", ["shared_across_products", "rounds_then_shared", "all_shared_mixed_pairs"])
def test_prefill_group_dealing(case):
    """The launch's tiles numbered product after product: whole rounds, then
    the leftover tiles' block pairs shared where those tiles belong to
    different products; and a launch below one round mixing pn3t (8 pairs
    a tile) with pn4t (10 pairs), where the fewer pairs set the ways."""
    G = cus()
    shapes = {"shared_across_products": [("pn3t", (G - 2) * 256, 1280, 1, None, None),
                                         ("pn4t", 3 * 256 - 50, 1280, 1, None, None),
                                         ("pn3t", 256 + 9, 1280, 1, None, None)],
              "rounds_then_shared": [("pn4t", G * 256, 1280, 1, None, None), ("pn3t", 300, 1280, 129, None, None)],
              "all_shared_mixed_pairs": [("pn3t", (G // 8) * 256 - 5, 1280, 130, None, None),
                                         ("pn4t", 256 + 3, 1280, 7, None, None)]}[case]
    say("prefill group dealing %s on %d CUs" % (case, G))
    check_group(group_specs(shapes, [41, G, len(case)]), "prefill group dealing %s" % case)


def test_prefill_group_layer_full_size():
    """A 27B-shaped layer's products in the groups a decoder can launch
    together ({q, k, v} and {gate, up}; {o} and {down} alone), 512-token
    chunk, as the benchmark runs them: every output against the oracle."""
    m = 512
    g = np.random.default_rng(23)
    layer = synth.SWEEP_LAYER
    for group in ((0, 1, 2), (4, 5)):
        specs = []
        for i in group:
            name, t, n, k = layer[i]
            specs.append((t, synth.random_blocks(g, t, n, k, unused_bits=True), n, k, synth.activation(g, k, m), k, n))
        say("prefill group full size %s M=%d" % ("+".join(layer[i][0] for i in group), m))
        check_group(specs, "prefill group full size")


def test_prefill_group_refuses_whole():
    """A group with one bad entry is refused before anything runs: the good
    entries' outputs stay untouched."""
    g = np.random.default_rng(51)
    t, n, k, m = "pn3t", 300, 640, 40
    w = dev(synth.random_blocks(g, t, n, k).reshape(-1))
    x = dev(synth.activation(g, k, m))
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    ybad = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    good = (t, w, n, k, x, k, m, y, n)
    bad = (t, w, n, 81, x, k, m, ybad, n)  # K not a whole number of blocks
    say("prefill group refused")
    assert B.pn_gemm_prefill_group([good, bad], check=False) == -2
    sync()
    assert torch.isnan(y).all() and torch.isnan(ybad).all()
    B.pn_gemm_prefill_group([good])
    sync()
    assert not torch.isnan(y).any()


def test_prefill_group_eight():
    """The largest group (PN_PREFILL_GROUP_MAX products), small shapes of
    both types: every tile finds its product among all eight records."""
    assert B.PREFILL_GROUP_MAX == 8
    shapes = [("pn3t" if i % 2 else "pn4t", 40 + 67 * i, 640 if i % 2 else 512, 17 + 23 * i, None, None)
              for i in range(8)]
    say("prefill group of 8")
    check_group(group_specs(shapes, 61), "prefill group of 8")
