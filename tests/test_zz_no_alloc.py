"""pn_gemv_batch, the allocation-free form of pn_group_create + pn_group_run
(its plan lives in the library's static per-device batch buffer): through
the C ABI, its outputs equal those of a plan over the same descriptors, bit
for bit, and are within 1e-5 * sum|w x| of the oracle, on two calls in a row
(the second smaller), on both kernels, and up to the buffer's row limit."""
import numpy as np
import pytest

from gpu_util import assert_bits_equal, assert_gemv_close, dev, say, sync

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from bit_quantized_decode_pn3t_amd import _binding as B  # noqa: E402
from bit_quantized_decode_pn3t_amd import synth  # noqa: E402
from oracle import pnref  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield


def make_problems(specs, seed):
    host, probs = [], []
    for i, (t, n, k) in enumerate(specs):
        g = np.random.default_rng([seed, i])
        w = synth.random_blocks(g, t, n, k, unused_bits=True)
        x = synth.activation(g, k)
        y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        host.append((t, w, n, k, x))
        probs.append((t, dev(w), n, k, dev(x), y))
    return host, probs


def run_both(probs, variant):
    """The batch call, then a plan over the same problems into fresh outputs:
    returns both outputs per problem."""
    for p in probs:
        p[5].fill_(float("nan"))
    B.pn_gemv_batch(probs)
    sync()
    assert B.pn_variant_name(B.pn_last_variant()) == variant
    got = [p[5].cpu().numpy() for p in probs]
    ref_probs = [p[:5] + (torch.full((p[2],), float("nan"), dtype=torch.float32, device="cuda"),)
                 for p in probs]
    grp = B.Group(ref_probs)
    grp.run()
    sync()
    grp.close()
    ref = [p[5].cpu().numpy() for p in ref_probs]
    return got, ref


def check(host, got, ref, what, oracle=True):
    for (t, w, n, k, x), y, yr in zip(host, got, ref):
        assert_bits_equal(y, yr, "%s: batch vs plan %s %dx%d" % (what, t, n, k))
        if oracle:
            y64, a = pnref.gemv_f64(t, w, n, k, x)
            assert_gemv_close(y, y64, a, "%s: %s %dx%d" % (what, t, n, k))


# problems of whole 8-block passes (the register-pipeline kernel takes them)
STREAM_1 = [("pn3t", 100, 5120), ("pn4t", 37, 5120), ("pn4t", 300, 6144), ("pn3t", 1, 640),
            ("pn4t", 65, 17408), ("pn3t", 2000, 1280)]
STREAM_2 = [("pn4t", 9, 6144), ("pn3t", 33, 640)]
# every problem fits the row-tile kernel (periods per row 8, 10, 12, 1, 34, 3, 7)
ROWS_1 = [("pn3t", 100, 5120), ("pn4t", 37, 5120), ("pn4t", 300, 6144), ("pn3t", 1, 640),
          ("pn4t", 65, 17408), ("pn3t", 2000, 80 * 24), ("pn4t", 3, 64 * 56)]
ROWS_2 = [("pn4t", 20, 5120), ("pn3t", 5, 80 * 24)]


def test_batch_stream_two_calls():
    say("batch on the register kernel: two calls, the second smaller")
    h1, p1 = make_problems(STREAM_1, 1)
    got, ref = run_both(p1, "gemv_stream_batch")
    check(h1, got, ref, "call 1")
    h2, p2 = make_problems(STREAM_2, 2)
    got2, ref2 = run_both(p2, "gemv_stream_batch")
    check(h2, got2, ref2, "call 2")
    # the first call's outputs are untouched by the second
    for p, y in zip(p1, got):
        assert_bits_equal(p[5].cpu().numpy(), y, "call 1 outputs after call 2")


def test_batch_rows_forced_two_calls():
    say("batch on the row-tile kernel (forced): two calls, the second smaller")
    B.pn_set_gemv_kernel("rows")
    try:
        h1, p1 = make_problems(ROWS_1, 3)
        got, ref = run_both(p1, "gemv_rows_batch")
        check(h1, got, ref, "call 1")
        h2, p2 = make_problems(ROWS_2, 4)
        got2, ref2 = run_both(p2, "gemv_rows_batch")
        check(h2, got2, ref2, "call 2")
    finally:
        B.pn_set_gemv_kernel("auto")


def test_batch_rows_large_two_calls():
    """Launches large enough for the row-tile kernel by the library's own rule
    (at least 32 tiles per CU): eight gate-shaped matrices, then nine smaller
    ones, back to back on one stream, checked after both ran."""
    say("batch, large: 8 x pn3t 17408x5120, then 9 x pn3t 15000x5120")
    h1, p1 = make_problems([("pn3t", 17408, 5120)] * 8, 5)
    h2, p2 = make_problems([("pn3t", 15000, 5120)] * 9, 6)
    B.pn_gemv_batch(p1)
    B.pn_gemv_batch(p2)
    sync()
    assert B.pn_variant_name(B.pn_last_variant()) == "gemv_rows_batch"
    for host, probs in ((h1, p1), (h2, p2)):
        for (t, w, n, k, x), p in zip(host, probs):
            y64, a = pnref.gemv_f64(t, w, n, k, x)
            assert_gemv_close(p[5].cpu().numpy(), y64, a, "large batch %s %dx%d" % (t, n, k))
    got, ref = run_both(p2, "gemv_rows_batch")
    check(h2, got, ref, "call 2 vs plan", oracle=False)


def test_batch_rows_limit():
    """Exactly PN_BATCH_MAX_ROWS rows on the row-tile kernel run; one row
    more is refused before any launch."""
    B.pn_set_gemv_kernel("rows")
    try:
        n = B.BATCH_MAX_ROWS // B.BATCH_MAX_PROBLEMS
        say("batch at the row limit: %d x pn4t %dx512" % (B.BATCH_MAX_PROBLEMS, n))
        g = np.random.default_rng(7)
        w = synth.random_blocks(g, "pn4t", n, 512)
        wd = dev(w)
        xs = [synth.activation(g, 512) for _ in range(B.BATCH_MAX_PROBLEMS)]
        ys = [torch.full((n,), float("nan"), dtype=torch.float32, device="cuda") for _ in xs]
        probs = [("pn4t", wd, n, 512, dev(x), y) for x, y in zip(xs, ys)]
        B.pn_gemv_batch(probs)
        sync()
        assert B.pn_variant_name(B.pn_last_variant()) == "gemv_rows_batch"
        for i in (0, 13, B.BATCH_MAX_PROBLEMS - 1):
            y64, a = pnref.gemv_f64("pn4t", w, n, 512, xs[i])
            assert_gemv_close(ys[i].cpu().numpy(), y64, a, "row limit, problem %d" % i)
        # (the refused call is given buffers of its full size all the same)
        w_over = dev(synth.random_blocks(g, "pn4t", n + 16, 512))
        y_over = torch.empty(n + 16, dtype=torch.float32, device="cuda")
        over = probs[:-1] + [("pn4t", w_over, n + 16, 512, probs[-1][4], y_over)]
        assert B.pn_gemv_batch(over, check=False) == -4
    finally:
        B.pn_set_gemv_kernel("auto")
