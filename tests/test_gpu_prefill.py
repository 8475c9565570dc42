"""Parity of the prefill GEMM (pn_gemm_prefill: any number of activation
rows, weights decoded inside an MFMA GEMM) against the CPU oracle's fp64
product, within 1e-5 * sum|w x| for every (row of X, weight row)."""
import numpy as np
import pytest

from gpu_util import assert_gemv_close, dev, say, sync

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
# period to the down projection's 17408
SHAPES = [("pn3t", 256, 5120, 1), ("pn3t", 256, 5120, 17), ("pn3t", 256, 5120, 300), ("pn4t", 320, 6144, 129),
          ("pn4t", 130, 17408, 64), ("pn3t", 1000, 640, 257), ("pn4t", 96, 128, 200), ("pn3t", 33, 160, 5)]


@pytest.mark.parametrize("t,n,k,m", SHAPES)
def test_prefill_matches_oracle(t, n, k, m):
    g = np.random.default_rng([n, k, m])
    w = synth.random_blocks(g, t, n, k)
    xm = synth.activation(g, k, m)
    say("prefill %s N=%d K=%d M=%d" % (t, n, k, m))
    y = gpu_prefill(t, w, n, k, xm)
    y64, a = pnref.gemm_f64(t, w, n, k, xm)
    assert_gemv_close(y, y64, a, "prefill %s %dx%d M=%d" % (t, n, k, m))


def test_prefill_leading_dimensions():
    g = np.random.default_rng(5)
    t, n, k, m = "pn4t", 200, 1024, 150
    w = synth.random_blocks(g, t, n, k)
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
    w2 = synth.random_blocks(g, t, 140, k)
    say("prefill outliers %s" % t)
    y64, a = pnref.gemm_f64(t, w2, 140, k, xm)
    assert_gemv_close(gpu_prefill(t, w2, 140, k, xm), y64, a, "prefill outliers")


def test_prefill_full_size_sampled():
    """The gate projection's shape (pn3t 17408 x 5120) with a 512-token
    prompt: every output of sampled weight rows (first, last, random)."""
    t, n, k, m = "pn3t", 17408, 5120, 512
    g = np.random.default_rng(21)
    w = synth.random_blocks(g, t, n, k)
    xm = synth.activation(g, k, m)
    say("prefill full size %s %dx%d M=%d" % (t, n, k, m))
    y = gpu_prefill(t, w, n, k, xm)
    rows = np.array(sorted(set([0, 1, 127, 128, n - 1] + list(g.integers(0, n, 11)))))
    y64, a = pnref.gemm_f64(t, w[rows], len(rows), k, xm)
    assert_gemv_close(y[:, rows], y64, a, "prefill full size")
