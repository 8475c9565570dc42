"""Full-size parity on the 64-layer 27B-shaped sweep (10.16 GB of packed
weights), in the launch configurations the benchmark times.  The oracle
computes sampled rows of every one of the 448 matrices (first, last and
seeded random rows), kept aside while the weights are generated."""
import numpy as np
import pytest

from gpu_util import assert_gemv_close, say, sync

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from bit_quantized_decode_pn3t_amd import _binding as B  # noqa: E402
from bit_quantized_decode_pn3t_amd import sweep as S  # noqa: E402
from oracle import pnref  # noqa: E402

ROWS = 6


def _check_samples(sw, store, m=None, rotated=False):
    outs = {(e["layer"], e["mat"]): e["y"].cpu().numpy() for e in sw.mats}
    worst = 0.0
    for key, smp in store.items():
        y = outs[key]
        n_rows = len(smp["rows"])
        if m is None:
            x = pnref.rotate(smp["x"]) if rotated else smp["x"]
            y64, a = pnref.gemv_f64(smp["type"], smp["W"], n_rows, smp["K"], x)
            worst = max(worst, assert_gemv_close(y[smp["rows"]], y64, a, "sweep %s" % (key,)))
        else:
            y64, a = pnref.gemm_f64(smp["type"], smp["W"], n_rows, smp["K"], smp["x"])
            worst = max(worst, assert_gemv_close(y[:, smp["rows"]], y64, a, "sweep M=8 %s" % (key,)))
    return worst


@pytest.fixture(scope="module")
def sweep_m1():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    store = {}
    say("sweep M=1: generating 64 layers")
    sw = S.Sweep(sample=lambda rec: S.sample_rows(rec, ROWS, store))
    say("sweep M=1: %.2f GB of weights resident" % (sw.weight_bytes / 1e9))
    yield sw, store
    sw.close()
    del sw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("schedule", ["layer", "token", "gemv", "token_rot"])
def test_sweep_m1(sweep_m1, schedule):
    sw, store = sweep_m1
    for e in sw.mats:
        e["y"].fill_(float("nan"))
    say("sweep M=1 schedule %s" % schedule)
    sw.step(schedule)
    sync()
    worst = _check_samples(sw, store, rotated=schedule == "token_rot")
    say("sweep M=1 %s: worst |y-y64|/sum|wx| = %.3g" % (schedule, worst))


def test_sweep_m1_graph(sweep_m1):
    sw, store = sweep_m1
    say("sweep M=1 graph replays")
    g = sw.capture("layer")
    for rep in range(3):
        for e in sw.mats:
            e["y"].fill_(float("nan"))
        sync()
        g.replay()
        sync()
        _check_samples(sw, store)


@pytest.fixture(scope="module")
def sweep_m8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    store = {}
    say("sweep M=8: generating 64 layers")
    sw = S.Sweep(m=8, sample=lambda rec: S.sample_rows(rec, ROWS, store))
    yield sw, store
    sw.close()
    del sw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("math", ["mfma", "mfma_stream", "valu"])
def test_sweep_m8(sweep_m8, math):
    """M = 8 over the full sweep: one grouped launch per token (the benchmark's
    configuration) and one launch per matrix, with the given arithmetic (and
    for MFMA, the library's kernel choice, gemm_rows for these shapes, or
    gemm_stream forced)."""
    sw, store = sweep_m8
    B.pn_set_smallm_math("valu" if math == "valu" else "mfma")
    B.pn_set_gemv_kernel("stream" if math == "mfma_stream" else "auto")
    sw.close()  # plans keep the arithmetic they were created with
    kernel = "gemm_rows_mfma" if math == "mfma" else "gemm_stream_" + ("valu" if math == "valu" else "mfma")
    try:
        for schedule in ("token", "gemv"):
            for e in sw.mats:
                e["y"].fill_(float("nan"))
            say("sweep M=8 %s schedule %s" % (math, schedule))
            sw.step(schedule)
            sync()
            assert B.pn_variant_name(B.pn_last_variant()) == kernel + ("_group" if schedule == "token" else "")
            worst = _check_samples(sw, store, m=8)
            say("sweep M=8 %s %s: worst %.3g" % (math, schedule, worst))
    finally:
        B.pn_set_smallm_math("mfma")
        B.pn_set_gemv_kernel("auto")
        sw.close()
