"""Full-size parity on the 64-layer 27B-shaped sweep (10.16 GB of packed
weights), in the launch configurations the benchmark times.  The oracle
computes every output row of all 448 matrices (its fp64 sums and sum|w x|,
taken while the weights are generated), and every row of the GPU's output is
checked against them.  pn3t words carry random junk in their unused bits 15
and 31, which every reader must ignore."""
import numpy as np
import pytest

from gpu_util import assert_gemv_close, say, sync

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from bit_quantized_decode_pn3t_amd import _binding as B  # noqa: E402
from bit_quantized_decode_pn3t_amd import sweep as S  # noqa: E402
from bit_quantized_decode_pn3t_amd import synth  # noqa: E402
from oracle import pnref  # noqa: E402

# the kernel each M = 1 schedule runs at these shapes
M1_VARIANT = {"token": "gemv_rows_group", "token_rot": "gemv_rows_group", "layer": "gemv_stream_group",
              "gemv": "gemv_stream"}


def oracle_rows(store, rotated=False, batch=None):
    """Callback for Sweep(sample=...): the oracle's y64 and sum|w x| for every
    row of the matrix (and, with `rotated`, for its rotated input too; with
    `batch`, also for the M = batch activations that Sweep.batch_view draws)."""
    def sample(rec):
        key = (rec["layer"], rec["mat"])
        t, n, k, w, x = rec["type"], rec["N"], rec["K"], rec["W"], rec["x"]
        if x.ndim == 1:
            ent = {"plain": pnref.gemv_f64(t, w, n, k, x)}
            if rotated:
                ent["rot"] = pnref.gemv_f64(t, w, n, k, pnref.rotate(x))
        else:
            ent = {"plain": pnref.gemm_f64(t, w, n, k, x)}
        if batch:
            xb = synth.activation(synth.rng(4, rec["layer"], rec["mat"]), k, batch)
            ent["batch"] = pnref.gemm_f64(t, w, n, k, xb)
        store[key] = ent
    return sample


def check_all_rows(sw, store, which="plain"):
    """Every output of every matrix within 1e-5 * sum|w x| of the oracle."""
    worst, rows = 0.0, 0
    for e in sw.mats:
        key = (e["layer"], e["mat"])
        y64, a = store[key][which]
        y = e["y"].cpu().numpy()
        worst = max(worst, assert_gemv_close(y, y64, a, "sweep %s %s" % (which, key)))
        rows += y.size
    return worst, rows


@pytest.fixture(scope="module")
def sweep_m1():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    store = {}
    say("sweep M=1: generating 64 layers and the oracle's rows")
    sw = S.Sweep(sample=oracle_rows(store, rotated=True), unused_bits=True)
    say("sweep M=1: %.2f GB of weights resident" % (sw.weight_bytes / 1e9))
    yield sw, store
    sw.close()
    del sw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("schedule", ["token", "layer", "gemv", "token_rot"])
def test_sweep_m1(sweep_m1, schedule):
    sw, store = sweep_m1
    for e in sw.mats:
        e["y"].fill_(float("nan"))
    say("sweep M=1 schedule %s" % schedule)
    sw.step(schedule)
    sync()
    assert B.pn_variant_name(B.pn_last_variant()) == M1_VARIANT[schedule]
    worst, rows = check_all_rows(sw, store, "rot" if schedule == "token_rot" else "plain")
    assert rows == 64 * (6144 + 2 * 1024 + 5120 + 2 * 17408 + 5120)
    say("sweep M=1 %s: %d rows, worst |y-y64|/sum|wx| = %.3g" % (schedule, rows, worst))


@pytest.mark.parametrize("schedule", ["layer", "token"])
def test_sweep_m1_graph(sweep_m1, schedule):
    """A captured token (one launch) or layer (256 launches) schedule, replayed
    three times with eager work between the replays: every row every time
    (the token plan's tile counters must be reset by each run for the next)."""
    sw, store = sweep_m1
    say("sweep M=1 graph replays, %s schedule" % schedule)
    g = sw.capture(schedule)
    for rep in range(3):
        for e in sw.mats:
            e["y"].fill_(float("nan"))
        sync()
        g.replay()
        sync()
        check_all_rows(sw, store)
    sw.graph = None


@pytest.fixture(scope="module")
def sweep_m8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    store = {}
    say("sweep M=8: generating 64 layers and the oracle's rows (M = 8 and 16)")
    sw = S.Sweep(m=8, sample=oracle_rows(store, batch=16), unused_bits=True)
    yield sw, store
    sw.close()
    del sw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("math", ["mfma", "mfma_stream", "valu"])
def test_sweep_m8(sweep_m8, math):
    """M = 8 over the full sweep: one grouped launch per token (the benchmark's
    configuration) and one launch per matrix, with the given arithmetic (and
    for MFMA, the library's kernel choice, gemm_rows for these shapes, or
    gemm_stream forced).  Every one of the 27.3 M outputs is checked."""
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
            worst, rows = check_all_rows(sw, store)
            say("sweep M=8 %s %s: %d outputs, worst %.3g" % (math, schedule, rows, worst))
    finally:
        B.pn_set_smallm_math("mfma")
        B.pn_set_gemv_kernel("auto")
        sw.close()


def test_sweep_m16(sweep_m8):
    """M = 16 (the widest small-batch tile) over the full sweep, one grouped
    launch per token on the same resident weights: every one of the 54.5 M
    outputs against the oracle."""
    sw, store = sweep_m8
    v = sw.batch_view(16)
    try:
        for e in v.mats:
            e["y"].fill_(float("nan"))
        say("sweep M=16 token schedule")
        v.step("token")
        sync()
        assert B.pn_variant_name(B.pn_last_variant()) == "gemm_rows_mfma_group"
        worst, rows = check_all_rows(v, store, "batch")
        assert rows == 16 * 64 * (6144 + 2 * 1024 + 5120 + 2 * 17408 + 5120)
        say("sweep M=16: %d outputs, worst %.3g" % (rows, worst))
    finally:
        v.close()
