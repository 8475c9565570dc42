"""Entry points under HIP graph capture: a split-K prefill product (its zero
fill is a kernel, so the call can be captured), a plan with rotated inputs
(its rotation launch is replayed with the GEMV launch), a row-tile M = 1
plan (its tile counters are reset by the kernel itself) and a small-M plan
on the DMA kernel.  Each graph is replayed several times, with eager work
and synchronizations between the replays, and every replay is checked
against the oracle."""
import numpy as np
import pytest

from gpu_util import assert_gemv_close, dev, say, sync

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from bit_quantized_decode_pn3t_amd import _binding as B  # noqa: E402
from bit_quantized_decode_pn3t_amd import synth  # noqa: E402
from oracle import pnref  # noqa: E402


def test_prefill_split_k_graph_replays():
    t, n, k, m = "pn4t", 1024, 5120, 96  # four output tiles: the launch splits K
    g = np.random.default_rng(31)
    w = synth.random_blocks(g, t, n, k, unused_bits=True)
    xm = synth.activation(g, k, m)
    y64, a = pnref.gemm_f64(t, w, n, k, xm)
    wd = dev(w.reshape(-1))
    xd = dev(xm)
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    say("prefill graph: eager")
    B.pn_gemm_prefill(t, wd, n, k, xd, k, m, y, n)
    sync()
    assert_gemv_close(y.cpu().numpy(), y64, a, "prefill eager")
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        B.pn_gemm_prefill(t, wd, n, k, xd, k, m, y, n)
    sync()
    for rep in range(3):
        say("prefill graph: replay %d" % rep)
        y.fill_(float("nan"))  # eager work between the replays
        sync()
        gr.replay()
        sync()
        assert_gemv_close(y.cpu().numpy(), y64, a, "prefill replay %d" % rep)


def test_prefill_group_graph_replays():
    """A grouped prefill launch (three products of both types, tiles shared
    across products) captured into a graph: its arguments are captured by
    value, so every replay recomputes the same products."""
    specs = [("pn3t", 700, 1280, 150), ("pn4t", 300, 1280, 150), ("pn4t", 129, 2560, 33)]
    host, probs = [], []
    for i, (t, n, k, m) in enumerate(specs):
        g = np.random.default_rng([43, i])
        w = synth.random_blocks(g, t, n, k, unused_bits=True)
        xm = synth.activation(g, k, m)
        y64, a = pnref.gemm_f64(t, w, n, k, xm)
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        host.append((t, n, m, y64, a, y))
        probs.append((t, dev(w.reshape(-1)), n, k, dev(xm), k, m, y, n))
    say("prefill group graph: eager")
    B.pn_gemm_prefill_group(probs)
    sync()
    for t, n, m, y64, a, y in host:
        assert_gemv_close(y.cpu().numpy(), y64, a, "prefill group eager %s N=%d" % (t, n))
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        B.pn_gemm_prefill_group(probs)
    sync()
    for rep in range(3):
        say("prefill group graph: replay %d" % rep)
        for *_, y in host:
            y.fill_(float("nan"))  # eager work between the replays
        sync()
        gr.replay()
        sync()
        for t, n, m, y64, a, y in host:
            assert_gemv_close(y.cpu().numpy(), y64, a, "prefill group replay %d %s N=%d" % (rep, t, n))


def test_rotated_plan_graph_replays():
    specs = [("pn3t", 64, 5120), ("pn4t", 48, 6144), ("pn4t", 32, 17408)]
    host, probs = [], []
    for i, (t, n, k) in enumerate(specs):
        g = np.random.default_rng([41, i])
        w = synth.random_blocks(g, t, n, k, unused_bits=True)
        host.append((t, w, n, k, g))
        probs.append((t, dev(w.reshape(-1)), n, k, dev(synth.activation(g, k)),
                      torch.empty(n, dtype=torch.float32, device="cuda")))
    plan = B.Group(probs, rotate=True)
    plan.run()  # warm
    sync()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        plan.run()
    sync()
    for rep in range(3):
        # new activations each time: the replayed rotation must see them
        for (t, w, n, k, g), p in zip(host, probs):
            p[4].copy_(dev(synth.activation(g, k)))
            p[5].fill_(float("nan"))
        sync()
        say("rotated plan graph: replay %d" % rep)
        gr.replay()
        sync()
        for (t, w, n, k, g), p in zip(host, probs):
            x = p[4].cpu().numpy()
            y64, a = pnref.gemv_f64(t, w, n, k, pnref.rotate(x))
            assert_gemv_close(p[5].cpu().numpy(), y64, a, "rotated plan replay %d %s" % (rep, t))
    plan.close()


def _replay_plan(plan, host, probs, fresh, check, what):
    """Capture plan.run() and replay it three times; before each replay the
    inputs are refreshed and the outputs poisoned eagerly."""
    plan.run()  # warm
    sync()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        plan.run()
    sync()
    for rep in range(3):
        for h, p in zip(host, probs):
            fresh(h, p)
        sync()
        say("%s graph: replay %d" % (what, rep))
        gr.replay()
        sync()
        for h, p in zip(host, probs):
            check(h, p, "%s replay %d" % (what, rep))


def test_row_tile_plan_graph_replays():
    """A gemv_rows group plan (pool counters reset by the last wave of each
    run, so the next replay finds them at zero)."""
    specs = [("pn3t", 300, 5120), ("pn4t", 100, 17408), ("pn4t", 64, 6144)]
    host, probs = [], []
    for i, (t, n, k) in enumerate(specs):
        g = np.random.default_rng([43, i])
        w = synth.random_blocks(g, t, n, k, unused_bits=True)
        host.append((t, w, n, k, g))
        probs.append((t, dev(w.reshape(-1)), n, k, dev(synth.activation(g, k)),
                      torch.empty(n, dtype=torch.float32, device="cuda")))
    B.pn_set_gemv_kernel("rows")
    try:
        plan = B.Group(probs)
    finally:
        B.pn_set_gemv_kernel("auto")

    def fresh(h, p):
        p[4].copy_(dev(synth.activation(h[4], h[3])))
        p[5].fill_(float("nan"))

    def check(h, p, what):
        t, w, n, k, _ = h
        y64, a = pnref.gemv_f64(t, w, n, k, p[4].cpu().numpy())
        assert_gemv_close(p[5].cpu().numpy(), y64, a, what)

    _replay_plan(plan, host, probs, fresh, check, "row-tile plan")
    assert B.pn_variant_name(B.pn_last_variant()) == "gemv_rows_group"
    plan.close()


def test_dma_smallm_plan_graph_replays():
    """A small-M plan run by gemm_rows (weights staged by DMA), M = 8 and 16,
    one problem with activations restaged in chunks."""
    specs = [("pn3t", 300, 5120, 8), ("pn4t", 130, 17408, 8), ("pn4t", 64, 6144, 16)]
    host, probs = [], []
    for i, (t, n, k, m) in enumerate(specs):
        g = np.random.default_rng([47, i])
        w = synth.random_blocks(g, t, n, k, unused_bits=True)
        host.append((t, w, n, k, m, g))
        probs.append((t, dev(w.reshape(-1)), n, k, dev(synth.activation(g, k, m)), k, m,
                      torch.empty((m, n), dtype=torch.float32, device="cuda"), n))
    plan = B.Group(probs, smallm=True)

    def fresh(h, p):
        p[4].copy_(dev(synth.activation(h[5], h[3], h[4])))
        p[7].fill_(float("nan"))

    def check(h, p, what):
        t, w, n, k, m, _ = h
        y64, a = pnref.gemm_f64(t, w, n, k, p[4].cpu().numpy())
        assert_gemv_close(p[7].cpu().numpy(), y64, a, what)

    _replay_plan(plan, host, probs, fresh, check, "small-M plan")
    assert B.pn_variant_name(B.pn_last_variant()) == "gemm_rows_mfma_group"
    plan.close()
