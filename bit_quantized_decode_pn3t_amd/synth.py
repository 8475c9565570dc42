"""Seeded synthetic inputs for the PN GEMV workloads.

Shared by the tests and the benchmark; it holds no PN arithmetic (no decode,
no dot products): it draws random code words, fp16 scales and fp16
activations and lays them out as 34-byte blocks (scale first, then eight
little-endian words, tensorless "Why a P100-native weight format", "Every
block is 34 bytes").

Recipe (numpy PCG64, seeded by SeedSequence([0x504E, config, layer, matrix]),
draws in this order: code words, scale magnitudes, scale signs, activation):
  - pn4t words: uniform u32 (the low and high halves of PCG64's raw 64-bit
    outputs), i.e. eight i.i.d. uniform 4-bit codes per word;
    pn3t words: the same & 0x7fff7fff, i.e. ten i.i.d. uniform 3-bit codes
    with the unused bits 15 and 31 zero (optionally left random);
  - scale d = fp16(s * |N(0,1)| * 0.01) with s = +-1 equiprobable;
  - activations fp16(N(0,1)).
Shapes follow Qwen3.8-27B as the tensorless pages describe it: most GEMV
inputs are 5120 wide, the others 6144 and 17408 ("Every block is 34 bytes":
5120 = 64 pn3t blocks; 6144 and 17408 use pn4t).
"""
import concurrent.futures as _cf

import numpy as np

BLOCK_BYTES = 34
WEIGHTS_PER_BLOCK = {"pn3t": 80, "pn4t": 64}

# One decoder layer of the 27B-shaped sweep: (name, type, N rows, K columns).
SWEEP_LAYER = (
    ("q", "pn3t", 6144, 5120),
    ("k", "pn4t", 1024, 5120),
    ("v", "pn4t", 1024, 5120),
    ("o", "pn4t", 5120, 6144),
    ("gate", "pn3t", 17408, 5120),
    ("up", "pn3t", 17408, 5120),
    ("down", "pn4t", 5120, 17408),
)
SWEEP_LAYERS = 64

CONFIGS = {
    0: "pn3t GEMV, M=1, N=256 x K=5120",
    1: "pn4t GEMV, M=1, down projection N=5120 x K=17408",
    2: "fused gate+up pn3t GEMV, M=1, 2 x (N=17408 x K=5120), quantized N(0,0.02) weights",
    3: "64-layer 27B-shaped sweep, M=1 (q, k, v, o, gate, up, down per layer)",
    4: "64-layer 27B-shaped sweep, M=8",
}


def rng(config, layer=0, matrix=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0x504E, config, layer, matrix])))


def row_bytes(pn_type, k):
    w = WEIGHTS_PER_BLOCK[pn_type]
    if k % w:
        raise ValueError("K=%d is not a multiple of %d" % (k, w))
    return k // w * BLOCK_BYTES


def pack_blocks(scale_bits, words):
    """Lay out blocks: scale_bits uint16 [nblk], words uint32 [nblk, 8] -> uint8 [nblk*34]."""
    nblk = scale_bits.shape[0]
    out = np.empty((nblk, BLOCK_BYTES), np.uint8)
    out[:, 0:2] = np.ascontiguousarray(scale_bits, dtype="<u2").view(np.uint8).reshape(nblk, 2)
    out[:, 2:] = np.ascontiguousarray(words, dtype="<u4").view(np.uint8).reshape(nblk, 32)
    return out.reshape(-1)


def random_blocks(g, pn_type, n, k, unused_bits=False):
    """Random packed matrix, uint8 [n, row_bytes]."""
    nblk = n * (k // WEIGHTS_PER_BLOCK[pn_type])
    row_bytes(pn_type, k)
    words = g.bit_generator.random_raw(nblk * 4).view(np.uint32).reshape(nblk, 8)
    if pn_type == "pn3t" and not unused_bits:
        words &= np.uint32(0x7FFF7FFF)
    mag = np.abs(g.standard_normal(nblk)) * 0.01
    sign = g.integers(0, 2, size=nblk) * 2 - 1
    d = (sign * mag).astype(np.float16).view(np.uint16)
    return pack_blocks(d, words).reshape(n, -1)


def activation(g, k, m=None):
    shape = (k,) if m is None else (m, k)
    return g.standard_normal(shape).astype(np.float16)


def gaussian_weights(g, n, k, sigma=0.02):
    return (g.standard_normal((n, k)) * sigma).astype(np.float32)


def config0():
    g = rng(0)
    w = random_blocks(g, "pn3t", 256, 5120)
    return dict(type="pn3t", N=256, K=5120, W=w, x=activation(g, 5120))


def config1():
    g = rng(1)
    w = random_blocks(g, "pn4t", 5120, 17408)
    return dict(type="pn4t", N=5120, K=17408, W=w, x=activation(g, 17408))


def config2_weights():
    """fp32 gate and up weights of config 2 (quantized by the caller) and x."""
    wg = gaussian_weights(rng(2, 0, 0), 17408, 5120)
    wu = gaussian_weights(rng(2, 0, 1), 17408, 5120)
    x = activation(rng(2, 0, 2), 5120)
    return wg, wu, x


def sweep_matrix(layer, mat, with_x=True, m=None, config=3, unused_bits=False):
    """One matrix of the sweep: weights from config 3's stream (config 4 reuses
    them) and an activation (or an [m, K] batch) from `config`'s stream.
    With `unused_bits`, pn3t words keep random bits 15 and 31 (readers must
    ignore them); the codes are the same either way."""
    name, t, n, k = SWEEP_LAYER[mat]
    g = rng(3, layer, mat)
    w = random_blocks(g, t, n, k, unused_bits=unused_bits)
    out = dict(name=name, type=t, N=n, K=k, W=w)
    if with_x:
        if m is None and config == 3:
            out["x"] = activation(g, k)
        else:
            out["x"] = activation(rng(config, layer, mat), k, m)
    return out


def sweep_matrices(layers=SWEEP_LAYERS, m=None, config=3, threads=8, consume=None, unused_bits=False):
    """Generate every (layer, matrix) of the sweep with a thread pool (numpy's
    generators release the GIL).  With `consume`, each result is handed to it
    (in layer/matrix order) and dropped, so the host never holds the whole set."""
    jobs = [(l, j) for l in range(layers) for j in range(len(SWEEP_LAYER))]
    results = []
    window = 2 * threads  # bounded look-ahead keeps host memory small
    with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
        futs = {}
        for i in range(min(window, len(jobs))):
            futs[i] = ex.submit(sweep_matrix, jobs[i][0], jobs[i][1], True, m, config, unused_bits)
        for i, (l, j) in enumerate(jobs):
            r = futs.pop(i).result()
            nxt = i + window
            if nxt < len(jobs):
                futs[nxt] = ex.submit(sweep_matrix, jobs[nxt][0], jobs[nxt][1], True, m, config, unused_bits)
            r["layer"], r["mat"] = l, j
            if consume is not None:
                consume(r)
            else:
                results.append(r)
    return None if consume is not None else results
