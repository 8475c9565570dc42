"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin takes an ``oracle.pnref.Oracle`` and raises AssertionError when the
oracle disagrees with what the pages and the mathematics fix:
  - hand-worked golden blocks and GEMVs (tests/golden/, worked by hand from the
    tensorless page "Why a P100-native weight format");
  - IEEE fp16 conversions against numpy's (a library routine);
  - closed forms: 34-byte blocks, 3.40 / 4.25 bits per weight, 5120 = 64 pn3t
    blocks ("Every block is 34 bytes");
  - invariants: zero is a code and every weight is d times an integer in
    -4..+3 (pn3t) or -8..+7 (pn4t) ("Zero is a code, and the scale has a
    sign"); decode is exact ("Exact decode in fp32"); the two 16-bit halves
    decode independently ("Codes never straddle the two halves of a word");
  - brute force: exact rational GEMV sums (fractions.Fraction) on tiny inputs
    and an exhaustive nearest-code search for the quantizer;
  - the activation rotation: a case worked by hand, the closed-form columns
    of the Sylvester matrix, scipy's Hadamard matrix with numpy's fp16
    rounding, and length preservation.
The same pins run against deliberately broken copies of the oracle in
test_oracle_mutants.py, to show that a plausible mistake fails at least one.
"""
import struct
from fractions import Fraction

import numpy as np

from golden_io import load_blocks, load_gemv

Z = {"pn3t": 4, "pn4t": 8}
BITS = {"pn3t": 3, "pn4t": 4}
CODES_PER_WORD = {"pn3t": 10, "pn4t": 8}
WPB = {"pn3t": 80, "pn4t": 64}


def _f32_bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _same_bits(a, b):
    """Bit equality, any NaN equal to any NaN."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(nan | (_f32_bits(a) == _f32_bits(b))))


# ---------------------------------------------------------------------------
# fp16 conversions
# ---------------------------------------------------------------------------
def pin_half_to_float_all(o):
    bits = np.arange(65536, dtype=np.uint32)
    ours = np.array([o.half_to_float(int(b)) for b in bits], np.float32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float32)
    assert _same_bits(ours, ref), "half_to_float differs from IEEE binary16"


def pin_double_to_half(o):
    rs = np.random.default_rng(7)
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, -65520.0, 1e9, 2.0 ** -24,
            2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -12),
            1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -11 + 2.0 ** -30, 2049.0, 2051.0]
    vals += list(rs.standard_normal(2000) * 0.01) + list(rs.standard_normal(2000) * 1000)
    vals += list(rs.uniform(-2.0 ** -13, 2.0 ** -13, 2000))
    # exact midpoints between neighbouring halves (ties to even)
    h = rs.integers(0, 0x7bff, 500).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    vals += list((lo + hi) / 2)
    for v in vals:
        ours = o.double_to_half(v)
        with np.errstate(over="ignore"):
            ref = int(np.array([v], np.float64).astype(np.float16).view(np.uint16)[0])
        assert ours == ref, "double_to_half(%r) = %#06x, IEEE gives %#06x" % (v, ours, ref)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
def pin_closed_forms(o):
    assert o.lib.pnref_block_bytes() == 34
    assert o.weights_per_block("pn3t") == 80 and o.weights_per_block("pn4t") == 64
    assert abs(34 * 8 / 80 - 3.40) < 1e-12 and abs(34 * 8 / 64 - 4.25) < 1e-12
    assert o.row_bytes("pn3t", 5120) == 64 * 34
    assert o.zero_point("pn3t") == 4 and o.zero_point("pn4t") == 8


def pin_goldens(o):
    for gid, (t, blk, expect) in load_blocks().items():
        got = o.decode_block(t, blk)
        assert got.size == expect.size, gid
        assert np.array_equal(_f32_bits(got), expect), "golden %s: %s != %s" % (
            gid, _f32_bits(got)[:10], expect[:10])


def pin_golden_alignment(o):
    """G4 as block 1 of a row whose base sits 2 bytes into the buffer."""
    blocks = load_blocks()
    _, g1, _ = blocks["G1"]
    _, g4, e4 = blocks["G4"]
    buf = np.zeros(2 + 68, np.uint8)
    buf[2:36] = g1
    buf[36:70] = g4
    out = o.dequantize("pn3t", buf[2:], 1, 160)
    assert np.array_equal(_f32_bits(out[0, 80:]), e4)


def _random_blocks(rs, t, nblk, junk_bits=False):
    words = rs.integers(0, 2 ** 32, size=(nblk, 8), dtype=np.uint64).astype(np.uint32)
    if t == "pn3t" and not junk_bits:
        words &= np.uint32(0x7FFF7FFF)
    d = rs.integers(0, 0x10000, size=nblk).astype(np.uint16)
    # keep scales finite for the arithmetic pins
    d = np.where((d & 0x7C00) == 0x7C00, d & 0x83FF, d).astype(np.uint16)
    raw = np.empty((nblk, 34), np.uint8)
    raw[:, :2] = d.view(np.uint8).reshape(nblk, 2)
    raw[:, 2:] = words.view(np.uint8).reshape(nblk, 32)
    return raw, d, words


def pin_range_and_zero(o):
    rs = np.random.default_rng(11)
    for t in ("pn3t", "pn4t"):
        raw, d, _ = _random_blocks(rs, t, 300)
        z = Z[t]
        for i in range(raw.shape[0]):
            w = o.decode_block(t, raw[i]).astype(np.float64)
            dd = float(np.float16(d[i:i + 1].view(np.float16)[0]))
            if dd == 0.0:
                assert np.all(w == 0.0)
                continue
            steps = w / dd
            assert np.all(steps == np.round(steps)), "decoded weight is not d times an integer"
            assert steps.min() >= -z and steps.max() <= z - 1, "step outside -z..z-1"
            # exactness: the fp32 product equals the exact rational product
            assert np.all(w == dd * steps)


def pin_halves_independent(o):
    """Zeroing all high halves changes only odd slots; zeroing low halves only even ones."""
    rs = np.random.default_rng(12)
    for t in ("pn3t", "pn4t"):
        raw, _, words = _random_blocks(rs, t, 50)
        for i in range(raw.shape[0]):
            base = o.decode_block(t, raw[i])
            for keep_mask, changed_parity in ((0x0000FFFF, 1), (0xFFFF0000, 0)):
                r2 = raw[i].copy()
                r2[2:] = (words[i] & np.uint32(keep_mask)).view(np.uint8)
                out = o.decode_block(t, r2)
                unchanged = np.arange(out.size) % 2 != changed_parity
                assert _same_bits(out[unchanged], base[unchanged])


def pin_unused_bits_ignored(o):
    rs = np.random.default_rng(13)
    raw, _, words = _random_blocks(rs, "pn3t", 50)
    for i in range(raw.shape[0]):
        r2 = raw[i].copy()
        r2[2:] = (words[i] | np.uint32(0x80008000)).view(np.uint8)
        assert _same_bits(o.decode_block("pn3t", r2), o.decode_block("pn3t", raw[i]))


def pin_one_hot_codes(o):
    """A block with every code at z except slot j: only weight j is nonzero.
    Slot j lives in word j // C, half j % 2, at offset b * ((j % C) // 2)."""
    for t in ("pn3t", "pn4t"):
        b, c, z = BITS[t], CODES_PER_WORD[t], Z[t]
        for j in range(WPB[t]):
            codes = np.full(WPB[t], z)
            codes[j] = 0
            words = []
            for wi in range(8):
                q = 0
                for s in range(c):
                    slot = wi * c + s
                    q |= int(codes[slot]) << (16 * (s % 2) + b * (s // 2))
                words.append(q)
            blk = np.frombuffer(struct.pack("<H8I", 0x3C00, *words), np.uint8)
            out = o.decode_block(t, blk)
            nz = np.nonzero(out)[0]
            assert list(nz) == [j] and out[j] == -z, (t, j, nz)


# ---------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------
def pin_gemv_goldens(o):
    for gid, g in load_gemv().items():
        y, a = o.gemv_f64(g["type"], g["w"], g["w"].shape[0], g["k"], g["x"])
        assert np.array_equal(y, g["y"]), "%s: y %s != %s" % (gid, y, g["y"])
        assert np.array_equal(a, g["a"]), "%s: a %s != %s" % (gid, a, g["a"])


def _exact_dot(weights_f32, x_f16):
    s = Fraction(0)
    t = Fraction(0)
    for w, x in zip(weights_f32.tolist(), x_f16.astype(np.float64).tolist()):
        p = Fraction(w) * Fraction(x)
        s += p
        t += abs(p)
    return s, t


def pin_gemv_exact(o):
    """fp64 oracle vs exact rational sums, within (K-1) * 2^-53 * a, on tiny
    random inputs whose exact weights come from the closed form d*(n-z)."""
    rs = np.random.default_rng(21)
    for t in ("pn3t", "pn4t"):
        b, c, z, wpb = BITS[t], CODES_PER_WORD[t], Z[t], WPB[t]
        n, nb = 3, 2
        k = nb * wpb
        codes = rs.integers(0, 2 ** b, size=(n, nb, wpb))
        dbits = (rs.standard_normal((n, nb)) * 0.05).astype(np.float16).view(np.uint16)
        rows = []
        for r in range(n):
            blks = []
            for j in range(nb):
                words = []
                for wi in range(8):
                    q = 0
                    for s in range(c):
                        q |= int(codes[r, j, wi * c + s]) << (16 * (s % 2) + b * (s // 2))
                    words.append(q)
                blks.append(struct.pack("<H8I", int(dbits[r, j]), *words))
            rows.append(np.frombuffer(b"".join(blks), np.uint8))
        w = np.stack(rows)
        x = (rs.standard_normal(k) * 2).astype(np.float16)
        y, a = o.gemv_f64(t, w, n, k, x)
        for r in range(n):
            exact_w = np.array([float(Fraction(float(dbits[r, j:j + 1].view(np.float16)[0]))
                                      * (int(codes[r, j, s]) - z))
                                for j in range(nb) for s in range(wpb)], np.float64)
            s_exact, a_exact = _exact_dot(exact_w, x)
            bound = (k - 1) * 2.0 ** -53 * float(a_exact)
            assert abs(Fraction(y[r]) - s_exact) <= Fraction(bound) + Fraction(1, 2 ** 1074)
            assert abs(Fraction(a[r]) - a_exact) <= Fraction(bound) + Fraction(1, 2 ** 1074)


def pin_gemv_special(o):
    """One-hot x returns the decoded weight exactly; codes all z give +-0;
    d = 1 and x = 1 give the exact integer sum of (n - z)."""
    rs = np.random.default_rng(22)
    for t in ("pn3t", "pn4t"):
        wpb = WPB[t]
        raw, _, _ = _random_blocks(rs, t, 4)
        w = raw.reshape(2, -1)
        k = 2 * wpb
        dense = o.dequantize(t, w, 2, k)
        for kk in (0, 1, wpb - 1, wpb, k - 1, int(rs.integers(0, k))):
            x = np.zeros(k, np.float16)
            x[kk] = 1.0
            y, _ = o.gemv_f64(t, w, 2, k, x)
            assert np.array_equal(y, dense[:, kk].astype(np.float64))
        # all codes z
        blocks = load_blocks()
        zero_blk = blocks["G2"][1] if t == "pn3t" else blocks["G6"][1]
        wz = np.tile(zero_blk, 3).reshape(1, -1)
        y, a = o.gemv_f64(t, wz, 1, 3 * wpb, (rs.standard_normal(3 * wpb)).astype(np.float16))
        assert y[0] == 0.0 and a[0] == 0.0
        # d = 1, x = 1
        raw2 = raw.copy()
        raw2[:, 0] = 0x00
        raw2[:, 1] = 0x3C
        y, _ = o.gemv_f64(t, raw2.reshape(1, -1), 1, 4 * wpb, np.ones(4 * wpb, np.float16))
        dense = o.dequantize(t, raw2.reshape(1, -1), 1, 4 * wpb)
        codes_sum = 0
        b, c, z = BITS[t], CODES_PER_WORD[t], Z[t]
        for i in range(4):
            words = raw2[i, 2:].view(np.uint32)
            for q in words.tolist():
                for s in range(c):
                    codes_sum += ((q >> (16 * (s % 2) + b * (s // 2))) & (2 ** b - 1)) - z
        assert y[0] == float(codes_sum), (y[0], codes_sum)
        assert float(dense.sum()) == float(codes_sum)


def pin_gemm_reduces_to_gemv(o):
    rs = np.random.default_rng(23)
    for t in ("pn3t", "pn4t"):
        raw, _, _ = _random_blocks(rs, t, 15)
        w = raw.reshape(5, -1)
        k = 3 * WPB[t]
        xm = rs.standard_normal((4, k)).astype(np.float16)
        ym, am = o.gemm_f64(t, w, 5, k, xm)
        for m in range(4):
            y, a = o.gemv_f64(t, w, 5, k, xm[m])
            assert np.array_equal(ym[m], y) and np.array_equal(am[m], a)


# ---------------------------------------------------------------------------
# quantizer
# ---------------------------------------------------------------------------
def pin_quantizer_round_trip(o):
    """Decode a block whose largest weight sits on code 0 (the -z step), then
    quantize it again: the bytes come back identical (the step grid is exact)."""
    rs = np.random.default_rng(31)
    for t in ("pn3t", "pn4t"):
        b, c, z, wpb = BITS[t], CODES_PER_WORD[t], Z[t], WPB[t]
        for _ in range(40):
            codes = rs.integers(1, 2 ** b, size=wpb)
            codes[rs.integers(0, wpb)] = 0  # the full -z step, strictly largest |w|
            d16 = np.float16(abs(rs.standard_normal()) * 0.01 + 1e-3) * (1 if rs.random() < 0.5 else -1)
            words = []
            for wi in range(8):
                q = 0
                for s in range(c):
                    q |= int(codes[wi * c + s]) << (16 * (s % 2) + b * (s // 2))
                words.append(q)
            blk = np.frombuffer(struct.pack("<H8I", int(np.array([d16], np.float16).view(np.uint16)[0]),
                                            *words), np.uint8)
            wf = o.decode_block(t, blk)
            again = o.quantize(t, wf.reshape(1, -1), 1, wpb)
            assert np.array_equal(again.reshape(-1), blk), t


def pin_quantizer_rules(o):
    """Scale = fp16(-w*/z) (checked against numpy's fp16 rounding); the argmax
    weight decodes to exactly -z*d; every code is the nearest one (exhaustive
    search over all 2^b codes, ties to even) and unclamped errors are <= |d|/2."""
    rs = np.random.default_rng(32)
    for t in ("pn3t", "pn4t"):
        b, z, wpb = BITS[t], Z[t], WPB[t]
        wf = (rs.standard_normal((6, wpb * 3)) * 0.02).astype(np.float32)
        packed = o.quantize(t, wf, 6, wpb * 3)
        dense = o.dequantize(t, packed, 6, wpb * 3)
        for r in range(6):
            for j in range(3):
                blkw = wf[r, j * wpb:(j + 1) * wpb].astype(np.float64)
                istar = int(np.argmax(np.abs(blkw)))
                d_expect = np.array([-blkw[istar] / z], np.float64).astype(np.float16)[0]
                raw = packed[r, j * 34:(j + 1) * 34]
                d_got = raw[:2].view(np.float16)[0]
                assert d_got.view(np.uint16) == d_expect.view(np.uint16)
                d = float(d_got)
                wq = dense[r, j * wpb:(j + 1) * wpb].astype(np.float64)
                assert wq[istar] == -z * d
                for i in range(wpb):
                    cand = [abs(blkw[i] - d * (n - z)) for n in range(2 ** b)]
                    best = min(cand)
                    n_got = int(round(wq[i] / d)) + z
                    assert cand[n_got] == best, (t, r, j, i)
                    ties = [n for n in range(2 ** b) if cand[n] == best]
                    if len(ties) > 1:  # exact tie: rint picks the even step (n - z even)
                        assert (n_got - z) % 2 == 0
                    if 0 < n_got < 2 ** b - 1:
                        assert abs(blkw[i] - wq[i]) <= abs(d) / 2


def pin_quantizer_edges(o):
    # all-zero block: scale +0, every code z
    for t in ("pn3t", "pn4t"):
        wpb = WPB[t]
        packed = o.quantize(t, np.zeros((1, wpb), np.float32), 1, wpb)
        assert packed[0, 0] == 0 and packed[0, 1] == 0
        assert np.all(o.dequantize(t, packed, 1, wpb) == 0)
    # ties in |w| go to the lowest index: the first of two equal magnitudes of
    # opposite sign sets the sign of the scale
    for t in ("pn3t", "pn4t"):
        wpb, z = WPB[t], Z[t]
        w = np.zeros((1, wpb), np.float32)
        w[0, 5] = 0.5
        w[0, 9] = -0.5
        packed = o.quantize(t, w, 1, wpb)
        d = float(packed[0, :2].view(np.float16)[0])
        assert d == -0.5 / z
    # exact half-step ties round to the even step; a weight past the top step
    # clamps to code 2^b - 1.  pn3t: max 0.5 -> d = fp16(-0.5/4) = -0.125
    w = np.zeros((1, 80), np.float32)
    w[0, 0] = 0.5
    w[0, 1] = -0.3125   # w/d = 2.5  -> step 2 (not 3)
    w[0, 2] = 0.1875    # w/d = -1.5 -> step -2 (not -1)
    w[0, 3] = 0.0625    # w/d = -0.5 -> step 0 (code z: decodes to -0.0)
    packed = o.quantize("pn3t", w, 1, 80)
    dq = o.dequantize("pn3t", packed, 1, 80)[0]
    assert float(packed[0, :2].view(np.float16)[0]) == -0.125
    assert dq[0] == 0.5 and dq[1] == -0.25 and dq[2] == 0.25 and dq[3] == 0.0
    w = np.zeros((1, 80), np.float32)
    w[0, 0] = -0.5      # d = +0.125
    w[0, 1] = 0.49      # w/d = 3.92 -> step 4 does not exist: clamps to +3
    packed = o.quantize("pn3t", w, 1, 80)
    dq = o.dequantize("pn3t", packed, 1, 80)[0]
    assert dq[0] == -0.5 and dq[1] == 0.375 and np.all(dq[2:] == 0)
    # out of fp16 range refuses
    w = np.full((1, 80), 1e6, np.float32)
    try:
        o.quantize("pn3t", w, 1, 80)
    except ValueError:
        pass
    else:
        raise AssertionError("quantizer accepted a block whose scale overflows fp16")


# ---------------------------------------------------------------------------
# Hadamard rotation of the activations (tensorless, "How Qwen3.8-27B-PN3 uses
# it"; block size, order and scale are readings, see pnref.c)
# ---------------------------------------------------------------------------
def _sylvester_sign(i, j):
    return -1.0 if bin(i & j).count("1") & 1 else 1.0


def pin_rotate_hand_worked(o):
    """B = 4 worked by hand: H4 [1,2,3,4] / 2 = [10,-2,-4,0] / 2; zeros are +0."""
    got = o.rotate(np.array([1, 2, 3, 4], np.float16), 4)
    assert got.tolist() == [5.0, -1.0, -2.0, 0.0], got
    assert not np.signbit(got[3])
    got = o.rotate(np.array([-0.0, -0.0, -0.0, -0.0], np.float16), 4)
    assert got.tolist() == [0.0] * 4 and not np.any(np.signbit(got)), got
    # B = 16: x = e_5 * 4 -> column 5 of H16 (entries +-1), times 4 / 4
    x = np.zeros(16, np.float16)
    x[5] = 4.0
    got = o.rotate(x, 16)
    assert got.tolist() == [_sylvester_sign(i, 5) for i in range(16)], got


def pin_rotate_unit_columns(o):
    """Closed form: the rotation of 32 e_j is column j of the 1024 Sylvester
    matrix, (-1)^popcount(i & j), and rotating it again gives 32 e_j back
    (H / 32 is symmetric and orthogonal)."""
    for j in (0, 1, 2, 3, 77, 512, 1000, 1023):
        x = np.zeros(2048, np.float16)
        x[1024 + j] = 32.0
        got = o.rotate(x).astype(np.float64)
        want = np.zeros(2048)
        want[1024:] = [_sylvester_sign(i, j) for i in range(1024)]
        assert np.array_equal(got, want), "column %d" % j
        back = o.rotate(got.astype(np.float16))
        assert np.array_equal(back.astype(np.float64), x.astype(np.float64)), "involution %d" % j


def pin_rotate_library(o):
    """Against scipy's Sylvester Hadamard matrix and numpy's fp16 rounding of
    the fp64 product (exact here), for every block size the oracle takes:
    N(0,1), wide-range and tie-prone inputs, results that overflow fp16 and
    results that are fp16 subnormals."""
    import scipy.linalg
    rs = np.random.default_rng(11)
    for b in (4, 16, 64, 256, 1024):
        h = scipy.linalg.hadamard(b).astype(np.float64)
        xs = [rs.standard_normal(4 * b),
              rs.standard_normal(4 * b) * np.exp2(rs.integers(-20, 12, 4 * b)),
              np.round(rs.standard_normal(4 * b) * 64) / 64 + np.exp2(-11.0),
              np.full(4 * b, 60000.0),
              rs.standard_normal(4 * b) * 2.0 ** -18]
        for x in xs:
            x = x.astype(np.float16)
            exact = ((x.astype(np.float64).reshape(-1, b) @ h) / np.sqrt(b)).reshape(-1)
            with np.errstate(over="ignore"):
                want = exact.astype(np.float16)
            # an exact zero is +0; a tiny negative value still rounds to -0
            want = np.where(exact == 0, np.float16(0), want)
            got = o.rotate(x, b)
            assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), "block %d" % b


def pin_rotate_norm(o):
    """Orthonormal: the rotated block keeps the vector's length, up to the
    fp16 rounding of each output."""
    rs = np.random.default_rng(12)
    x = rs.standard_normal(5120).astype(np.float16)
    got = o.rotate(x).astype(np.float64).reshape(5, 1024)
    n0 = np.linalg.norm(x.astype(np.float64).reshape(5, 1024), axis=1)
    assert np.allclose(np.linalg.norm(got, axis=1), n0, rtol=2.0 ** -10)


def pin_rotate_rejects_shapes(o):
    for k, b in ((1000, 1024), (1024, 512), (1024, 2048), (12, 3)):
        try:
            o.rotate(np.zeros(k, np.float16), b)
        except ValueError:
            continue
        raise AssertionError("rotate took K=%d, block %d" % (k, b))


ALL_PINS = [pin_half_to_float_all, pin_double_to_half, pin_closed_forms, pin_goldens,
            pin_golden_alignment, pin_range_and_zero, pin_halves_independent,
            pin_unused_bits_ignored, pin_one_hot_codes, pin_gemv_goldens, pin_gemv_exact,
            pin_gemv_special, pin_gemm_reduces_to_gemv, pin_quantizer_round_trip,
            pin_quantizer_rules, pin_quantizer_edges, pin_rotate_hand_worked,
            pin_rotate_unit_columns, pin_rotate_library, pin_rotate_norm, pin_rotate_rejects_shapes]
