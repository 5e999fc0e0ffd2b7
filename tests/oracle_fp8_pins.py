"""Checks that pin the FP8 (e4m3) oracle to things other than itself.

Each ``pin_*`` takes the forward oracle ``A`` and the FP8 oracle ``F`` and
raises AssertionError when the FP8 oracle disagrees with: the e4m3 format's
properties (largest value 448, smallest normal 2^-6, smallest subnormal
2^-9, 8 evenly spaced values per binade, mirrored signs), a pure-Python
brute force of round-to-nearest-even over all codes in exact rational
arithmetic, the quantisation's defining properties (the scale is the
smallest power of two 2^e, e >= -126, with amax <= 448 * 2^e: values worked
out by hand and the bracketing 448 * 2^(e-1) < amax checked exactly; a zero block gives zero codes and scale 1; each code is the
brute-force encoding of the exactly rounded float32 x * c times 2^-e, also
for a product constructed to land on a tie only after that rounding; heads
are scaled independently), the query's c (log2(e) as the float32 0x3FB8AA3B
times the softmax scale, 1/8 exactly at d = 64), or the plain attention
definition when the inputs are exactly representable (also through a
power-of-two c on the query).  test_oracle_fp8.py runs the same functions
against deliberately broken copies of the oracle.
"""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np


def _f32(x) -> float:
    """Round a Fraction or float to float32 (round to nearest even), as a float."""
    return struct.unpack("<f", struct.pack("<f", float(x)))[0] if not isinstance(x, Fraction) else _f32_frac(x)


def _f32_frac(q: Fraction) -> float:
    # float(q) is correctly rounded to float64; float64 -> float32 double rounding is exact enough
    # only if no tie is created; resolve ties exactly by comparing with neighbours.
    f = struct.unpack("<f", struct.pack("<f", float(q)))[0]
    up = np.nextafter(np.float32(f), np.float32(np.inf))
    dn = np.nextafter(np.float32(f), np.float32(-np.inf))
    best = min((abs(Fraction(float(c)) - q), c) for c in (np.float32(f), up, dn))
    return float(best[1])


def pin_fp8_table(A, F):
    v = F.e4m3_values()
    assert v[0x7E] == 448.0 and np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9 and v[0x00] == 0.0 and v[0x38] == 1.0
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes not increasing"
    for c in range(0x7F):
        assert v[0x80 | c] == -pos[c] or (c == 0 and v[0x80] == 0.0)
    for e in range(1, 16):
        lo = 2.0 ** (e - 7)
        vals = [x for x in pos if lo <= x < 2 * lo]
        assert len(vals) == (8 if e < 15 else 7), ("binade size", e, len(vals))
        assert np.allclose(np.diff(vals), lo / 8), ("spacing", e)
    assert np.allclose(np.diff(pos[:9]), 2.0 ** -9), "subnormal spacing"


def _brute_encode(x: float) -> int:
    """Pure Python: the nearest of all finite magnitudes in exact arithmetic,
    ties to the even code; sign bit from x."""
    q = abs(Fraction(x))
    best_c, best_d = None, None
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        val = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        d = abs(val - q)
        if best_d is None or d < best_d or (d == best_d and c % 2 == 0):
            best_c, best_d = c, d
    return best_c | (0x80 if np.signbit(x) else 0)


def pin_fp8_encode(A, F):
    v = F.e4m3_values()
    xs = []
    for c in range(0x7E):                                   # every tie and quarter point
        a, b = v[c], v[c + 1]
        xs += [a, (a + b) / 2, 0.75 * a + 0.25 * b, 0.25 * a + 0.75 * b, -(a + b) / 2]
    rng = np.random.default_rng(4)
    xs += list(rng.uniform(-448, 448, 300)) + list(rng.standard_normal(300) * 0.01) + [0.0, -0.0, 448.0, -448.0]
    xs = [float(np.float32(x)) for x in xs]
    got = F.e4m3_encode(np.asarray(xs))
    for x, g in zip(xs, got):
        assert int(g) == _brute_encode(x), ("encode", x, hex(int(g)), hex(_brute_encode(x)))


def _exponent_ok(amax: float, e: int) -> bool:
    """e is the scale exponent of amax: 448 * 2^(e-1) < amax <= 448 * 2^e, or
    e = -126 with amax <= 448 * 2^-126, or e = 0 for amax = 0 (exact
    rationals)."""
    if amax == 0:
        return e == 0
    a = Fraction(amax)
    upper = a <= 448 * Fraction(2) ** e
    return upper and (e == -126 or a > 448 * Fraction(2) ** (e - 1))


def _check_block(F, x, c, out, b, h):
    """codes and scale of one (b, h) of quantize_heads(x, c) against exact
    arithmetic: y = float32(x * c) rounded from the exact product, e by the
    exact search, each code the brute-force encoding of y * 2^-e."""
    blk = x[b, :, h, :]
    # the scale needs the whole block's amax (rounding is monotonic, so the
    # float32 products give it); the codes are checked exactly on the first rows
    amax = float(np.abs(np.float32(blk) * np.float32(c)).max())
    y = np.array([[_f32(Fraction(float(v)) * Fraction(float(np.float32(c)))) for v in row] for row in blk[:12]])
    sc = float(out["scale"][b, h])
    e = int(np.log2(sc))
    assert sc == 2.0 ** e and _exponent_ok(amax, e), ("scale", b, h, sc, amax)
    if amax == 0:
        assert np.all(F.e4m3_decode(out["codes"][b, :, h, :]) == 0)
        return
    assert amax <= 448 * 2.0 ** e and (e == -126 or amax > 224 * 2.0 ** e), "scale not the smallest power of two"
    for r in range(y.shape[0]):                       # the first 12 rows element by element
        for k in range(blk.shape[1]):
            want = _brute_encode(float(Fraction(float(y[r, k])) / Fraction(2) ** e))
            assert out["codes"][b, r, h, k] == want, ("code", b, r, h, k)


def pin_fp8_quantize(A, F):
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((2, 37, 3, 16)) * np.array([1.0, 1e-3, 50.0])[None, None, :, None]).astype(np.float32)
    x[1, :, 2, :] = 0.0                                      # one all-zero (b, h)
    for c in (1.0, float(F.query_prescale(16)), 0.3):
        out = F.quantize_heads(x, c)
        for b in range(2):
            for h in range(3):
                _check_block(F, x, c, out, b, h)
        # dequantised values within half a step of x (relative 2^-4; 2^-10 of the scale near zero)
        vals = F.dequantize_heads(out["codes"], out["scale"], c)
        tol = np.maximum(np.abs(x) / 16, 2.0 ** -10 * out["scale"][:, None, :, None] / c) * (1 + 1e-6)
        assert np.all(np.abs(vals - x) <= tol), ("dequantised error above half a step", c)
    # heads are scaled independently: scaling one head leaves the others' codes alone
    codes = F.quantize_heads(x)["codes"]
    x2 = x.copy()
    x2[:, :, 0, :] *= 1000
    assert np.array_equal(F.quantize_heads(x2)["codes"][:, :, 1:, :], codes[:, :, 1:, :])


def pin_fp8_scale_exponent(A, F):
    """Values worked out by hand (448 = 0.875 * 2^9): e(448) = 0, e(449) = 1,
    e(224) = -1, e(1) = -8 (0.875 < 1 <= 1.75), e(3.4e38) = 120 (2^119 is
    below 3.4e38 / 448, 2^120 above), e(1e-40) = e(2^-149) = -126 (clamped),
    e(0) = 0; then, at and next to 448 * 2^k and 224 * 2^k and on random
    magnitudes, the bracketing 448 * 2^(e-1) < amax <= 448 * 2^e in exact
    rationals."""
    hand = {448.0: 0, 449.0: 1, 224.0: -1, 224.00002: 0, 1.0: -8, 3.4e38: 120, 1e-40: -126, 2.0 ** -149: -126,
            0.0: 0, 448.0 * 2.0 ** -126: -126, 448.0 * 2.0 ** -125: -125}
    got = F.scale_exponent(np.asarray(list(hand), dtype=np.float32))
    for (a, want), g in zip(hand.items(), got):
        assert int(g) == want, ("scale exponent", a, int(g), want)
    am = []
    for k in (-140, -130, -126, -125, -10, -1, 0, 1, 7, 60, 100, 119):
        for base in (448.0, 224.0, 300.0):
            v = np.float32(base * 2.0 ** k)
            if not np.isfinite(v) or v == 0:
                continue
            am += [float(v), float(np.nextafter(v, np.float32(np.inf))), float(np.nextafter(v, np.float32(0)))]
    rng = np.random.default_rng(20)
    am += [float(np.float32(v)) for v in np.exp(rng.uniform(-90, 88, 500))]
    got = F.scale_exponent(np.asarray(am, dtype=np.float32))
    for a, g in zip(am, got):
        assert _exponent_ok(a, int(g)), ("scale exponent", a, int(g))


def pin_fp8_query_prescale(A, F):
    """c = float32(s * float32(log2 e)): log2(e) in float32 is 0x3FB8AA3B;
    at d = 64 the default s is 1/8 exactly; a given scale is used as its
    float32; at d = 128, s is 1 / float32(sqrt(128)) rounded to float32
    (sqrt(128) = 8 sqrt(2) rounded to the nearest float32, checked against
    the squares of its neighbours' midpoints)."""
    l2e = Fraction(float(np.frombuffer(struct.pack("<I", 0x3FB8AA3B), dtype=np.float32)[0]))
    assert float(np.float32(F.LOG2E)) == float(l2e)
    assert float(F.query_prescale(64)) == _f32(Fraction(1, 8) * l2e)
    assert float(F.query_prescale(128, 0.3)) == _f32(Fraction(float(np.float32(0.3))) * l2e)
    r = np.float32(np.sqrt(128.0))
    lo = (Fraction(float(r)) + Fraction(float(np.nextafter(r, np.float32(0))))) / 2
    hi = (Fraction(float(r)) + Fraction(float(np.nextafter(r, np.float32(np.inf))))) / 2
    assert lo * lo < 128 < hi * hi, "float32 sqrt(128) not correctly rounded"
    s = _f32(1 / Fraction(float(r)))
    assert float(F.query_prescale(128)) == _f32(Fraction(s) * l2e)
    assert float(F.query_prescale(128, 0.0)) == float(F.query_prescale(128))


def pin_fp8_prescale_rounding(A, F):
    """The product x * c is rounded to float32 once, before the e4m3
    rounding: an element whose float32 product lands exactly on a tie
    between two codes, while its exact product lies on the odd code's side,
    gets the tie's even code (its block's amax element puts e at 0)."""
    v = F.e4m3_values()
    c = F.query_prescale(16)
    cq = Fraction(float(c))
    big = np.float32(400.0 / float(c))
    assert 224 < float(np.float32(big * c)) <= 448
    for k in range(0x30, 0x76):
        t = (v[k] + v[k + 1]) / 2
        x0 = np.float32(t / float(c))
        for x in (x0, np.nextafter(x0, np.float32(np.inf)), np.nextafter(x0, np.float32(0))):
            y32 = float(np.float32(np.float32(x) * c))
            exact = Fraction(float(x)) * cq                 # exact in float64 (48 significant bits)
            if y32 == t and exact != Fraction(t) and _brute_encode(float(exact)) != _brute_encode(t):
                blk = np.asarray([[[[big, x]]]], dtype=np.float32)
                got = F.quantize_heads(blk, c)["codes"][0, 0, 0, 1]
                assert int(got) == _brute_encode(t), ("prescaled tie", float(x), hex(int(got)))
                return
    raise AssertionError("no distinguishing case found")


def pin_fp8_exact_inputs(A, F):
    """Inputs that are e4m3 values times a power of two, with +-448 present in
    every (b, h): the codes are exact, scale is that power of two, and the FP8
    attention equals the plain definition on the same inputs."""
    rng = np.random.default_rng(12)
    v = F.e4m3_values()[:0x7F]
    N, L, H, d = 2, 6, 2, 8

    def mk(p):
        x = rng.choice(np.concatenate([v, -v]), size=(1, L, H, d)) * 2.0 ** p
        x[0, 0, :, 0] = 448.0 * 2.0 ** p
        return x.astype(np.float32)

    q = mk(-6)
    ks, vs = [mk(-7) for _ in range(N)], [mk(-5) for _ in range(N)]
    qq = F.quantize_heads(q)
    kq = [F.quantize_heads(x) for x in ks]
    vq = [F.quantize_heads(x) for x in vs]
    assert np.all(qq["scale"] == 2.0 ** -6)
    assert np.array_equal(F.dequantize_heads(qq["codes"], qq["scale"]), q.astype(np.float64))
    for mask in ("none", "causal"):
        got = F.fp8_rank_attention(qq["codes"], qq["scale"], [x["codes"] for x in kq], [x["scale"] for x in kq],
                                   [x["codes"] for x in vq], [x["scale"] for x in vq], 1, N, mask)
        ref = A.rank_attention(q.astype(np.float64), [x.astype(np.float64) for x in ks],
                               [x.astype(np.float64) for x in vs], 1, N, mask)
        for name in ("o", "lse"):
            assert np.allclose(got[name], ref[name], rtol=1e-12, atol=1e-12), (mask, name)
    # the query through a power-of-two c: codes of q * c, scale 2^-6 * c, and
    # decode * scale / c gives q back exactly, so the attention is unchanged
    c = 0.25
    qc = F.quantize_heads(q, c)
    assert np.all(qc["scale"] == 2.0 ** -8) and np.array_equal(qc["codes"], qq["codes"])
    assert np.array_equal(F.dequantize_heads(qc["codes"], qc["scale"], c), q.astype(np.float64))
    got = F.fp8_rank_attention(qc["codes"], qc["scale"], [x["codes"] for x in kq], [x["scale"] for x in kq],
                               [x["codes"] for x in vq], [x["scale"] for x in vq], 1, N, "causal", q_prescale=c)
    ref = A.rank_attention(q.astype(np.float64), [x.astype(np.float64) for x in ks],
                           [x.astype(np.float64) for x in vs], 1, N, "causal")
    for name in ("o", "lse"):
        assert np.allclose(got[name], ref[name], rtol=1e-12, atol=1e-12), ("prescaled query", name)


# cheap pins first: a planted mistake is usually caught before the slow ones run
ALL_FP8_PINS = [pin_fp8_table, pin_fp8_scale_exponent, pin_fp8_query_prescale, pin_fp8_prescale_rounding,
                pin_fp8_exact_inputs, pin_fp8_quantize, pin_fp8_encode]
