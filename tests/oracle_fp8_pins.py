"""Checks that pin the FP8 (e4m3) oracle to things other than itself.

Each ``pin_*`` takes the forward oracle ``A`` and the FP8 oracle ``F`` and
raises AssertionError when the FP8 oracle disagrees with: the e4m3 format's
properties (largest value 448, smallest normal 2^-6, smallest subnormal
2^-9, 8 evenly spaced values per binade, mirrored signs), a pure-Python
brute force of round-to-nearest-even over all codes in exact rational
arithmetic, the quantisation's defining properties (the amax element maps to
+-448, a zero block gives zero codes and scale 1, the dequantised error is
within half a step, heads are scaled independently, the inverse scale is the
correctly rounded float32 of 448 / amax), or the plain attention definition
when the inputs are exactly representable.  test_oracle_fp8.py runs the same
functions against deliberately broken copies of the oracle.
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


def pin_fp8_quantize(A, F):
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((2, 37, 3, 16)) * np.array([1.0, 1e-3, 50.0])[None, None, :, None]).astype(np.float32)
    x[1, :, 2, :] = 0.0                                      # one all-zero (b, h)
    out = F.quantize_heads(x)
    codes, scale = out["codes"], out["scale"]
    vals = F.e4m3_decode(codes)
    for b in range(2):
        for h in range(3):
            blk = x[b, :, h, :]
            amax = float(np.abs(blk).max())
            if amax == 0:
                assert scale[b, h] == 1.0 and np.all(vals[b, :, h, :] == 0)
                continue
            assert scale[b, h] == _f32(Fraction(amax) / 448), "scale not the correctly rounded amax / 448"
            inv = _f32(Fraction(448) / Fraction(amax))
            i, j = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert abs(vals[b, i, h, j]) == 448.0, "amax element does not map to +-448"
            y = np.clip(np.float32(blk) * np.float32(inv), -448, 448)     # float32 product, one rounding
            assert np.all(np.abs(vals[b, :, h, :] - y) <= np.maximum(np.abs(y) / 16, 2.0 ** -10) + 1e-12), \
                "dequantised error above half a step"
            for r in range(blk.shape[0]):
                for k in range(blk.shape[1]):
                    assert codes[b, r, h, k] == _brute_encode(float(y[r, k])), "code of one element"
    # heads are scaled independently: scaling one head leaves the others' codes alone
    x2 = x.copy()
    x2[:, :, 0, :] *= 1000
    out2 = F.quantize_heads(x2)
    assert np.array_equal(out2["codes"][:, :, 1:, :], codes[:, :, 1:, :])


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


def pin_fp8_inverse_scale(A, F):
    """The inverse scale is float32(448 / amax) correctly rounded, not
    1 / float32(amax / 448): a block holding amax and an element whose scaled
    value lands on an e4m3 tie under the correct inverse (and off it under
    the other) gets the tie's even code."""
    v = F.e4m3_values()
    rng = np.random.default_rng(16)
    for _ in range(2000):
        amax = float(np.float32(rng.uniform(0.5, 4.0)))
        inv_c = _f32(Fraction(448) / Fraction(amax))
        inv_d = float(np.float32(1) / np.float32(_f32(Fraction(amax) / 448)))
        if inv_c == inv_d:
            continue
        for c in range(0x30, 0x60):
            t = (v[c] + v[c + 1]) / 2                        # a tie between codes c and c+1
            for x in (np.float32(t / inv_c), np.nextafter(np.float32(t / inv_c), np.float32(1)),
                      np.nextafter(np.float32(t / inv_c), np.float32(0))):
                if abs(float(x)) >= amax:
                    continue
                yc = float(np.float32(x) * np.float32(inv_c))
                yd = float(np.float32(x) * np.float32(inv_d))
                if yc == t and _brute_encode(yc) != _brute_encode(yd):
                    blk = np.zeros((1, 1, 1, 2), np.float32)
                    blk[0, 0, 0, 0], blk[0, 0, 0, 1] = amax, x
                    got = F.quantize_heads(blk)["codes"][0, 0, 0, 1]
                    assert int(got) == _brute_encode(yc), ("inverse scale", amax, float(x))
                    return
    raise AssertionError("no distinguishing case found")


ALL_FP8_PINS = [pin_fp8_table, pin_fp8_encode, pin_fp8_quantize, pin_fp8_exact_inputs, pin_fp8_inverse_scale]
