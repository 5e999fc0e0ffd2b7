"""The FP8 (e4m3) oracle against the format's properties, an exact
brute-force round-to-nearest-even, the quantisation's defining properties
and the plain definition on exactly representable inputs
(tests/oracle_fp8_pins.py); and planted mistakes the pins must catch: a
wrong exponent bias, ties rounded away from even, a lost sign of zero, a
scale exponent for the largest value 240 (the fnuz variant), a boundary
compared the wrong way, the clamp at -126 lost, a zero block given a
nonzero exponent, a wrong log2(e) or sqrt, one scale for all
heads, the query's c ignored or applied without the float32 rounding, codes
off by a factor of two, and a dequantisation that multiplies where it
divides."""
import inspect
import textwrap

import pytest

import oracle.attention as A
import oracle.fp8 as F
from tests.oracle_fp8_pins import ALL_FP8_PINS


@pytest.mark.parametrize("pin", ALL_FP8_PINS, ids=[p.__name__ for p in ALL_FP8_PINS])
def test_fp8_pin(pin):
    pin(A, F)


MUTATIONS = [
    ("e4m3_values", "(1.0 + m / 8.0) * 2.0 ** (e - 7)", "(1.0 + m / 8.0) * 2.0 ** (e - 8)"),
    ("e4m3_encode", "((d_hi == d_lo) & (hi % 2 == 0))", "((d_hi == d_lo))"),
    ("e4m3_encode", "return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)",
     "return (code | np.where(np.signbit(x) & (code != 0), 0x80, 0)).astype(np.uint8)"),
    ("scale_exponent", "while v > E4M3_MAX * 2.0 ** e:", "while v > 240.0 * 2.0 ** e:"),
    ("scale_exponent", "while v > E4M3_MAX * 2.0 ** e:", "while v >= E4M3_MAX * 2.0 ** e:"),
    ("scale_exponent", "e = -126", "e = -127"),
    ("scale_exponent", "if v > 0:", "if v >= 0:"),
    ("query_prescale", "np.float32(LOG2E)", "np.float32(1.4427)"),
    ("query_prescale", "np.float32(1) / np.sqrt(np.float32(d))", "np.float32(1) / np.float32(np.sqrt(float(d)) * 1.0000001)"),
    ("quantize_heads", "amax = np.abs(y).max(axis=(1, 3))", "amax = np.abs(y).max(axis=(1, 3)) * 0 + np.abs(y).max()"),
    ("quantize_heads", "y = (x * np.float32(prescale)).astype(np.float32)", "y = x.astype(np.float32)"),
    ("quantize_heads", "y = (x * np.float32(prescale)).astype(np.float32)",
     "y = (x.astype(np.float64) * float(np.float32(prescale)))"),
    ("quantize_heads", "np.exp2(-e.astype(np.float64))", "np.exp2(-e.astype(np.float64) - 1)"),
    ("dequantize_heads", "e4m3_decode(codes) * np.asarray(scale", "e4m3_decode(codes) / np.asarray(scale"),
    ("dequantize_heads", "/ float(prescale)", "* float(prescale)"),
]


def _apply(monkeypatch, fname, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(F, fname)))
    assert old in src, "mutation target text not found"
    scope = {}
    exec(compile(src.replace(old, new), f"<mutant {fname}>", "exec"), F.__dict__, scope)
    monkeypatch.setattr(F, fname, scope[fname])
    if fname == "e4m3_values":          # the module's tables are built from it
        monkeypatch.setattr(F, "_VALUES", scope[fname]())
        monkeypatch.setattr(F, "_POS", F._VALUES[:0x7F])


@pytest.mark.parametrize("fname,old,new", MUTATIONS, ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_fp8_mutation_is_caught(monkeypatch, fname, old, new):
    _apply(monkeypatch, fname, old, new)
    caught = False
    for pin in ALL_FP8_PINS:
        try:
            pin(A, F)
        except Exception:  # noqa: BLE001 - any failure counts as detection
            caught = True
            break
    assert caught, f"no pin caught mutation in {fname}: {old!r} -> {new!r}"
