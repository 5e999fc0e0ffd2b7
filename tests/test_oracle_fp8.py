"""The FP8 (e4m3) oracle against the format's properties, an exact
brute-force round-to-nearest-even, the quantisation's defining properties
and the plain definition on exactly representable inputs
(tests/oracle_fp8_pins.py); and planted mistakes the pins must catch: a
wrong exponent bias, ties rounded away from even, a wrong scale constant,
one scale for all heads, a double-rounded inverse scale, a missing clamp."""
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
    ("quantize_heads", "safe / np.float32(E4M3_MAX)", "safe / np.float32(256.0)"),
    ("quantize_heads", "amax = np.abs(x).max(axis=(1, 3))", "amax = np.abs(x).max(axis=(1, 3)) * 0 + np.abs(x).max()"),
    ("quantize_heads", "inv = np.where(zero, np.float32(1), np.float32(E4M3_MAX) / safe).astype(np.float32)",
     "inv = np.where(zero, np.float32(1), np.float32(1) / scale).astype(np.float32)"),
    ("quantize_heads", "y = np.clip(y, -E4M3_MAX, E4M3_MAX)", "y = y * np.float32(1.001)"),
    ("dequantize_heads", "e4m3_decode(codes) * np.asarray(scale", "e4m3_decode(codes) / np.asarray(scale"),
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
