"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one: a dropped scale, a wrong operand, a sign error, an
off-by-one in a mask, a missing rescale, a reversed ring direction."""
import inspect
import textwrap

import pytest

import oracle.attention as A
from tests.oracle_pins import ALL_PINS

MUTATIONS = [
    ("attention_rows", "s = (q @ k.T) * scale", "s = (q @ k.T)"),
    ("attention_rows", "num = e @ v", "num = e @ k"),
    ("attention_rows", "m_safe + np.log(", "m_safe - np.log("),
    ("attention_rows", "l = e.sum(axis=1)", "l = e.sum(axis=1) + 1e-9"),
    ("visibility", "return C <= P", "return C < P"),
    ("visibility", "(C >= lo)", "(C > lo)"),
    ("doc_start", 'side="right"', 'side="left"'),
    ("rank_attention", "rank * L + rr", "rr"),
    ("block_partial", "c = j * L + np.arange", "c = rank * L + np.arange"),
    ("_combine", "oa * wa[:, None] + ob * wb[:, None]", "oa + ob * wb[:, None]"),
    ("_combine", "la * wa + lb * wb", "la + lb * wb"),
    ("_block_state", "E.sum(axis=1)", "E.sum(axis=1) + 1e-9"),
    ("merge_lse", "w = _exp_shift(np.asarray(lse_parts[j], np.float64), lse)",
     "w = _exp_shift(lse, np.asarray(lse_parts[j], np.float64))"),
    ("streaming_attention", "/ w.sum(axis=1)[:, None]", "/ w.sum(axis=0).mean()"),
    ("ring_schedule", "step = -1 if direction", "step = 1 if direction"),
    ("block_visible", "hi = np.minimum(p, (j + 1) * L - 1)", "hi = np.minimum(p, (j + 1) * L)"),
    ("visible_pairs", "np.sum(p - first + 1)", "np.sum(p - first)"),
    ("ring_traffic_bytes", "2 * (G // N) * (N - 1)", "2 * (G // N) * N"),
]


@pytest.mark.parametrize("fname,old,new", MUTATIONS, ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_mutation_is_caught(monkeypatch, fname, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(A, fname)))
    assert old in src, "mutation target text not found"
    scope = {}
    exec(compile(src.replace(old, new), f"<mutant {fname}>", "exec"), A.__dict__, scope)
    monkeypatch.setattr(A, fname, scope[fname])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(A)
        except Exception as e:  # noqa: BLE001 - any failure counts as detection
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"no pin caught mutation in {fname}: {old!r} -> {new!r}"
