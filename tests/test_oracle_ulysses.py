"""The fp64 all-to-all (Ulysses) oracle against the ring oracle, torch,
brute force, the all-to-all round trip and closed forms
(tests/oracle_ulysses_pins.py), and planted mistakes that the pins must
catch: a shifted head group, shards in the wrong order, pieces sent to the
wrong rank, positions off by a shard, a base-2 lse."""
import inspect
import textwrap

import pytest

import oracle.attention as A
import oracle.ulysses as U
from tests.oracle_ulysses_pins import ALL_ULYSSES_PINS


@pytest.mark.parametrize("pin", ALL_ULYSSES_PINS, ids=[p.__name__ for p in ALL_ULYSSES_PINS])
def test_ulysses_pin(pin):
    pin(A, U)


MUTATIONS = [
    ("heads_of", "return range(rank * hn, (rank + 1) * hn)", "return range((rank * hn + 1) % (N * hn - hn + 1), (rank * hn + 1) % (N * hn - hn + 1) + hn)"),
    ("heads_of", "return range(rank * hn, (rank + 1) * hn)", "return range((N - 1 - rank) * hn, (N - rank) * hn)"),
    ("seq_to_heads", "for x in shards], axis=1)", "for x in shards[::-1]], axis=1)"),
    ("seq_to_heads", "x)[:, :, hs.start:hs.stop, :]", "x)[:, :, hs.start:hs.stop, :][:, ::-1]"),
    ("heads_to_seq", "return [full[:, i * L:(i + 1) * L] for i in range(N)]",
     "return [full[:, i * L:(i + 1) * L] for i in reversed(range(N))]"),
    ("ulysses_rank", "pos = np.arange(S, dtype=np.int64)", "pos = np.arange(S, dtype=np.int64) + 1"),
    ("ulysses_rank", "LSE[b, h] = lse", "LSE[b, h] = lse * 1.4426950408889634"),
    ("ulysses_rank", "M[b, h] = m", "M[b, h] = lse"),
]


@pytest.mark.parametrize("fname,old,new", MUTATIONS, ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_ulysses_mutation_is_caught(monkeypatch, fname, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(U, fname)))
    assert old in src, "mutation target text not found"
    scope = {}
    exec(compile(src.replace(old, new), f"<mutant {fname}>", "exec"), U.__dict__, scope)
    monkeypatch.setattr(U, fname, scope[fname])
    caught = False
    for pin in ALL_ULYSSES_PINS:
        try:
            pin(A, U)
        except Exception:  # noqa: BLE001 - any failure counts as detection
            caught = True
            break
    assert caught, f"no pin caught mutation in {fname}: {old!r} -> {new!r}"
