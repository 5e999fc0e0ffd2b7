"""Plant plausible mistakes in the backward oracle (on the CPU) and check that
the pins catch each one: a dropped correction term, a dropped or extra scale,
a sign error, a wrong shift, a wrong layout, wrong positions."""
import inspect
import textwrap

import pytest

import oracle.attention as A
import oracle.backward as G
from tests.oracle_bwd_pins import ALL_BWD_PINS

MUTATIONS = [
    ("attention_grad_rows", "dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))", "dS = P * dP"),
    ("attention_grad_rows", "dq = (dS @ k) * scale", "dq = (dS @ k)"),
    ("attention_grad_rows", "dk = (dS.T @ q) * scale", "dk = (dS.T @ q) * scale * scale"),
    ("attention_grad_rows", "dv = P.T @ do", "dv = e.T @ do"),
    ("attention_grad_rows", "s = (q @ k.T) * scale", "s = (q @ k.T)"),
    ("bwd_delta", '"blhd,blhd->bhl"', '"blhd,blhd->blh"'),
    ("block_backward", "dO @ V.T - np.asarray(delta", "dO @ V.T + np.asarray(delta"),
    ("block_backward", "shifted = s - np.where", "shifted = s + np.where"),
    ("block_backward", 'out["dk"][b, :, h, :] = (dS.T @ Q) * scale', 'out["dk"][b, :, h, :] = (dS.T @ Q)'),
    ("block_backward", 'out["dv"][b, :, h, :] = P.T @ dO', 'out["dv"][b, :, h, :] = P.T @ dO * scale'),
    ("block_backward", "c = j * L + np.arange", "c = rank * L + np.arange"),
    ("rank_backward", "p = rank * L + np.arange", "p = np.arange"),
]


@pytest.mark.parametrize("fname,old,new", MUTATIONS, ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_bwd_mutation_is_caught(monkeypatch, fname, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(G, fname)))
    assert old in src, "mutation target text not found"
    scope = {}
    exec(compile(src.replace(old, new), f"<mutant {fname}>", "exec"), G.__dict__, scope)
    monkeypatch.setattr(G, fname, scope[fname])
    caught = False
    for pin in ALL_BWD_PINS:
        try:
            pin(A, G)
        except Exception:  # noqa: BLE001 - any failure counts as detection
            caught = True
            break
    assert caught, f"no pin caught mutation in {fname}: {old!r} -> {new!r}"
