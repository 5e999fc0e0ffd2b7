"""Helpers of the GPU parity tests: device transfer of seeded inputs, calls
through the C ABI binding, and the tolerance checks.

Tolerances (stated here, applied by every parity test):
  fp32 inputs: O max-abs <= 1e-4; m and lse max-abs <= 1e-4; l relative <= 1e-5.
  bf16 inputs: O max-abs <= 1.5e-2 and mean-abs <= 1e-3; m and lse max-abs
               <= 2e-3; l relative <= 1e-3.
The O bounds are the ones required for the path; the m/l/lse bounds are this
project's reading (the statement gives none): fp32 accumulation of at most
~1e5 terms keeps l within ~1e-5 relative in practice, and bf16 only enters
through the inputs (the oracle sees the same bf16-rounded values) and through
P rounded to bf16 before the PV product, which does not touch l.
"""
from __future__ import annotations

import sys

import numpy as np

from harness.inputs import bf16_bits, round_to_bf16

TOL = {
    "f32": dict(o_max=1e-4, o_mean=1e-4, ml_abs=1e-4, l_rel=1e-5),
    "bf16": dict(o_max=1.5e-2, o_mean=1e-3, ml_abs=2e-3, l_rel=1e-3),
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        bits = np.ascontiguousarray(bf16_bits(x)).view(np.int16)
        return torch.from_numpy(bits).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_o(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "o",
            rounding_floor: bool = False) -> dict:
    """O within the tolerance.  rounding_floor: add the mean error of the
    oracle's own values rounded to bf16 to the mean-abs bound - for outputs
    made of one or two V rows (a one-token shard), where the bf16 output
    format alone costs about 1e-3 and no kernel can do better."""
    t = TOL[dtype]
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    bound = t["o_mean"]
    if rounding_floor and dtype == "bf16":
        bound += float(np.mean(np.abs(round_to_bf16(ref.astype(np.float32)).astype(np.float64) - ref)))
    assert mx <= t["o_max"], f"{what}: max-abs {mx:.3e} > {t['o_max']}"
    assert mean <= bound, f"{what}: mean-abs {mean:.3e} > {bound:.3e}"
    return {"max_abs": mx, "mean_abs": mean}


def check_stat(got: np.ndarray, ref: np.ndarray, dtype: str, kind: str) -> float:
    t = TOL[dtype]
    assert got.shape == ref.shape, (kind, got.shape, ref.shape)
    ninf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf_ref), f"{kind}: -inf pattern differs"
    g, r = got[~ninf_ref], ref[~ninf_ref]
    assert np.all(np.isfinite(g)), f"{kind}: non-finite"
    if g.size == 0:
        return 0.0
    if kind == "l":
        err = float(np.max(np.abs(g - r) / np.maximum(np.abs(r), 1e-30)))
        assert err <= t["l_rel"], f"l: relative {err:.3e} > {t['l_rel']}"
    else:
        err = float(np.max(np.abs(g - r)))
        assert err <= t["ml_abs"], f"{kind}: max-abs {err:.3e} > {t['ml_abs']}"
    return err


def sample_rows(L: int, seed: int, n_random: int = 192, extra=()) -> np.ndarray:
    """Rows at the shard edges, at 64/128-row tile edges, given extras
    (document boundaries) and a seeded random set."""
    rng = np.random.default_rng(seed)
    rows = {0, 1, 2, L // 2 - 1, L // 2, L - 2, L - 1}
    for t in (64, 128, 256):
        for k in rng.choice(max(1, L // t), size=min(8, max(1, L // t)), replace=False):
            rows.update({int(k) * t, int(k) * t - 1})
    rows.update(int(x) for x in extra)
    rows.update(int(x) for x in rng.choice(L, size=min(n_random, L), replace=False))
    return np.asarray(sorted(r for r in rows if 0 <= r < L), dtype=np.int64)


def oracle_workers() -> int:
    """Threads for running oracle calls side by side: the host's cores, at
    most 16 (each call then uses one BLAS thread)."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def pooled_map(fn, items, workers: int = 0):
    """``[fn(x) for x in items]`` on a thread pool, one BLAS thread per call.
    numpy's matrix products and ufuncs release the GIL, so the calls run in
    parallel; each call is the unchanged oracle function on its own part."""
    import concurrent.futures as cf

    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        with cf.ThreadPoolExecutor(workers or oracle_workers()) as ex:
            return list(ex.map(fn, items))


def pooled_rows(fn, n_rows: int, chunk: int = 256, workers: int = 0):
    """``fn(rows)`` over consecutive row chunks [r0, r0 + chunk) of
    range(n_rows) (see pooled_map), results in row order."""
    chunks = [np.arange(r0, min(r0 + chunk, n_rows), dtype=np.int64) for r0 in range(0, n_rows, chunk)]
    return pooled_map(fn, chunks, workers)


def pooled_reduce(fn, n_rows: int, chunk: int = 256, workers: int = 0):
    """Like pooled_rows, but each worker thread takes a contiguous share of
    the chunks and folds the results of its chunks with ``fn(rows, acc) ->
    acc`` (acc is None for a worker's first chunk); returns the list of the
    workers' accumulators, in row order of their shares."""
    import concurrent.futures as cf

    from threadpoolctl import threadpool_limits
    nw = workers or oracle_workers()
    starts = list(range(0, n_rows, chunk))
    shares = [starts[len(starts) * w // nw: len(starts) * (w + 1) // nw] for w in range(nw)]

    def run(share):
        acc = None
        for r0 in share:
            acc = fn(np.arange(r0, min(r0 + chunk, n_rows), dtype=np.int64), acc)
        return acc

    with threadpool_limits(1):
        with cf.ThreadPoolExecutor(nw) as ex:
            return [a for a in ex.map(run, shares) if a is not None]
