"""Checks that pin the fp64 oracle to things other than itself.

Each ``pin_*`` function takes the oracle module and raises AssertionError when
the oracle disagrees with: pure-Python brute force, torch's CPU
scaled_dot_product_attention in float64 (an independent library routine),
closed forms, hand-derived values, or the pages' printed stage table and
causal block needs (fixtures under tests/golden/).  The same functions are run
against deliberately broken copies of the oracle (test_oracle_mutations.py) to
show that a plausible mistake fails at least one of them.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

from harness.inputs import ShardSpec, make_inputs, normal_block

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    same_inf = (np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b)))
    fa, fb = np.where(same_inf, 0.0, a), np.where(same_inf, 0.0, b)
    assert np.all(np.isfinite(fa)) and np.all(np.isfinite(fb)), (what, "non-finite mismatch")
    err = np.abs(fa - fb) - (atol + rtol * np.abs(fb))
    assert np.all(err <= 0), (what, float(np.max(np.abs(fa - fb))))


def _tiny_docs(S):
    """Hand-built boundaries with one document straddling every shard edge."""
    pts = [0]
    x = 0
    for n in (5, 9, 3, 13, 7, 2, 11, 6, 17, 4):
        x += n
        if x >= S:
            break
        pts.append(x)
    pts.append(S)
    return np.asarray(pts, np.int32)


def _full_kv(inp, N, b, h):
    K = np.concatenate([inp["k"][j][b, :, h, :] for j in range(N)]).astype(np.float64)
    V = np.concatenate([inp["v"][j][b, :, h, :] for j in range(N)]).astype(np.float64)
    return K, V


# ----------------------------------------------------------------------------

def pin_brute_force(A):
    """Definition vs pure-Python loops on every rank of tiny rings."""
    case = 0
    for N, H, d, mask in itertools.product((1, 2, 4), (1, 2), (2, 4, 8),
                                           ("none", "causal", "doc_causal")):
        S = 16 * N if N < 4 else 48
        case += 1
        cu = _tiny_docs(S) if mask == "doc_causal" else None
        spec = ShardSpec(S=S, N=N, H=H, d=d, dtype="f32", mask=mask, cfg_id=1000 + case,
                         cu_seqlens=cu)
        inp = make_inputs(spec, seed=7, ranks=range(N))
        L = spec.L
        for r in range(N):
            got = A.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, mask, cu)
            for h in range(H):
                K, V = _full_kv(inp, N, 0, h)
                o, m, l, lse = A.brute_force(inp["q"][r][0, :, h, :].astype(np.float64).tolist(),
                                             K.tolist(), V.tolist(),
                                             list(range(r * L, (r + 1) * L)), list(range(S)),
                                             mask, cu)
                _close(got["o"][0, :, h, :], o, what=("o", N, H, d, mask, r))
                _close(got["m"][0, h], m, what=("m", N, H, d, mask, r))
                _close(got["l"][0, h], l, what=("l", N, H, d, mask, r))
                _close(got["lse"][0, h], lse, what=("lse", N, H, d, mask, r))


def pin_golden_two_keys(A):
    g = _load("two_key_softmax.json")
    o, m, l, lse = A.attention_rows(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]),
                                    np.array(g["p"]), np.array(g["c"]), g["mask"])
    _close(o, g["expect"]["o"], what="o")
    _close(m, g["expect"]["m"], what="m")
    _close(l, g["expect"]["l"], what="l")
    _close(lse, g["expect"]["lse"], what="lse")


def pin_sdpa(A):
    """All ranks together = full-sequence attention from torch's own routine
    (float64, CPU).  N=1 is textbook attention; doc_causal equals causal
    attention run separately on each document."""
    import torch
    import torch.nn.functional as F
    for N, mask in itertools.product((1, 3), ("none", "causal", "doc_causal")):
        S, H, d = 96 if N == 3 else 40, 3, 16
        cu = np.asarray([0, 7, 29, 30, 61, S] if S == 96 else [0, 13, 14, 27, S], np.int32)
        cu = cu if mask == "doc_causal" else None
        spec = ShardSpec(S=S, N=N, H=H, d=d, dtype="f32", mask=mask, cfg_id=2000 + N,
                         cu_seqlens=cu)
        inp = make_inputs(spec, seed=3, ranks=range(N))
        got = np.concatenate([A.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, mask,
                                               cu)["o"] for r in range(N)], axis=1)
        Q = torch.from_numpy(np.concatenate([inp["q"][r] for r in range(N)], axis=1)
                             .astype(np.float64)).permute(0, 2, 1, 3).contiguous()
        K = torch.from_numpy(np.concatenate([inp["k"][j] for j in range(N)], axis=1)
                             .astype(np.float64)).permute(0, 2, 1, 3).contiguous()
        V = torch.from_numpy(np.concatenate([inp["v"][j] for j in range(N)], axis=1)
                             .astype(np.float64)).permute(0, 2, 1, 3).contiguous()
        if mask == "doc_causal":
            parts = []
            for a, b in zip(cu[:-1], cu[1:]):
                parts.append(F.scaled_dot_product_attention(Q[:, :, a:b], K[:, :, a:b],
                                                            V[:, :, a:b], is_causal=True))
            ref = torch.cat(parts, dim=2)
        else:
            ref = F.scaled_dot_product_attention(Q, K, V, is_causal=(mask == "causal"))
        _close(got, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-12, what=("sdpa", N, mask))


def pin_streaming(A):
    """The streaming numerator/denominator form equals the definition."""
    for mask in ("none", "causal", "doc_causal"):
        S, N, H, d = 64, 4, 2, 32
        cu = _tiny_docs(S) if mask == "doc_causal" else None
        spec = ShardSpec(S=S, N=N, H=H, d=d, dtype="f32", mask=mask, cfg_id=3000, cu_seqlens=cu)
        inp = make_inputs(spec, seed=5, ranks=range(N))
        L = spec.L
        for r in range(N):
            ref = A.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, mask, cu)["o"]
            for h in range(H):
                got = A.streaming_attention(inp["q"][r][0, :, h, :],
                                            [inp["k"][j][0, :, h, :] for j in range(N)],
                                            [inp["v"][j][0, :, h, :] for j in range(N)],
                                            np.arange(r * L, (r + 1) * L),
                                            [np.arange(j * L, (j + 1) * L) for j in range(N)],
                                            mask, cu)
                _close(got, ref[0, :, h, :], what=("stream", mask, r, h))


def pin_online_orders(A):
    """The online recurrence gives the definition's O, m, l in every order."""
    S, N, H, d = 64, 4, 1, 16
    for mask in ("none", "causal", "doc_causal"):
        cu = _tiny_docs(S) if mask == "doc_causal" else None
        spec = ShardSpec(S=S, N=N, H=H, d=d, dtype="f32", mask=mask, cfg_id=4000, cu_seqlens=cu)
        inp = make_inputs(spec, seed=11, ranks=range(N))
        L = spec.L
        for r in range(N):
            ref = A.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, mask, cu)
            for order in itertools.permutations(range(N)):
                o, m, l = A.online_merge(inp["q"][r][0, :, 0, :],
                                         [inp["k"][j][0, :, 0, :] for j in range(N)],
                                         [inp["v"][j][0, :, 0, :] for j in range(N)],
                                         np.arange(r * L, (r + 1) * L),
                                         [np.arange(j * L, (j + 1) * L) for j in range(N)],
                                         order, mask, cu)
                _close(o, ref["o"][0, :, 0, :], what=("online o", mask, r, order))
                _close(m, ref["m"][0, 0], what=("online m", mask, r, order))
                _close(l, ref["l"][0, 0], what=("online l", mask, r, order))


def pin_merge_lse(A):
    """Per-block normalised partials merged in shuffled orders give the
    definition's O and lse (8 blocks, peaked rows from Q x 3)."""
    S, N, H, d = 128, 8, 2, 16
    rng = np.random.default_rng(1)
    for mask in ("none", "causal", "doc_causal"):
        cu = _tiny_docs(S) if mask == "doc_causal" else None
        spec = ShardSpec(S=S, N=N, H=H, d=d, dtype="f32", mask=mask, cfg_id=5000, q_scale=3.0,
                         cu_seqlens=cu)
        r = 5
        inp = make_inputs(spec, seed=13, ranks=[r])
        ref = A.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, mask, cu)
        parts = [A.block_partial(inp["q"][r], inp["k"][j], inp["v"][j], r, j, N, mask, cu)
                 for j in range(N)]
        for _ in range(16):
            order = list(rng.permutation(N))
            o_parts = [pp["o"].transpose(0, 2, 1, 3) for pp in parts]   # [B,H,L,d]
            lse_parts = [pp["lse"] for pp in parts]                      # [B,H,L]
            o, lse = A.merge_lse(o_parts, lse_parts, order)
            _close(o.transpose(0, 2, 1, 3), ref["o"], what=("merge o", mask))
            _close(lse, ref["lse"], what=("merge lse", mask))


def pin_independence(A):
    """Rank i's result does not depend on blocks j > i (causal), nor on keys of
    other documents (doc_causal): replaced by fresh draws, the outputs are
    bit-identical."""
    S, N, H, d = 64, 4, 2, 8
    spec = ShardSpec(S=S, N=N, H=H, d=d, dtype="f32", mask="causal", cfg_id=6000)
    inp = make_inputs(spec, seed=17, ranks=range(N))
    for r in range(N):
        ref = A.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, "causal")
        k2 = dict(inp["k"])
        v2 = dict(inp["v"])
        for j in range(r + 1, N):
            k2[j] = normal_block(99, 6000, 1, j, spec.shard_shape())
            v2[j] = normal_block(99, 6000, 2, j, spec.shard_shape())
        got = A.rank_attention(inp["q"][r], k2, v2, r, N, "causal")
        for key in ("o", "m", "l", "lse"):
            assert np.array_equal(got[key], ref[key]), ("causal independence", r, key)
    cu = _tiny_docs(S)
    spec = ShardSpec(S=S, N=N, H=H, d=d, dtype="f32", mask="doc_causal", cfg_id=6001,
                     cu_seqlens=cu)
    inp = make_inputs(spec, seed=19, ranks=range(N))
    L = spec.L
    for r in range(N):
        ref = A.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, "doc_causal", cu)
        rows = np.arange(r * L, (r + 1) * L)
        docs_here = set(np.searchsorted(cu, rows, side="right") - 1)
        k2 = {j: inp["k"][j].copy() for j in range(N)}
        v2 = {j: inp["v"][j].copy() for j in range(N)}
        for j in range(N):
            keys = np.arange(j * L, (j + 1) * L)
            other = np.array([x not in docs_here for x in np.searchsorted(cu, keys, side="right") - 1])
            k2[j][:, other] = 1e3
            v2[j][:, other] = -1e3
        got = A.rank_attention(inp["q"][r], k2, v2, r, N, "doc_causal", cu)
        for key in ("o", "m", "l", "lse"):
            assert np.array_equal(got[key], ref[key]), ("doc independence", r, key)


def pin_rows_sum_to_one(A):
    """sum over visible keys of exp(s - lse) = 1, with s recomputed here."""
    S, N, H, d = 96, 3, 2, 16
    for mask in ("none", "causal", "doc_causal"):
        cu = _tiny_docs(S) if mask == "doc_causal" else None
        spec = ShardSpec(S=S, N=N, H=H, d=d, dtype="f32", mask=mask, cfg_id=7000, cu_seqlens=cu)
        inp = make_inputs(spec, seed=23, ranks=range(N))
        L = spec.L
        for r in range(N):
            got = A.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, mask, cu)
            for h in range(H):
                K, _ = _full_kv(inp, N, 0, h)
                q = inp["q"][r][0, :, h, :].astype(np.float64)
                for n in range(L):
                    p = r * L + n
                    if mask == "none":
                        keys = range(S)
                    elif mask == "causal":
                        keys = range(p + 1)
                    else:
                        start = max(int(x) for x in cu if x <= p)
                        keys = range(start, p + 1)
                    tot = math.fsum(math.exp(float(q[n] @ K[c]) / math.sqrt(d) - got["lse"][0, h, n])
                                    for c in keys)
                    assert abs(tot - 1.0) < 1e-12, (mask, r, h, n, tot)


def pin_closed_forms(A):
    """V = 1 gives O = 1; Q = 0 gives the mean of the visible V and
    lse = ln(#visible); rank 0 causal row 0 sees only key 0."""
    S, N, H, d = 64, 4, 2, 8
    cu = _tiny_docs(S)
    for mask in ("none", "causal", "doc_causal"):
        c = cu if mask == "doc_causal" else None
        spec = ShardSpec(S=S, N=N, H=H, d=d, dtype="f32", mask=mask, cfg_id=8000, cu_seqlens=c)
        inp = make_inputs(spec, seed=29, ranks=range(N))
        L = spec.L
        ones = {j: np.ones_like(inp["v"][j]) for j in range(N)}
        for r in range(N):
            got = A.rank_attention(inp["q"][r], inp["k"], ones, r, N, mask, c)
            _close(got["o"], np.ones_like(got["o"]), what=("V=1", mask, r))
            zq = np.zeros_like(inp["q"][r])
            got = A.rank_attention(zq, inp["k"], inp["v"], r, N, mask, c)
            for h in range(H):
                _, V = _full_kv(inp, N, 0, h)
                for n in range(L):
                    p = r * L + n
                    if mask == "none":
                        lo, hi = 0, S - 1
                    elif mask == "causal":
                        lo, hi = 0, p
                    else:
                        lo, hi = max(int(x) for x in cu if x <= p), p
                    cnt = hi - lo + 1
                    _close(got["o"][0, n, h], V[lo:hi + 1].mean(axis=0), what=("Q=0 mean", mask))
                    _close(got["lse"][0, h, n], math.log(cnt), what=("Q=0 lse", mask))
                    _close(got["m"][0, h, n], 0.0, what=("Q=0 m", mask))
                    _close(got["l"][0, h, n], float(cnt), what=("Q=0 l", mask))
    spec = ShardSpec(S=S, N=N, H=H, d=d, dtype="f32", mask="causal", cfg_id=8001)
    inp = make_inputs(spec, seed=31, ranks=[0])
    got = A.rank_attention(inp["q"][0], inp["k"], inp["v"], 0, N, "causal")
    for h in range(H):
        q0 = inp["q"][0][0, 0, h].astype(np.float64)
        k0 = inp["k"][0][0, 0, h].astype(np.float64)
        _close(got["o"][0, 0, h], inp["v"][0][0, 0, h], what="row0 o")
        _close(got["m"][0, h, 0], float(q0 @ k0) / math.sqrt(d), what="row0 m")
        _close(got["l"][0, h, 0], 1.0, what="row0 l")


def pin_schedule(A):
    """Ring order and mask-aware skipping against the pages' stage table and
    causal block needs; doc skipping against pair enumeration."""
    g = _load("ring_stage_table_gpu0.json")
    L = g["S"] // g["N"]
    order = A.ring_schedule(g["N"], g["rank"], L, "none", direction="reverse")
    assert [[j * L, (j + 1) * L] for j in order] == [s["kv"] for s in g["stages"]], order
    # forward: receive from the previous rank, so block (rank - t) mod N at step t
    for N in (2, 4, 8):
        for r in range(N):
            assert A.ring_schedule(N, r, 16, "none") == [(r - t) % N for t in range(N)]
    for case in _load("causal_block_needs.json")["cases"]:
        N = case["N"]
        for r in range(N):
            got = A.ring_schedule(N, r, 8, "causal")
            assert sorted(got) == case["needs"][r], (N, r, got)
            assert got[0] == r   # the local block first
    S, N = 96, 4
    cu = np.asarray([0, 10, 20, 47, 48, 51, 72, 90, 96], np.int32)
    L = S // N
    for r in range(N):
        p = np.arange(r * L, (r + 1) * L)
        want = []
        for j in range(N):
            c = np.arange(j * L, (j + 1) * L)
            lo = [max(int(x) for x in cu if x <= pp) for pp in p]
            if any(lo[a] <= cc <= p[a] for a in range(L) for cc in c):
                want.append(j)
        got = A.ring_schedule(N, r, L, "doc_causal", cu)
        assert sorted(got) == want, (r, got, want)


def pin_visible_pairs(A):
    """Visible-pair counts equal a count of the materialised boolean mask, and
    the causal count of rank i is i L^2 + L(L+1)/2."""
    for mask in ("none", "causal", "doc_causal"):
        S, N = 96, 4
        cu = np.asarray([0, 10, 20, 47, 48, 51, 72, 90, 96], np.int32)
        L = S // N
        for r in range(N):
            p = np.arange(r * L, (r + 1) * L)
            cnt = 0
            for pp in p:
                for cc in range(S):
                    if mask == "none":
                        cnt += 1
                    elif mask == "causal":
                        cnt += cc <= pp
                    else:
                        cnt += (max(int(x) for x in cu if x <= pp) <= cc <= pp)
            assert A.visible_pairs(N, L, r, mask, cu) == cnt, (mask, r)
    for N, L in ((4, 8192), (4, 32768), (8, 16384)):
        for r in range(N):
            assert A.visible_pairs(N, L, r, "causal") == r * L * L + L * (L + 1) // 2


def pin_ring_traffic(A):
    """2 (G/N)(N-1) against a step-by-step count of a simulated ring exchange:
    every rank forwards the K/V block it holds to the next rank, N-1 times."""
    for N, S, H, d, eb in ((4, 131072, 32, 128, 2), (8, 65536, 16, 128, 2), (3, 96, 2, 8, 4)):
        L = S // N
        block_bytes = 2 * L * H * d * eb            # one K block and one V block
        holding = list(range(N))
        sent = [0] * N
        recv = [0] * N
        for _ in range(N - 1):
            for r in range(N):
                sent[r] += block_bytes
                recv[(r + 1) % N] += block_bytes
            holding = [holding[(r - 1) % N] for r in range(N)]
        assert sorted(holding) == list(range(N))
        for r in range(N):
            assert sent[r] + recv[r] == A.ring_traffic_bytes(S, H, d, eb, N), (N, r)


ALL_PINS = [pin_brute_force, pin_golden_two_keys, pin_sdpa, pin_streaming, pin_online_orders,
            pin_merge_lse, pin_independence, pin_rows_sum_to_one, pin_closed_forms,
            pin_schedule, pin_visible_pairs, pin_ring_traffic]
