"""Checks that pin the fp64 all-to-all (Ulysses) oracle to things other than
itself.

Each ``pin_*`` function takes the forward oracle module ``A`` and the Ulysses
oracle module ``U`` and raises AssertionError when the Ulysses oracle
disagrees with: the ring oracle's per-rank definition (a different layout
path to the same rows and heads), torch softmax attention in float64 over all
heads (an independent library), pure-Python brute force on a tiny case, the
round trip of the two all-to-alls (every element placed exactly once), or
closed forms.  test_oracle_ulysses.py runs the same functions against
deliberately broken copies of the Ulysses oracle.
"""
from __future__ import annotations

import math

import numpy as np

from tests.oracle_pins import _close, _tiny_docs

CASES = [("none", None), ("causal", None), ("doc_causal", "docs")]


def _shards(seed, N, L, H, d, B=1):
    rng = np.random.default_rng(seed)
    mk = lambda: [rng.standard_normal((B, L, H, d)) for _ in range(N)]  # noqa: E731
    return mk(), mk(), mk()


def _cu(mask, S):
    return _tiny_docs(S) if mask == "doc_causal" else None


def _group(r, N, H):
    """The reading fixed here, independently of the oracle: rank r takes the
    contiguous head group [r H/N, (r+1) H/N)."""
    return range(r * (H // N), (r + 1) * (H // N))


def pin_ulysses_vs_ring(A, U):
    """Piece i of rank r's result = the ring oracle's rows of rank i for the
    heads of r (output and lse), for every r and i."""
    N, L, H, d = 3, 5, 6, 4
    for mask, _ in CASES:
        qs, ks, vs = _shards(7, N, L, H, d, B=2)
        cu = _cu(mask, N * L)
        for r in range(N):
            got = U.ulysses_rank(qs, ks, vs, r, N, mask, cu)
            hs = list(_group(r, N, H))
            assert list(U.heads_of(r, N, H)) == hs, ("head group", r)
            for i in range(N):
                ref = A.rank_attention(qs[i], ks, vs, i, N, mask, cu, heads=hs)
                _close(got["o_parts"][i], ref["o"], rtol=1e-11, atol=1e-12, what=f"o {mask} r{r} i{i}")
                for name in ("m", "l", "lse"):
                    _close(got[name][:, :, i * L:(i + 1) * L], ref[name], rtol=1e-11, atol=1e-12,
                           what=f"{name} {mask} r{r} i{i}")


def _torch_attention(q, k, v, mask, cu):
    """float64 torch softmax attention over [B, S, H, d] with the mask built
    from positions by torch ops."""
    import torch
    Q, K, V = (torch.tensor(x, dtype=torch.float64) for x in (q, k, v))
    S, d = Q.shape[1], Q.shape[3]
    sc = torch.einsum("bshd,bthd->bhst", Q, K) / math.sqrt(d)
    pos = torch.arange(S)
    if mask != "none":
        vis = pos[None, :] <= pos[:, None]
        if mask == "doc_causal":
            doc = torch.zeros(S, dtype=torch.long)
            for k_, start in enumerate(cu[:-1]):
                doc[int(start):int(cu[k_ + 1])] = k_
            vis = vis & (doc[None, :] == doc[:, None])
        sc = sc.masked_fill(~vis[None, None], float("-inf"))
    P = torch.softmax(sc, dim=-1)
    lse = torch.logsumexp(sc, dim=-1)
    return torch.einsum("bhst,bthd->bshd", P, V).numpy(), lse.numpy()


def pin_ulysses_torch(A, U):
    """All ranks' results put back in place = torch attention over all heads."""
    N, L, H, d = 4, 4, 8, 3
    for mask, _ in CASES:
        qs, ks, vs = _shards(13, N, L, H, d)
        cu = _cu(mask, N * L)
        ref_o, ref_lse = _torch_attention(np.concatenate(qs, 1), np.concatenate(ks, 1), np.concatenate(vs, 1),
                                          mask, cu)
        O = np.full((1, N * L, H, d), np.nan)
        LSE = np.full((1, H, N * L), np.nan)
        for r in range(N):
            got = U.ulysses_rank(qs, ks, vs, r, N, mask, cu)
            hs = _group(r, N, H)
            for i in range(N):
                O[:, i * L:(i + 1) * L, hs.start:hs.stop] = got["o_parts"][i]
            LSE[:, hs.start:hs.stop] = got["lse"]
        _close(O, ref_o, rtol=1e-10, atol=1e-12, what=f"o torch {mask}")
        _close(LSE, ref_lse, rtol=1e-10, atol=1e-12, what=f"lse torch {mask}")


def pin_ulysses_brute_force(A, U):
    """Tiny case against pure-Python loops (math.exp, math.fsum)."""
    N, L, H, d = 2, 3, 2, 2
    for mask, _ in CASES[:2]:
        qs, ks, vs = _shards(3, N, L, H, d)
        for r in range(N):
            got = U.ulysses_rank(qs, ks, vs, r, N, mask)
            h = _group(r, N, H).start
            q = np.concatenate(qs, 1)[0, :, h].tolist()
            k = np.concatenate(ks, 1)[0, :, h].tolist()
            v = np.concatenate(vs, 1)[0, :, h].tolist()
            bo, _, _, blse = A.brute_force(q, k, v, list(range(N * L)), list(range(N * L)), mask)
            o_all = np.concatenate([got["o_parts"][i][0, :, 0] for i in range(N)])
            _close(o_all, np.asarray(bo), rtol=1e-12, atol=1e-13, what=f"brute o {mask} r{r}")
            _close(got["lse"][0, 0], np.asarray(blse), rtol=1e-12, atol=1e-13, what=f"brute lse {mask} r{r}")


def pin_ulysses_round_trip(A, U):
    """seq_to_heads then heads_to_seq over all ranks puts every element of
    every shard back where it came from, exactly once."""
    N, L, H, d = 4, 3, 8, 2
    rng = np.random.default_rng(5)
    xs = [rng.standard_normal((2, L, H, d)) for _ in range(N)]
    back = [np.full((2, L, H, d), np.nan) for _ in range(N)]
    count = [np.zeros((2, L, H, d), int) for _ in range(N)]
    for r in range(N):
        full = U.seq_to_heads(xs, r, N)
        assert full.shape == (2, N * L, H // N, d)
        hs = _group(r, N, H)
        for i, piece in enumerate(U.heads_to_seq(full, N)):
            back[i][:, :, hs.start:hs.stop] = piece
            count[i][:, :, hs.start:hs.stop] += 1
    for i in range(N):
        assert np.all(count[i] == 1), f"shard {i}: elements not placed exactly once"
        assert np.array_equal(back[i], xs[i]), f"shard {i}: round trip changed values"


def pin_ulysses_closed_forms(A, U):
    """Identical V rows: every output row is that row.  N = 1: plain attention
    of the single shard.  H not a multiple of N is refused."""
    N, L, H, d = 2, 4, 4, 3
    qs, ks, vs = _shards(21, N, L, H, d)
    row = np.arange(1.0, d + 1.0)
    vc = [np.broadcast_to(row, x.shape).copy() for x in vs]
    for mask in ("none", "causal"):
        for r in range(N):
            got = U.ulysses_rank(qs, ks, vc, r, N, mask)
            for i in range(N):
                _close(got["o_parts"][i], np.broadcast_to(row, got["o_parts"][i].shape), rtol=1e-13, atol=1e-13,
                       what=f"const V {mask} r{r} i{i}")
    got = U.ulysses_rank(qs[:1], ks[:1], vs[:1], 0, 1, "causal")
    ref = A.rank_attention(qs[0], ks[:1], vs[:1], 0, 1, "causal")
    _close(got["o_parts"][0], ref["o"], rtol=1e-12, atol=1e-13, what="N=1")
    try:
        U.heads_of(0, 3, 4)
    except ValueError:
        pass
    else:
        raise AssertionError("H=4, N=3 accepted")


ALL_ULYSSES_PINS = [pin_ulysses_vs_ring, pin_ulysses_torch, pin_ulysses_brute_force, pin_ulysses_round_trip,
                    pin_ulysses_closed_forms]
