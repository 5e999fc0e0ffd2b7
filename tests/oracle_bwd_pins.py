"""Checks that pin the fp64 backward oracle to things other than itself.

Each ``pin_*`` function takes the forward oracle module ``A`` and the backward
oracle module ``G`` and raises AssertionError when the backward disagrees
with: central finite differences of the forward oracle's output (the
derivative by its definition), torch autograd in float64 through an attention
written here with torch ops (an independent library), closed forms, or the
full-sequence gradient split over ranks.  test_oracle_bwd_mutations.py runs
the same functions against deliberately broken copies of the backward oracle.
"""
from __future__ import annotations

import math

import numpy as np

from tests.oracle_pins import _close, _tiny_docs

CASES = [("none", None), ("causal", None), ("doc_causal", "docs")]


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _setup(seed, N, L, H, d, B=1):
    rng = np.random.default_rng(seed)
    q = _rand(rng, B, L, H, d)
    ks = [_rand(rng, B, L, H, d) for _ in range(N)]
    vs = [_rand(rng, B, L, H, d) for _ in range(N)]
    do = _rand(rng, B, L, H, d)
    return q, ks, vs, do


def _cu(mask, S):
    return _tiny_docs(S) if mask == "doc_causal" else None


def pin_bwd_finite_differences(A, G):
    """dQ, dK_j, dV_j of the definition = central differences of
    sum(O * dO) with O from the forward oracle, for every input element."""
    N, L, H, d = 2, 4, 2, 3
    for mask, _ in CASES:
        for rank in range(N):
            q, ks, vs, do = _setup(11 + rank, N, L, H, d)
            cu = _cu(mask, N * L)

            def loss(q_, ks_, vs_):
                o = A.rank_attention(q_, ks_, vs_, rank, N, mask, cu)["o"]
                return float(np.sum(o * do))

            got = G.rank_backward(q, ks, vs, do, rank, N, mask, cu)
            h = 1e-6

            def num_grad(arr, f):
                g = np.zeros_like(arr)
                for idx in np.ndindex(arr.shape):
                    x0 = arr[idx]
                    arr[idx] = x0 + h
                    fp = f()
                    arr[idx] = x0 - h
                    fm = f()
                    arr[idx] = x0
                    g[idx] = (fp - fm) / (2 * h)
                return g

            _close(got["dq"], num_grad(q, lambda: loss(q, ks, vs)), rtol=1e-6, atol=1e-7,
                   what=f"dq fd {mask} r{rank}")
            for j in range(N):
                _close(got["dk"][j], num_grad(ks[j], lambda: loss(q, ks, vs)), rtol=1e-6, atol=1e-7,
                       what=f"dk{j} fd {mask} r{rank}")
                _close(got["dv"][j], num_grad(vs[j], lambda: loss(q, ks, vs)), rtol=1e-6, atol=1e-7,
                       what=f"dv{j} fd {mask} r{rank}")


def pin_bwd_autograd(A, G):
    """The definition = torch autograd (float64, CPU) through masked softmax
    attention written with torch ops, on every rank of a small ring."""
    import torch
    N, L, H, d = 3, 5, 2, 4
    for mask, _ in CASES:
        q, ks, vs, do = _setup(23, N, L, H, d)
        cu = _cu(mask, N * L)
        S = N * L
        pos = np.arange(S)
        vis = np.asarray(A.visibility(pos, pos, mask, cu)) if mask != "none" else np.ones((S, S), bool)
        K = torch.tensor(np.concatenate(ks, axis=1), dtype=torch.float64, requires_grad=True)
        V = torch.tensor(np.concatenate(vs, axis=1), dtype=torch.float64, requires_grad=True)
        for rank in range(N):
            Q = torch.tensor(q, dtype=torch.float64, requires_grad=True)
            rows = slice(rank * L, (rank + 1) * L)
            sc = torch.einsum("blhd,bchd->bhlc", Q, K) / math.sqrt(d)
            m = torch.tensor(vis[rows][None, None])
            sc = sc.masked_fill(~m, float("-inf"))
            P = torch.softmax(sc, dim=-1)
            O = torch.einsum("bhlc,bchd->blhd", P, V)
            if K.grad is not None:
                K.grad = None
                V.grad = None
            (O * torch.tensor(do)).sum().backward()
            got = G.rank_backward(q, ks, vs, do, rank, N, mask, cu)
            _close(got["dq"], Q.grad.numpy(), rtol=1e-10, atol=1e-12, what=f"dq autograd {mask} r{rank}")
            for j in range(N):
                _close(got["dk"][j], K.grad.numpy()[:, j * L:(j + 1) * L], rtol=1e-10, atol=1e-12,
                       what=f"dk{j} autograd {mask} r{rank}")
                _close(got["dv"][j], V.grad.numpy()[:, j * L:(j + 1) * L], rtol=1e-10, atol=1e-12,
                       what=f"dv{j} autograd {mask} r{rank}")


def pin_bwd_block_form(A, G):
    """P recomputed block by block from the forward's lse, with delta =
    rowsum(dO * O), gives the definition: the blocks' dq parts sum to dQ and
    each block's dk, dv equal the definition's split of dK, dV."""
    N, L, H, d = 3, 6, 2, 4
    for mask, _ in CASES:
        for rank in range(N):
            q, ks, vs, do = _setup(5 + rank, N, L, H, d, B=2)
            cu = _cu(mask, N * L)
            f = A.rank_attention(q, ks, vs, rank, N, mask, cu)
            delta = G.bwd_delta(f["o"], do)
            ref = G.rank_backward(q, ks, vs, do, rank, N, mask, cu)
            dq = np.zeros_like(q)
            for j in range(N):
                part = G.block_backward(q, ks[j], vs[j], do, f["lse"], delta, rank, j, N, mask, cu)
                dq += part["dq"]
                _close(part["dk"], ref["dk"][j], rtol=1e-10, atol=1e-12, what=f"dk{j} {mask} r{rank}")
                _close(part["dv"], ref["dv"][j], rtol=1e-10, atol=1e-12, what=f"dv{j} {mask} r{rank}")
            _close(dq, ref["dq"], rtol=1e-10, atol=1e-12, what=f"dq {mask} r{rank}")


def pin_bwd_delta(A, G):
    """delta = rowsum(dO * O) equals rowsum(P * dP) of the materialised
    softmax (O = P V), computed here from the scores."""
    N, L, H, d = 2, 5, 2, 3
    q, ks, vs, do = _setup(3, N, L, H, d)
    f = A.rank_attention(q, ks, vs, 1, N, "causal")
    got = G.bwd_delta(f["o"], do)
    K = np.concatenate(ks, axis=1)
    V = np.concatenate(vs, axis=1)
    for h in range(H):
        s = q[0, :, h, :] @ K[0, :, h, :].T / math.sqrt(d)
        pos_q = L + np.arange(L)
        s = np.where(np.arange(N * L)[None, :] <= pos_q[:, None], s, -np.inf)
        P = np.exp(s - s.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        dP = do[0, :, h, :] @ V[0, :, h, :].T
        _close(got[0, h], (P * dP).sum(axis=1), rtol=1e-12, atol=1e-12, what=f"delta h{h}")


def pin_bwd_closed_forms(A, G):
    """One visible key: dQ = dK = 0 and dV = dO.  Identical V rows: O does
    not depend on the scores, so dQ = dK = 0 exactly.  Scale 0: uniform P over
    the visible keys, dQ = dK = 0, dV_c = sum over rows seeing c of dO / count."""
    rng = np.random.default_rng(9)
    # one visible key: causal, N = 1, L = 1
    q, k, v, do = (rng.standard_normal((1, 1, 2, 3)) for _ in range(4))
    g = G.rank_backward(q, [k], [v], do, 0, 1, "causal")
    _close(g["dq"], np.zeros_like(q), atol=1e-15, what="1key dq")
    _close(g["dk"][0], np.zeros_like(k), atol=1e-15, what="1key dk")
    _close(g["dv"][0], do, rtol=1e-14, atol=1e-15, what="1key dv")
    # identical V rows
    N, L, H, d = 2, 4, 2, 3
    q, ks, vs, do = _setup(17, N, L, H, d)
    row = rng.standard_normal(d)
    vs = [np.broadcast_to(row, v.shape).copy() for v in vs]
    for mask in ("none", "causal"):
        g = G.rank_backward(q, ks, vs, do, 1, N, mask)
        _close(g["dq"], np.zeros_like(q), atol=1e-13, what=f"constV dq {mask}")
        for j in range(N):
            _close(g["dk"][j], np.zeros_like(q), atol=1e-13, what=f"constV dk {mask}")
    # scale 0
    q, ks, vs, do = _setup(19, N, L, H, d)
    g = G.rank_backward(q, ks, vs, do, 1, N, "causal", scale=0.0)
    _close(g["dq"], np.zeros_like(q), atol=1e-15, what="scale0 dq")
    pos_q = L + np.arange(L)
    for j in range(N):
        _close(g["dk"][j], np.zeros_like(q), atol=1e-15, what="scale0 dk")
        expect = np.zeros_like(q)
        for c in range(L):
            cg = j * L + c
            for r in range(L):
                if cg <= pos_q[r]:
                    expect[:, c] += do[:, r] / (pos_q[r] + 1)
        _close(g["dv"][j], expect, rtol=1e-13, atol=1e-14, what=f"scale0 dv{j}")


def pin_bwd_ranks_sum(A, G):
    """Summed over all ranks, each block's dK, dV contributions are the
    full-sequence gradient of the same keys; each rank's dQ is its rows of the
    full-sequence dQ."""
    N, L, H, d = 3, 4, 1, 3
    for mask, _ in CASES:
        q_full, ks, vs, do_full = _setup(29, N, L, H, d)
        rng = np.random.default_rng(31)
        qs = [rng.standard_normal((1, L, H, d)) for _ in range(N)]
        dos = [rng.standard_normal((1, L, H, d)) for _ in range(N)]
        cu = _cu(mask, N * L)
        Qf = np.concatenate(qs, axis=1)[0, :, 0, :]
        dOf = np.concatenate(dos, axis=1)[0, :, 0, :]
        Kf = np.concatenate(ks, axis=1)[0, :, 0, :]
        Vf = np.concatenate(vs, axis=1)[0, :, 0, :]
        pos = np.arange(N * L)
        gq, gk, gv = G.attention_grad_rows(Qf, Kf, Vf, dOf, pos, pos, mask, cu)
        dk_sum = np.zeros((N * L, d))
        dv_sum = np.zeros((N * L, d))
        for rank in range(N):
            g = G.rank_backward(qs[rank], ks, vs, dos[rank], rank, N, mask, cu)
            _close(g["dq"][0, :, 0, :], gq[rank * L:(rank + 1) * L], rtol=1e-12, atol=1e-13,
                   what=f"dq rows {mask} r{rank}")
            for j in range(N):
                dk_sum[j * L:(j + 1) * L] += g["dk"][j][0, :, 0, :]
                dv_sum[j * L:(j + 1) * L] += g["dv"][j][0, :, 0, :]
        _close(dk_sum, gk, rtol=1e-12, atol=1e-13, what=f"dk sum {mask}")
        _close(dv_sum, gv, rtol=1e-12, atol=1e-13, what=f"dv sum {mask}")


ALL_BWD_PINS = [pin_bwd_finite_differences, pin_bwd_autograd, pin_bwd_block_form, pin_bwd_delta,
                pin_bwd_closed_forms, pin_bwd_ranks_sum]
