"""fp64 CPU oracle for the backward of one context-parallel rank's shard.

TEST INFRASTRUCTURE ONLY.  This module is the correctness reference for the
HIP library's backward entry points.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call it; the product path never does.  It shares no code with the
HIP path (it imports numpy, the standard library and the forward oracle).

What the pages fix: the backward of context parallelism differentiates the
same blockwise attention and walks the ring's K/V blocks again, recomputing
what the forward did not keep (compassingai.com context-parallelism page,
section "反向傳播"; the gradients of Q, K and V are sent back around the ring,
process-cxr.github.io page, section "Long Context Attention 中的通信").  The
pages print no gradient formulas; the functions below are the chain rule of
the forward definition (compassingai.com page, section "數學基礎": O =
softmax(Q K^T / sqrt(d)) V with the mask of section "因果掩碼的特殊處理"),
written out:

* ``attention_grad_rows`` - the definition: materialise P = softmax of the
  masked scaled scores, then dV = P^T dO, dP = dO V^T,
  dS = P * (dP - rowsum(P * dP)), dQ = scale dS K, dK = scale dS^T Q.
* ``bwd_delta`` - delta = rowsum(dO * O) per row; equal to rowsum(P * dP)
  because O = P V.
* ``block_backward`` - the contributions through one block j with P_j
  recomputed from the forward's log-sum-exp: P_j = exp(S_j - lse),
  dS_j = P_j * (dO V_j^T - delta); dQ gets dS_j K_j scale, the block gets
  dK_j = dS_j^T Q scale, dV_j = P_j^T dO.
* ``rank_backward`` - the definition over every block this rank sees: dQ of
  the shard and the shard's contributions to dK_j, dV_j of each block
  (zero for blocks it does not see).

Readings of points the pages leave open:
  * the backward of a rank shard returns that rank's dQ and its contributions
    to every block's dK, dV; summing the contributions of all ranks gives the
    gradient of the full-sequence attention (the ring carries them home);
  * P is recomputed from the global lse of the forward, and rows whose lse is
    -inf (no visible key anywhere) contribute nothing;
  * delta uses the forward output O as given (rowsum(dO * O)).
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

from . import attention as fwd

__all__ = ["attention_grad_rows", "bwd_delta", "block_backward", "rank_backward"]


def attention_grad_rows(q, k, v, do, p, c, mask: str, cu_seqlens=None,
                        scale: Optional[float] = None):
    """Gradients of O = softmax(mask(q k^T scale)) v for query rows q [R,d] at
    global positions p, keys k, v [T,d] at positions c, upstream dO [R,d].
    Returns dq [R,d], dk [T,d], dv [T,d] in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    s = (q @ k.T) * scale
    vis = fwd.visibility(p, c, mask, cu_seqlens)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    empty = ~np.isfinite(m)
    e = np.exp(s - np.where(empty, 0.0, m)[:, None])
    den = e.sum(axis=1)
    P = np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, den)[:, None])
    dv = P.T @ do
    dP = do @ v.T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    dq = (dS @ k) * scale
    dk = (dS.T @ q) * scale
    return dq, dk, dv


def bwd_delta(o, do) -> np.ndarray:
    """delta [B,H,L] = sum over the head dim of dO * O, for o, do [B,L,H,d]."""
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    return np.einsum("blhd,blhd->bhl", do, o)


def block_backward(q, k_j, v_j, do, lse, delta, rank: int, j: int, N: int, mask: str,
                   cu_seqlens=None, scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Contributions of shard ``rank`` through block ``j``: q, k_j, v_j, do
    [B,L,H,d]; lse, delta [B,H,L] of the whole forward (natural-log units).
    Returns dq (this block's part of dQ), dk, dv of block j, each [B,L,H,d]."""
    B, L, H, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    p = rank * L + np.arange(L, dtype=np.int64)
    c = j * L + np.arange(L, dtype=np.int64)
    vis = fwd.visibility(p, c, mask, cu_seqlens)
    out = {n: np.zeros((B, L, H, d)) for n in ("dq", "dk", "dv")}
    for b in range(B):
        for h in range(H):
            Q = np.asarray(q[b, :, h, :], dtype=np.float64)
            K = np.asarray(k_j[b, :, h, :], dtype=np.float64)
            V = np.asarray(v_j[b, :, h, :], dtype=np.float64)
            dO = np.asarray(do[b, :, h, :], dtype=np.float64)
            ls = np.asarray(lse[b, h], dtype=np.float64)
            s = (Q @ K.T) * scale
            finite = np.isfinite(ls)
            live = finite[:, None] & vis                    # recomputed entries
            shifted = s - np.where(finite, ls, 0.0)[:, None]
            P = np.where(live, np.exp(np.where(live, shifted, 0.0)), 0.0)
            dS = P * (dO @ V.T - np.asarray(delta[b, h], dtype=np.float64)[:, None])
            out["dq"][b, :, h, :] = (dS @ K) * scale
            out["dk"][b, :, h, :] = (dS.T @ Q) * scale
            out["dv"][b, :, h, :] = P.T @ dO
    return out


def rank_backward(q, k_blocks: Sequence, v_blocks: Sequence, do, rank: int, N: int, mask: str,
                  cu_seqlens=None, scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """The definition for shard ``rank``: dq [B,L,H,d] and, for every block j,
    the shard's contribution dk[j], dv[j] [B,L,H,d] (zero when the shard sees
    no key of block j).  All N blocks must be given."""
    B, L, H, d = q.shape
    assert len(k_blocks) == N and len(v_blocks) == N
    p = rank * L + np.arange(L, dtype=np.int64)
    c = np.arange(N * L, dtype=np.int64)
    dq = np.zeros((B, L, H, d))
    dk = np.zeros((N, B, L, H, d))
    dv = np.zeros((N, B, L, H, d))
    for b in range(B):
        for h in range(H):
            K = np.concatenate([np.asarray(k_blocks[j][b, :, h, :], dtype=np.float64) for j in range(N)])
            V = np.concatenate([np.asarray(v_blocks[j][b, :, h, :], dtype=np.float64) for j in range(N)])
            gq, gk, gv = attention_grad_rows(q[b, :, h, :], K, V, do[b, :, h, :], p, c, mask,
                                             cu_seqlens, scale)
            dq[b, :, h, :] = gq
            for j in range(N):
                dk[j, b, :, h, :] = gk[j * L:(j + 1) * L]
                dv[j, b, :, h, :] = gv[j * L:(j + 1) * L]
    return {"dq": dq, "dk": dk, "dv": dv}
