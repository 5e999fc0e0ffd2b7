"""fp64 CPU oracle for one context-parallel rank's ring-attention shard.

TEST INFRASTRUCTURE ONLY.  This module is the correctness reference for the
HIP library.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call it; the product path
never does.  It shares no code with the HIP path (it imports only numpy and
the standard library).

What it computes (all in float64):

* ``rank_attention`` - the definition: softmax(Q_i [K_0;...;K_{N-1}]^T / sqrt(d))
  [V_0;...;V_{N-1}] for the query rows of rank i, with the mask applied to the
  materialised score rows.  Sources: compassingai.com context-parallelism page
  (section "數學基礎", the Attn and Attn_i formulas; section "因果掩碼的特殊處理"
  for the causal rule); wangyu.me page (section "上下文并行的原理", the
  softmax(QK^T/sqrt(d_k))V formula); process-cxr.github.io page (sections
  "配置关注点" and "常见失败模式": document-boundary masks must hold across
  shards).
* ``streaming_attention`` - the streaming form of the wangyu.me page (section
  "Attention 的流式计算"): no max shift, the output is the ratio of the sum of
  exp(score) V over the sum of exp(score); both sums are taken here over all
  blocks' keys at once.
* ``online_merge`` - the online-softmax form of the compassingai.com page
  (section "線上 Softmax"): per-block partial states (O_j, m_j, l_j) folded
  into a running state in the visiting order with the pairwise merge rule
  (``_combine``), O / l at the end.
* ``block_partial`` / ``merge_lse`` - per-block normalised partials (O_j, lse_j)
  and their log-sum-exp merge (the same recurrence written in lse form: the
  process-cxr.github.io page, section "Long Context Attention 中的通信", asks
  that the blockwise softmax keep the max/sum reductions).
* ``ring_schedule`` - ring visit order and mask-aware block skipping
  (compassingai.com page, sections "方案一：Ring Attention" and "因果掩碼的特殊處理";
  wangyu.me page, sections "Ring Attention" and "通信模式").
* ``brute_force`` - pure-Python loops with math.exp / math.fsum for tiny inputs.

Readings of points the pages leave open:
  * causal visibility includes the diagonal: key c is visible to query p iff
    c <= p (the pages say a token sees the tokens before it; without the
    diagonal the first row of rank 0 would see nothing);
  * doc_causal: visible iff doc_start(p) <= c <= p, doc_start(p) = cu[k] with
    cu[k] <= p < cu[k+1]; cu_seqlens are global positions over all S tokens;
  * a row with no visible key in a block has m = -inf, l = 0, O = 0,
    lse = -inf, and contributes nothing to a merge;
  * m is the row max of the scaled scores in natural-log units, l = sum of
    exp(s - m) over visible keys, lse = m + ln l;
  * default scale 1/sqrt(d).
"""
from __future__ import annotations

import itertools
import math
from typing import Dict, Iterable, List, Mapping, Optional, Sequence

import numpy as np

NONE, CAUSAL, DOC_CAUSAL = "none", "causal", "doc_causal"

__all__ = [
    "doc_start", "visibility", "attention_rows", "rank_attention", "block_partial",
    "streaming_attention", "online_merge", "merge_lse", "ring_schedule", "block_visible",
    "visible_pairs", "brute_force", "ring_traffic_bytes",
]


# ----------------------------------------------------------------------------
# masks
# ----------------------------------------------------------------------------

def doc_start(p: np.ndarray, cu_seqlens: np.ndarray) -> np.ndarray:
    """First position of the document holding global position p."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    idx = np.searchsorted(cu, np.asarray(p, dtype=np.int64), side="right") - 1
    return cu[idx]


def visibility(p: np.ndarray, c: np.ndarray, mask: str,
               cu_seqlens: Optional[np.ndarray] = None) -> np.ndarray:
    """Boolean [len(p), len(c)]: may query at global position p attend to key c."""
    P = np.asarray(p, dtype=np.int64)[:, None]
    C = np.asarray(c, dtype=np.int64)[None, :]
    if mask == NONE:
        return np.ones((P.shape[0], C.shape[1]), dtype=bool)
    if mask == CAUSAL:
        return C <= P
    if mask == DOC_CAUSAL:
        lo = doc_start(P[:, 0], cu_seqlens)[:, None]
        return (C <= P) & (C >= lo)
    raise ValueError(mask)


# ----------------------------------------------------------------------------
# the definition
# ----------------------------------------------------------------------------

def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, p: np.ndarray,
                   c: np.ndarray, mask: str, cu_seqlens=None, scale: Optional[float] = None):
    """Masked softmax attention of query rows q [R,d] (global positions p) over
    keys k, v [T,d] (global positions c).  Returns O [R,d], m, l, lse [R].

    Score rows are materialised in full, invisible entries set to -inf,
    softmax taken with the row max subtracted, multiplied by V.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    s = (q @ k.T) * scale
    vis = visibility(p, c, mask, cu_seqlens)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 for invisible entries
    l = e.sum(axis=1)
    num = e @ v
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(empty[:, None], 0.0, num / np.where(empty, 1.0, l)[:, None])
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    l = np.where(empty, 0.0, l)
    return o, m, l, lse


def _as_block_list(blocks, N: int):
    if isinstance(blocks, Mapping):
        return [blocks.get(j) for j in range(N)]
    blocks = list(blocks)
    assert len(blocks) == N
    return blocks


def block_visible(N: int, L: int, rank: int, j: int, mask: str,
                  cu_seqlens: Optional[np.ndarray] = None) -> bool:
    """Does any query row of shard ``rank`` see any key of block ``j``?

    Checked row by row: row p sees keys [lo_p, hi_p] of block j with
    lo_p = max(jL, first visible key of p), hi_p = min((j+1)L-1, p) (causal
    forms) - the block is visible iff some row has lo_p <= hi_p.
    """
    if mask == NONE:
        return True
    p = np.arange(rank * L, (rank + 1) * L, dtype=np.int64)
    first = p * 0 if mask == CAUSAL else doc_start(p, cu_seqlens)
    lo = np.maximum(first, j * L)
    hi = np.minimum(p, (j + 1) * L - 1)
    return bool(np.any(lo <= hi))


def rank_attention(q: np.ndarray, k_blocks, v_blocks, rank: int, N: int, mask: str,
                   cu_seqlens=None, scale: Optional[float] = None,
                   rows: Optional[np.ndarray] = None, heads: Optional[Iterable[int]] = None,
                   chunk: int = 512) -> Dict[str, np.ndarray]:
    """The definition for rank ``rank``: q [B,L,H,d]; k_blocks, v_blocks are the
    N blocks [B,L,H,d] (a list, or a dict that may omit blocks that no row of
    this rank can see).  ``rows`` (shard-local indices) and ``heads`` select a
    subset of outputs.  Returns O [B,R,Hs,d], m, l, lse [B,Hs,R] in float64.
    """
    B, L, H, d = q.shape
    kb = _as_block_list(k_blocks, N)
    vb = _as_block_list(v_blocks, N)
    present = [j for j in range(N) if kb[j] is not None]
    for j in range(N):
        if kb[j] is None:
            assert not block_visible(N, L, rank, j, mask, cu_seqlens), \
                f"block {j} is visible to rank {rank} and must be supplied"
    c = np.concatenate([np.arange(j * L, (j + 1) * L, dtype=np.int64) for j in present])
    rows = np.arange(L, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(H)) if heads is None else list(heads)
    R, Hs = rows.shape[0], len(heads)
    O = np.zeros((B, R, Hs, d))
    M = np.zeros((B, Hs, R))
    Lsum = np.zeros((B, Hs, R))
    LSE = np.zeros((B, Hs, R))
    for b in range(B):
        for hi, h in enumerate(heads):
            K = np.concatenate([np.asarray(kb[j][b, :, h, :], dtype=np.float64) for j in present])
            V = np.concatenate([np.asarray(vb[j][b, :, h, :], dtype=np.float64) for j in present])
            for r0 in range(0, R, chunk):
                rr = rows[r0:r0 + chunk]
                o, m, l, lse = attention_rows(q[b, rr, h, :], K, V, rank * L + rr, c, mask,
                                              cu_seqlens, scale)
                O[b, r0:r0 + chunk, hi, :] = o
                M[b, hi, r0:r0 + chunk] = m
                Lsum[b, hi, r0:r0 + chunk] = l
                LSE[b, hi, r0:r0 + chunk] = lse
    return {"o": O, "m": M, "l": Lsum, "lse": LSE}


def block_partial(q: np.ndarray, k_j: np.ndarray, v_j: np.ndarray, rank: int, j: int, N: int,
                  mask: str, cu_seqlens=None, scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Attention of shard ``rank``'s queries over the keys of block ``j`` alone:
    normalised O_j [B,L,H,d] and m_j, l_j, lse_j [B,H,L]; rows that see no key
    of the block get O = 0, m = lse = -inf, l = 0."""
    B, L, H, d = q.shape
    p = rank * L + np.arange(L, dtype=np.int64)
    c = j * L + np.arange(L, dtype=np.int64)
    O = np.zeros((B, L, H, d))
    M = np.zeros((B, H, L))
    Ls = np.zeros((B, H, L))
    LSE = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            o, m, l, lse = attention_rows(q[b, :, h, :], k_j[b, :, h, :], v_j[b, :, h, :], p, c,
                                          mask, cu_seqlens, scale)
            O[b, :, h, :] = o
            M[b, h] = m
            Ls[b, h] = l
            LSE[b, h] = lse
    return {"o": O, "m": M, "l": Ls, "lse": LSE}


# ----------------------------------------------------------------------------
# the pages' blockwise forms
# ----------------------------------------------------------------------------

def streaming_attention(q: np.ndarray, k_blocks: Sequence[np.ndarray],
                        v_blocks: Sequence[np.ndarray], p: np.ndarray,
                        c_blocks: Sequence[np.ndarray], mask: str, cu_seqlens=None,
                        scale: Optional[float] = None) -> np.ndarray:
    """Rows q [R,d] against all K/V blocks in the streaming form of the
    wangyu.me page (section "Attention 的流式计算"): no maximum is subtracted,
    the output is a ratio of two sums over the visible keys, the weights
    w = exp(score) times V over the weights alone.  Both sums run over every
    block, so here they are taken over the blocks' keys concatenated.  Valid
    while scores stay far below ~700 (float64 exp range)."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    k_all = np.concatenate([np.asarray(k, np.float64) for k in k_blocks])
    v_all = np.concatenate([np.asarray(v, np.float64) for v in v_blocks])
    c_all = np.concatenate([np.asarray(c) for c in c_blocks])
    w = np.where(visibility(p, c_all, mask, cu_seqlens), np.exp((q @ k_all.T) * scale), 0.0)
    return (w @ v_all) / w.sum(axis=1)[:, None]


def _exp_shift(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """exp(a - b), taken as 0 where a = -inf (an empty contribution)."""
    with np.errstate(invalid="ignore"):
        return np.where(np.isneginf(a), 0.0, np.exp(a - np.where(np.isneginf(b), 0.0, b)))


def _block_state(q: np.ndarray, k: np.ndarray, v: np.ndarray, p: np.ndarray, c: np.ndarray,
                 mask: str, cu_seqlens, scale: float):
    """The unnormalised partial state of rows q against one K/V block: m = the
    row maximum of the visible scaled scores, l = the row sum of exp(score -
    m), O = those exponentials times V.  A row that sees no key of the block
    has m = -inf, l = 0, O = 0."""
    S = np.where(visibility(p, c, mask, cu_seqlens), (q @ np.asarray(k, np.float64).T) * scale, -np.inf)
    m = S.max(axis=1) if S.shape[1] else np.full(q.shape[0], -np.inf)
    E = _exp_shift(S, m[:, None])
    return E @ np.asarray(v, np.float64), m, E.sum(axis=1)


def _combine(a, b):
    """Merge two partial states (O, m, l) of the same rows: both are brought
    to the larger of the two maxima and added (the merge step of the
    compassingai.com page, section "線上 Softmax").  The rule is associative
    and commutative up to rounding, which is what lets the blocks arrive in
    any ring order."""
    (oa, ma, la), (ob, mb, lb) = a, b
    m = np.maximum(ma, mb)
    wa, wb = _exp_shift(ma, m), _exp_shift(mb, m)
    return oa * wa[:, None] + ob * wb[:, None], m, la * wa + lb * wb


def online_merge(q: np.ndarray, k_blocks: Sequence[np.ndarray], v_blocks: Sequence[np.ndarray],
                 p: np.ndarray, c_blocks: Sequence[np.ndarray], order: Sequence[int], mask: str,
                 cu_seqlens=None, scale: Optional[float] = None):
    """The online-softmax form over K/V blocks visited in ``order``: the
    running state starts empty (O = 0, m = -inf, l = 0), each block's partial
    state is folded into it with the merge rule, and the output is O / l
    (compassingai.com page, section "線上 Softmax").  Returns O [R,d], m, l [R]."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    R = q.shape[0]
    state = (np.zeros_like(q), np.full(R, -np.inf), np.zeros(R))
    for j in order:
        state = _combine(state, _block_state(q, k_blocks[j], v_blocks[j], p, c_blocks[j], mask, cu_seqlens, scale))
    O, m, l = state
    with np.errstate(invalid="ignore", divide="ignore"):
        O = np.where((l > 0)[:, None], O / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return O, m, l


def merge_lse(o_parts: Sequence[np.ndarray], lse_parts: Sequence[np.ndarray],
              order: Optional[Sequence[int]] = None):
    """Merge normalised partials in the given order.

    lse = log sum_j exp(lse_j); O = sum_j exp(lse_j - lse) O_j.  o_parts[j] is
    [..., R, d] and lse_parts[j] is [..., R] with matching leading dims (the
    caller aligns layouts).  Parts with lse_j = -inf contribute nothing; rows
    where every part is empty give O = 0, lse = -inf.
    """
    n = len(o_parts)
    order = list(range(n)) if order is None else list(order)
    lse_stack = np.stack([np.asarray(lse_parts[j], np.float64) for j in order])
    mx = lse_stack.max(axis=0)
    mx_safe = np.where(np.isneginf(mx), 0.0, mx)
    tot = np.zeros_like(mx)
    for j in order:
        tot = tot + _exp_shift(np.asarray(lse_parts[j], np.float64), mx_safe)
    with np.errstate(divide="ignore"):
        lse = np.where(tot > 0, mx_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    O = np.zeros_like(np.asarray(o_parts[0], np.float64))
    for j in order:
        w = _exp_shift(np.asarray(lse_parts[j], np.float64), lse)
        O = O + w[..., None] * np.asarray(o_parts[j], np.float64)
    return O, lse


# ----------------------------------------------------------------------------
# ring schedule and work counts
# ----------------------------------------------------------------------------

def ring_schedule(N: int, rank: int, L: int, mask: str, cu_seqlens=None,
                  direction: str = "forward") -> List[int]:
    """Blocks rank ``rank`` computes on, in the order the ring delivers them.

    direction="forward": each rank sends its current block to the next rank
    and receives from the previous one, so at step t it holds block
    (rank - t) mod N.  direction="reverse": it holds block (rank + t) mod N,
    the order of the wangyu.me page's GPU 0 stage table.  Blocks no row of
    this rank can see are dropped (mask-aware skipping)."""
    step = -1 if direction == "forward" else 1
    seq = [(rank + step * t) % N for t in range(N)]
    return [j for j in seq if block_visible(N, L, rank, j, mask, cu_seqlens)]


def visible_pairs(N: int, L: int, rank: int, mask: str, cu_seqlens=None) -> int:
    """Number of visible (query, key) pairs of one head of shard ``rank``."""
    p = np.arange(rank * L, (rank + 1) * L, dtype=np.int64)
    if mask == NONE:
        return int(L * N * L)
    first = np.zeros_like(p) if mask == CAUSAL else doc_start(p, cu_seqlens)
    return int(np.sum(p - first + 1))


def ring_traffic_bytes(S: int, H: int, d: int, elt_bytes: int, N: int, B: int = 1) -> int:
    """Per-GPU bytes sent plus received over a full ring: 2 (G/N) (N-1), G = the
    bytes of K and V of the whole sequence (wangyu.me page, section "通信模式")."""
    G = 2 * B * S * H * d * elt_bytes
    return 2 * (G // N) * (N - 1)


# ----------------------------------------------------------------------------
# brute force
# ----------------------------------------------------------------------------

def brute_force(q: List[List[float]], k: List[List[float]], v: List[List[float]],
                p: List[int], c: List[int], mask: str, cu_seqlens=None,
                scale: Optional[float] = None):
    """Pure-Python loops: for each query row, list the visible keys, take the
    max score, sum exp(s - max) with math.fsum, average V.  Returns lists
    (O, m, l, lse)."""
    d = len(q[0])
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    cu = None if cu_seqlens is None else [int(x) for x in cu_seqlens]

    def first_key(pp):
        if mask == NONE:
            return None
        if mask == CAUSAL:
            return 0
        start = 0
        for a in cu:
            if a <= pp:
                start = a
        return start

    O, M, Lsum, LSE = [], [], [], []
    for qi, pp in zip(q, p):
        lo = first_key(pp)
        keys = [n for n, cc in enumerate(c) if mask == NONE or (lo <= cc <= pp)]
        if not keys:
            O.append([0.0] * d)
            M.append(-math.inf)
            Lsum.append(0.0)
            LSE.append(-math.inf)
            continue
        s = {n: math.fsum(qi[t] * k[n][t] for t in range(d)) * scale for n in keys}
        mx = max(s.values())
        w = {n: math.exp(s[n] - mx) for n in keys}
        den = math.fsum(w.values())
        O.append([math.fsum(w[n] * v[n][t] for n in keys) / den for t in range(d)])
        M.append(mx)
        Lsum.append(den)
        LSE.append(mx + math.log(den))
    return O, M, Lsum, LSE


def all_orders(n: int):
    """Every visit order of n blocks (for order-invariance checks)."""
    return itertools.permutations(range(n))
