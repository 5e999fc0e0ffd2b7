"""fp64 CPU oracle for one rank's share of all-to-all (Ulysses) context parallelism.

TEST INFRASTRUCTURE ONLY.  This module is the correctness reference for the
HIP library's ``cp_attn_ulysses_forward``.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call it; the product path never does.  It shares no code with the
HIP path (it imports numpy, the standard library and the forward oracle).

What the pages fix (compassingai.com context-parallelism page, section
"方案二：All-to-All（全交換）"): the ranks hold sequence shards; a first
all-to-all regroups Q, K and V from split-by-sequence to split-by-head; each
rank then computes attention over the whole sequence for its heads; a second
all-to-all regroups the outputs back to split-by-sequence.  The same page
(section "技術路線對比") notes that under a causal mask this scheme masks the
invalid region instead of skipping ring steps, and (section "通訊量分析")
that it moves about 2 x S H d elements per layer forward (the regroup and
its inverse).

Functions:

* ``heads_of`` - the head group of a rank.
* ``seq_to_heads`` - the first all-to-all as seen by one receiving rank:
  every rank's tokens of the receiver's heads, concatenated in rank order,
  [B, S, H/N, d].
* ``heads_to_seq`` - the second all-to-all as sent by one rank: its
  full-sequence result [B, S, H/N, d] cut into the N token ranges, piece i
  for rank i, [B, L, H/N, d].
* ``ulysses_rank`` - the three steps for one rank, with the attention of
  step 2 taken from the definition (``attention.attention_rows``: masked
  softmax over materialised score rows).

Readings of points the pages leave open:
  * rank r takes the contiguous head group [r H/N, (r+1) H/N); H must be a
    multiple of N;
  * after the first all-to-all the sequence is the ranks' shards in rank
    order, shard i covering global positions [i L, (i+1) L): the same
    positions the ring uses, so the causal and document masks are the same;
  * m, l and lse are exported per head over the whole sequence, [B, H/N, S],
    in natural-log units as the ring exports them.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from . import attention as fwd

__all__ = ["heads_of", "seq_to_heads", "heads_to_seq", "ulysses_rank"]


def heads_of(rank: int, N: int, H: int) -> range:
    """Head group of ``rank``: [rank H/N, (rank+1) H/N)."""
    if H % N:
        raise ValueError(f"H={H} is not a multiple of N={N}")
    hn = H // N
    return range(rank * hn, (rank + 1) * hn)


def seq_to_heads(shards: Sequence[np.ndarray], rank: int, N: int) -> np.ndarray:
    """First all-to-all, receiving side of ``rank``: shards are the N ranks'
    [B, L, H, d] tensors; returns [B, N L, H/N, d] with the receiver's heads of
    every shard, shards in rank order along the sequence."""
    assert len(shards) == N
    H = shards[0].shape[2]
    hs = heads_of(rank, N, H)
    return np.concatenate([np.asarray(x)[:, :, hs.start:hs.stop, :] for x in shards], axis=1)


def heads_to_seq(full: np.ndarray, N: int) -> List[np.ndarray]:
    """Second all-to-all, sending side: ``full`` [B, N L, H/N, d] of one rank's
    heads is cut into N token ranges; piece i [B, L, H/N, d] goes to rank i."""
    S = full.shape[1]
    assert S % N == 0
    L = S // N
    return [full[:, i * L:(i + 1) * L] for i in range(N)]


def ulysses_rank(q_shards: Sequence[np.ndarray], k_shards: Sequence[np.ndarray],
                 v_shards: Sequence[np.ndarray], rank: int, N: int, mask: str,
                 cu_seqlens=None, scale: Optional[float] = None) -> Dict[str, object]:
    """The three steps for ``rank``.  Returns ``o_parts`` (a list of N
    [B, L, H/N, d] arrays: piece i is what this rank sends back to rank i, the
    outputs of rank i's tokens for this rank's heads) and ``m``, ``l``,
    ``lse`` [B, H/N, S] over the whole sequence, all float64."""
    Q = seq_to_heads(q_shards, rank, N).astype(np.float64)
    K = seq_to_heads(k_shards, rank, N).astype(np.float64)
    V = seq_to_heads(v_shards, rank, N).astype(np.float64)
    B, S, Hn, d = Q.shape
    pos = np.arange(S, dtype=np.int64)
    O = np.zeros((B, S, Hn, d))
    M = np.zeros((B, Hn, S))
    Lsum = np.zeros((B, Hn, S))
    LSE = np.zeros((B, Hn, S))
    for b in range(B):
        for h in range(Hn):
            o, m, l, lse = fwd.attention_rows(Q[b, :, h], K[b, :, h], V[b, :, h], pos, pos, mask,
                                              cu_seqlens, scale)
            O[b, :, h] = o
            M[b, h] = m
            Lsum[b, h] = l
            LSE[b, h] = lse
    return {"o_parts": heads_to_seq(O, N), "m": M, "l": Lsum, "lse": LSE}
