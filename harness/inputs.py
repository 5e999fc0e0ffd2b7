"""Seeded synthetic inputs for one context-parallel rank's ring-attention shard.

This module is shared by the CPU oracle checks, the GPU parity tests and the
benchmark.  It holds NO attention arithmetic: it only draws numbers, rounds
them to the storage type, samples packed-document boundaries and describes the
workload shapes.

Shapes follow the shard statement of the compassingai.com context-parallelism
page (section "數學基礎"): rank i holds Q_i, K_i, V_i of shape (S/N) x H x d,
contiguous token ranges, here with a leading batch dimension: [B, L, H, d],
L = S/N.

Every tensor block is drawn from its own counter-style stream
``PCG64(SeedSequence([seed, cfg_id, tensor_id, block]))`` so that any one shard
can be regenerated alone, in any order.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_DOCS, TENSOR_DO = 0, 1, 2, 3, 4

MASK_NONE, MASK_CAUSAL, MASK_DOC_CAUSAL = "none", "causal", "doc_causal"
MASKS = (MASK_NONE, MASK_CAUSAL, MASK_DOC_CAUSAL)


def rng_for(seed: int, cfg_id: int, tensor_id: int, block: int) -> np.random.Generator:
    """Independent generator for one (tensor, block) of one workload."""
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([int(seed), int(cfg_id), int(tensor_id), int(block)])))


def normal_block(seed: int, cfg_id: int, tensor_id: int, block: int,
                 shape: Sequence[int]) -> np.ndarray:
    """Standard-normal float32 draw for one block."""
    return rng_for(seed, cfg_id, tensor_id, block).standard_normal(tuple(shape), dtype=np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16, so the
    same numbers can be handed to the device (as bf16) and to an fp64 checker
    (upcast exactly).  Inputs here are finite normal draws; NaN/Inf handling is
    not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x_bf16_exact: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values already rounded to bfloat16."""
    u = np.ascontiguousarray(x_bf16_exact, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def lognormal_cu_seqlens(seed: int, cfg_id: int, S: int, median: float = 4096.0,
                         sigma: float = 1.0, lo: int = 256, hi: int = 32768) -> np.ndarray:
    """Packed-document boundaries over a whole sequence of S tokens.

    Document lengths are lognormal with the given median and sigma; a draw
    outside [lo, hi] is redrawn; lengths are rounded to integers; documents are
    appended until the sequence is full, and the last one is cut to the
    remainder (so it may be shorter than ``lo``).  Returns int32
    ``cu_seqlens`` with cu[0] = 0, cu[-1] = S, strictly increasing.
    """
    rng = rng_for(seed, cfg_id, TENSOR_DOCS, 0)
    mu = float(np.log(median))
    cu: List[int] = [0]
    while cu[-1] < S:
        while True:
            n = int(round(float(rng.lognormal(mu, sigma))))
            if lo <= n <= hi:
                break
        cu.append(min(S, cu[-1] + n))
    return np.asarray(cu, dtype=np.int32)


@dataclasses.dataclass
class ShardSpec:
    """One rank's workload: a total sequence S split over N ring ranks."""
    S: int
    N: int
    H: int
    d: int
    dtype: str = "bf16"          # "f32" or "bf16": storage/compute type of Q, K, V
    mask: str = MASK_CAUSAL
    rank: int = 0
    B: int = 1
    q_scale: float = 1.0
    cu_seqlens: Optional[np.ndarray] = None
    cfg_id: int = 0
    name: str = ""

    @property
    def L(self) -> int:
        assert self.S % self.N == 0, "equal contiguous shards"
        return self.S // self.N

    def shard_shape(self):
        return (self.B, self.L, self.H, self.d)


def draw_shard(spec: ShardSpec, seed: int, tensor_id: int, block: int) -> np.ndarray:
    """Q (tensor_id=TENSOR_Q, block=rank) or K/V block ``block``, float32,
    already rounded to bf16 when spec.dtype == 'bf16'."""
    x = normal_block(seed, spec.cfg_id, tensor_id, block, spec.shard_shape())
    if tensor_id == TENSOR_Q and spec.q_scale != 1.0:
        x = x * np.float32(spec.q_scale)
    if spec.dtype == "bf16":
        x = round_to_bf16(x)
    return x


def draw_grad(spec: ShardSpec, seed: int, rank: int) -> np.ndarray:
    """Upstream gradient dO of rank ``rank``'s output, N(0, 1), float32,
    rounded to bf16 when spec.dtype == 'bf16' (the backward's input)."""
    x = normal_block(seed, spec.cfg_id, TENSOR_DO, rank, spec.shard_shape())
    if spec.dtype == "bf16":
        x = round_to_bf16(x)
    return x


def make_inputs(spec: ShardSpec, seed: int, ranks: Optional[Sequence[int]] = None,
                blocks: Optional[Sequence[int]] = None) -> Dict[str, object]:
    """Q shards for ``ranks`` (default: spec.rank) and K/V for ``blocks``
    (default: all N)."""
    ranks = [spec.rank] if ranks is None else list(ranks)
    blocks = list(range(spec.N)) if blocks is None else list(blocks)
    return {
        "q": {r: draw_shard(spec, seed, TENSOR_Q, r) for r in ranks},
        "k": {j: draw_shard(spec, seed, TENSOR_K, j) for j in blocks},
        "v": {j: draw_shard(spec, seed, TENSOR_V, j) for j in blocks},
    }


def standard_configs(seed: int = 0) -> Dict[int, ShardSpec]:
    """The five workloads: a tiny fp32 ring of 4 ranks, two causal last-rank
    shards (32K and the 128K-over-4-GPUs example), a bidirectional merge
    stress case and a packed-document case."""
    cfgs = {
        1: ShardSpec(S=1024, N=4, H=2, d=64, dtype="f32", mask=MASK_CAUSAL, rank=3, cfg_id=1,
                     name="tiny fp32 ring S=1024 N=4 H=2 d=64 causal"),
        2: ShardSpec(S=32768, N=4, H=8, d=128, dtype="bf16", mask=MASK_CAUSAL, rank=3, cfg_id=2,
                     name="causal last-rank S=32768 N=4 H=8 d=128 bf16"),
        3: ShardSpec(S=131072, N=4, H=32, d=128, dtype="bf16", mask=MASK_CAUSAL, rank=3, cfg_id=3,
                     name="causal last-rank S=131072 N=4 H=32 d=128 bf16 ring-prefetch"),
        4: ShardSpec(S=65536, N=8, H=16, d=128, dtype="bf16", mask=MASK_NONE, rank=5, cfg_id=4,
                     q_scale=3.0, name="bidirectional partial+merge S=65536 N=8 H=16 d=128 bf16 Qx3"),
        5: ShardSpec(S=131072, N=8, H=32, d=128, dtype="bf16", mask=MASK_DOC_CAUSAL, rank=7, cfg_id=5,
                     name="packed documents S=131072 N=8 H=32 d=128 bf16 doc+causal"),
    }
    cfgs[5].cu_seqlens = lognormal_cu_seqlens(seed, 5, cfgs[5].S)
    return cfgs


def shuffled_order(seed: int, cfg_id: int, n: int) -> List[int]:
    """Seeded random permutation of range(n) (merge order for the merge stress case)."""
    return [int(x) for x in rng_for(seed, cfg_id, 99, 0).permutation(n)]
