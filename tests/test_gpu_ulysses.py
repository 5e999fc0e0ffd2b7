"""GPU parity of the all-to-all (Ulysses) share: cp_attn_ulysses_forward
through the C ABI against the fp64 oracle (oracle/ulysses.py) on the same
seeded inputs.  Tolerances are those of the forward (tests/gpu_util.py).

Small cases: every rank of the group, both input types and head dims, every
mask, ragged lengths (S not a multiple of any tile), batch 2; each call must
write exactly its heads of every output shard (the other heads hold a
sentinel that must survive), and after all ranks every head is written.
Degenerate cases: N = 1 (plain attention of one shard) and one head per
rank.  Full size: the 128K example regrouped over 4 ranks (8 heads each,
S = 131072), checked on sampled rows of every shard.
"""
import numpy as np
import pytest

import oracle
import oracle.ulysses as U
from harness.inputs import TENSOR_K, TENSOR_Q, TENSOR_V, ShardSpec, draw_shard
from tests.gpu_util import check_o, check_stat, dev, host, sample_rows, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENTINEL = 7.0


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_ring_attention_cp_amd as cp
    cp.lib()     # raises if the library is not built: no fallback
    return cp


def _shards(spec, seed):
    return ([draw_shard(spec, seed, TENSOR_Q, i) for i in range(spec.N)],
            [draw_shard(spec, seed, TENSOR_K, i) for i in range(spec.N)],
            [draw_shard(spec, seed, TENSOR_V, i) for i in range(spec.N)])


def _dt(spec):
    return torch.bfloat16 if spec.dtype == "bf16" else torch.float32


def run_rank(cp, spec, r, qd, kd, vd, od):
    cu_dev = None
    if spec.mask == "doc_causal":
        cu_dev = torch.from_numpy(np.asarray(spec.cu_seqlens, np.int32)).cuda()
    d = cp.Desc(spec.B, spec.H, spec.d, spec.N, spec.L, r, spec.dtype, spec.mask,
                cu_seqlens=spec.cu_seqlens, cu_seqlens_dev=cu_dev)
    vec = (spec.B, spec.H // spec.N, spec.S)
    m, l, lse = (torch.full(vec, float("nan"), device="cuda") for _ in range(3))
    ws = cp.alloc_ulysses_workspace(d)
    cp.cp_attn_ulysses_forward(d, qd, kd, vd, od, m, l, lse, workspace=ws)
    torch.cuda.synchronize()
    return host(m), host(l), host(lse)


def _small_cu(S):
    pts, x = [0], 0
    for n in (37, 130, 5, 300, 64, 1, 211, 90, 400):
        x += n
        if x >= S:
            break
        pts.append(x)
    return np.asarray(pts + [S], np.int32)


def _every_rank(cp, spec, seed):
    q, k, v = _shards(spec, seed)
    qd, kd, vd = ([dev(x, spec.dtype) for x in t] for t in (q, k, v))
    od = [torch.full(spec.shard_shape(), SENTINEL, dtype=_dt(spec), device="cuda") for _ in range(spec.N)]
    hn = spec.H // spec.N
    for r in range(spec.N):
        say(f"[ulysses] S={spec.S} N={spec.N} H={spec.H} d={spec.d} {spec.dtype} {spec.mask} rank {r}")
        m, l, lse = run_rank(cp, spec, r, qd, kd, vd, od)
        ref = U.ulysses_rank(q, k, v, r, spec.N, spec.mask, spec.cu_seqlens)
        for i in range(spec.N):
            o = host(od[i])
            check_o(o[:, :, r * hn:(r + 1) * hn], ref["o_parts"][i], spec.dtype, what=f"o shard {i}")
            assert np.all(o[:, :, (r + 1) * hn:] == SENTINEL), f"rank {r} wrote heads of later ranks in shard {i}"
        check_stat(m, ref["m"], spec.dtype, "m")
        check_stat(l, ref["l"], spec.dtype, "l")
        check_stat(lse, ref["lse"], spec.dtype, "lse")
    for i in range(spec.N):
        assert not np.any(host(od[i]) == SENTINEL), f"shard {i}: some head was never written"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", ["none", "causal", "doc_causal"])
def test_small_every_rank(cp, dtype, d, mask):
    N, L, H, B = 3, 100, 6, 2
    spec = ShardSpec(S=N * L, N=N, H=H, d=d, dtype=dtype, mask=mask, B=B, cfg_id=201,
                     cu_seqlens=_small_cu(N * L) if mask == "doc_causal" else None)
    _every_rank(cp, spec, seed=2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", ["none", "doc_causal"])
@pytest.mark.parametrize("N,L", [(4, 48), (2, 96)])
def test_whole_tile_sequences(cp, d, mask, N, L):
    """bf16 over a whole number of 64-key tiles (S = 192): V is gathered
    straight into the tiled layout, and shard boundaries fall inside tiles."""
    H, B = 2 * N, 2
    spec = ShardSpec(S=N * L, N=N, H=H, d=d, dtype="bf16", mask=mask, B=B, cfg_id=203,
                     cu_seqlens=_small_cu(N * L) if mask == "doc_causal" else None)
    _every_rank(cp, spec, seed=4)


@pytest.mark.parametrize("N,L,H", [(1, 333, 2), (4, 70, 4), (8, 40, 8)])
def test_degenerate_groups(cp, N, L, H):
    """One rank (plain attention of one shard), and one head per rank."""
    spec = ShardSpec(S=N * L, N=N, H=H, d=128, dtype="bf16", mask="causal", B=1, cfg_id=202)
    _every_rank(cp, spec, seed=3)


def test_full_size_128k(cp):
    """The 128K example regrouped over 4 ranks: ranks 0 and 3 (heads 0-7 and
    24-31 of 32, S = 131072), sampled rows of every shard."""
    spec = ShardSpec(S=131072, N=4, H=32, d=128, dtype="bf16", mask="causal", B=1, cfg_id=3)
    q, k, v = _shards(spec, 0)
    qd, kd, vd = ([dev(x, "bf16") for x in t] for t in (q, k, v))
    od = [torch.full(spec.shard_shape(), SENTINEL, dtype=torch.bfloat16, device="cuda") for _ in range(spec.N)]
    hn = spec.H // spec.N
    for r in (0, 3):
        say(f"[ulysses full 128K] rank {r}")
        m, l, lse = run_rank(cp, spec, r, qd, kd, vd, od)
        heads = [r * hn, r * hn + 5]
        for i in range(spec.N):
            rows = sample_rows(spec.L, 40 + i, n_random=24)
            ref = oracle.rank_attention(q[i], k, v, i, spec.N, spec.mask, rows=rows, heads=heads)
            o = host(od[i][:, torch.from_numpy(rows).cuda()][:, :, heads])
            stats = check_o(o, ref["o"], "bf16", what=f"o shard {i}")
            pos = i * spec.L + rows
            hl = [h - r * hn for h in heads]
            check_stat(lse[:, hl][:, :, pos], ref["lse"], "bf16", "lse")
            check_stat(m[:, hl][:, :, pos], ref["m"], "bf16", "m")
            check_stat(l[:, hl][:, :, pos], ref["l"], "bf16", "l")
            say(f"[ulysses full 128K] rank {r} shard {i}: {len(rows)} rows x {len(heads)} heads {stats}")
        assert np.all(np.isfinite(lse)) and np.all(np.isfinite(m))
