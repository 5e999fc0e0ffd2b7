"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs (bf16 inputs are handed to the oracle as the same
bf16-rounded values).  Tolerances are in tests/gpu_util.py.

Small cases span several query and key tiles with ragged tails (L not a
multiple of any tile), batch > 1, every mask, both head dims and both input
types, and are checked element by element on every rank.  The full-size
workloads run in the launch configuration the benchmark times and are
checked on sampled rows that the oracle computes one by one.
"""
import numpy as np
import pytest

import oracle
from harness.inputs import (TENSOR_K, TENSOR_Q, TENSOR_V, ShardSpec, draw_shard, make_inputs,
                            normal_block, shuffled_order, standard_configs)
from tests.gpu_util import check_o, check_stat, dev, host, pooled_map, pooled_rows, sample_rows, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_ring_attention_cp_amd as cp
    cp.lib()     # raises if the library is not built: no fallback
    return cp


def _desc(cp, spec, rank, cu_dev=None, scale=0.0):
    return cp.Desc(spec.B, spec.H, spec.d, spec.N, spec.L, rank, spec.dtype, spec.mask,
                   cu_seqlens=spec.cu_seqlens, cu_seqlens_dev=cu_dev, scale=scale)


def _outs(spec):
    big = (spec.B, spec.L, spec.H, spec.d)
    vec = (spec.B, spec.H, spec.L)
    dt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    return (torch.full(big, float("nan"), dtype=dt, device="cuda"),
            torch.full(vec, float("nan"), device="cuda"), torch.full(vec, float("nan"), device="cuda"),
            torch.full(vec, float("nan"), device="cuda"))


def run_rank(cp, spec, rank, q, kb, vb, flags, scale=0.0):
    """cp_attn_rank_forward on a fresh compute/copy stream pair."""
    cu_dev = None
    if spec.mask == "doc_causal":
        cu_dev = torch.from_numpy(np.asarray(spec.cu_seqlens, np.int32)).cuda()
    d = _desc(cp, spec, rank, cu_dev, scale)
    out, m, l, lse = _outs(spec)
    ws = cp.alloc_workspace(d)
    cs, xs = torch.cuda.Stream(), torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        cp.cp_attn_rank_forward(d, q, kb, vb, out, m, l, lse, workspace=ws, compute_stream=cs,
                                copy_stream=xs, flags=flags)
    cs.synchronize()
    torch.cuda.synchronize()
    return host(out), host(m), host(l), host(lse)


def _check_all(got, ref, dtype, rows=None, heads=None, rounding_floor=False):
    o, m, l, lse = got
    if rows is not None:
        o = o[:, rows][:, :, heads]
        m, l, lse = (x[:, heads][:, :, rows] for x in (m, l, lse))
    stats = check_o(o, ref["o"], dtype, rounding_floor=rounding_floor)
    check_stat(m, ref["m"], dtype, "m")
    check_stat(l, ref["l"], dtype, "l")
    check_stat(lse, ref["lse"], dtype, "lse")
    return stats


def _blocks(spec, inp):
    return [dev(inp["k"][j], spec.dtype) for j in range(spec.N)], [dev(inp["v"][j], spec.dtype) for j in range(spec.N)]


# ----------------------------------------------------------------------------
# small cases, every rank, element by element


def test_tiny_fp32_ring_all_ranks(cp):
    """Four simulated ranks of S=1024 (H=2, d=64, fp32, causal) together give
    full attention over the sequence."""
    spec = standard_configs()[1]
    inp = make_inputs(spec, seed=0, ranks=range(spec.N))
    kb, vb = _blocks(spec, inp)
    for r in range(spec.N):
        say(f"[tiny fp32] rank {r}")
        got = run_rank(cp, spec, r, dev(inp["q"][r], "f32"), kb, vb, cp.CP_RING_PREFETCH)
        ref = oracle.rank_attention(inp["q"][r], inp["k"], inp["v"], r, spec.N, spec.mask)
        _check_all(got, ref, "f32")


def _small_cu(S):
    pts, x = [0], 0
    for n in (37, 130, 5, 300, 64, 1, 211, 90, 400):
        x += n
        if x >= S:
            break
        pts.append(x)
    return np.asarray(pts + [S], np.int32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", ["none", "causal", "doc_causal"])
def test_small_every_rank(cp, dtype, d, mask):
    N, L, H, B = 3, 300, 2, 2
    spec = ShardSpec(S=N * L, N=N, H=H, d=d, dtype=dtype, mask=mask, B=B, cfg_id=101,
                     cu_seqlens=_small_cu(N * L) if mask == "doc_causal" else None)
    inp = make_inputs(spec, seed=1, ranks=range(N))
    kb, vb = _blocks(spec, inp)
    for r in range(N):
        say(f"[small] dtype={dtype} d={d} mask={mask} rank={r}")
        got = run_rank(cp, spec, r, dev(inp["q"][r], dtype), kb, vb, cp.CP_RING_PREFETCH)
        ref = oracle.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, mask, spec.cu_seqlens)
        _check_all(got, ref, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_partial_modes_and_merge(cp, dtype):
    """INIT / ACCUMULATE + finalize reproduce the rank's attention; each
    PARTIAL_LSE block matches the oracle's per-block partial (including rows
    with no visible key: lse = -inf, O = 0); merge_lse in a shuffled order
    reproduces the rank's attention."""
    N, L, H, d = 4, 200, 3, 128
    spec = ShardSpec(S=N * L, N=N, H=H, d=d, dtype=dtype, mask="doc_causal", cfg_id=102,
                     cu_seqlens=np.asarray([0, 90, 333, 450, 600, 601, 800], np.int32))
    r = 2
    inp = make_inputs(spec, seed=2, ranks=[r])
    cu_dev = torch.from_numpy(spec.cu_seqlens).cuda()
    desc = _desc(cp, spec, r, cu_dev)
    q = dev(inp["q"][r], dtype)
    kb, vb = _blocks(spec, inp)
    big, vec = (1, L, H, d), (1, H, L)
    ref = oracle.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, spec.mask, spec.cu_seqlens)

    say(f"[modes] {dtype} init/accumulate/finalize")
    st = (torch.zeros(big, device="cuda"), torch.zeros(vec, device="cuda"), torch.zeros(vec, device="cuda"))
    for t, j in enumerate([2, 0, 3, 1]):
        cp.cp_attn_block_partial(desc, j, cp.CP_MODE_INIT if t == 0 else cp.CP_MODE_ACCUMULATE, q, kb[j], vb[j],
                                 state=st)
    out, m, l, lse = _outs(spec)
    cp.cp_attn_finalize(desc, st, out, m, l, lse)
    torch.cuda.synchronize()
    _check_all((host(out), host(m), host(l), host(lse)), ref, dtype)

    say(f"[modes] {dtype} partial_lse + merge")
    o_parts, lse_parts = [], []
    for j in range(N):
        op = torch.full(big, float("nan"), device="cuda")
        lp = torch.full(vec, float("nan"), device="cuda")
        cp.cp_attn_block_partial(desc, j, cp.CP_MODE_PARTIAL_LSE, q, kb[j], vb[j], o_part=op, lse_part=lp)
        torch.cuda.synchronize()
        bref = oracle.block_partial(inp["q"][r], inp["k"][j], inp["v"][j], r, j, N, spec.mask, spec.cu_seqlens)
        check_o(host(op), bref["o"], dtype, what=f"o_part[{j}]")
        check_stat(host(lp), bref["lse"], dtype, "lse")
        o_parts.append(op)
        lse_parts.append(lp)
    out, _, _, lse = _outs(spec)
    cp.cp_attn_merge_lse(desc, o_parts, lse_parts, [3, 1, 0, 2], out, lse)
    torch.cuda.synchronize()
    check_o(host(out), ref["o"], dtype)
    check_stat(host(lse), ref["lse"], dtype, "lse")


def test_prefetch_and_direction(cp):
    """Prefetch on/off give bit-identical results (same kernels, same order);
    the reversed ring order agrees within tolerance."""
    spec = ShardSpec(S=4 * 512, N=4, H=2, d=128, dtype="bf16", mask="causal", cfg_id=103)
    inp = make_inputs(spec, seed=3, ranks=[3])
    kb, vb = _blocks(spec, inp)
    q = dev(inp["q"][3], "bf16")
    say("[ring] prefetch on/off, reverse")
    a = run_rank(cp, spec, 3, q, kb, vb, cp.CP_RING_PREFETCH)
    b = run_rank(cp, spec, 3, q, kb, vb, 0)
    c = run_rank(cp, spec, 3, q, kb, vb, cp.CP_RING_PREFETCH | cp.CP_RING_REVERSE)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    ref = oracle.rank_attention(inp["q"][3], inp["k"], inp["v"], 3, 4, "causal")
    _check_all(c, ref, "bf16")


@pytest.mark.parametrize("flags", ["forward", "reverse"])
def test_document_rows_per_step(cp, flags):
    """Under the document mask each step runs only the shard rows that see
    its block (a prefix of the shard), and a row stores its final output at
    the last step that sees it.  Documents spanning several blocks make the
    prefixes differ per block; in the reverse ring order they grow from step
    to step instead of shrinking.  Every rank of a 5-block ring of ragged
    shards (L = 200, rows in several query tiles), against the oracle, with
    the ring prefetch on and off bit-identical."""
    N, L, H, d = 5, 200, 2, 128
    cu = np.asarray([0, 150, 330, 333, 620, 1000], np.int32)   # documents across 1, 2 and 3 blocks
    spec = ShardSpec(S=N * L, N=N, H=H, d=d, dtype="bf16", mask="doc_causal", cfg_id=110, cu_seqlens=cu)
    inp = make_inputs(spec, seed=11, ranks=range(N))
    kb, vb = _blocks(spec, inp)
    fl = cp.CP_RING_REVERSE if flags == "reverse" else 0
    for r in range(N):
        say(f"[document rows] {flags} rank {r}")
        got = run_rank(cp, spec, r, dev(inp["q"][r], "bf16"), kb, vb, fl | cp.CP_RING_PREFETCH)
        serial = run_rank(cp, spec, r, dev(inp["q"][r], "bf16"), kb, vb, fl)
        for x, y in zip(got, serial):
            assert np.array_equal(x, y)
        ref = oracle.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, "doc_causal", cu)
        _check_all(got, ref, "bf16")


@pytest.mark.parametrize("L,d,B", [(1000, 128, 1), (1243, 128, 1), (1243, 64, 1), (1243, 128, 2)])
def test_key_split_diagonal(cp, L, d, B):
    """A causal shard whose diagonal launch fills the chip at most once runs
    the upper half of its query tiles as two workgroups each (the keys before
    and after the split point), and the next ring step merges the two running
    states.  An even (4) and an odd, ragged (5) number of query tiles, both
    ring directions, every rank with a step after the diagonal, against the
    oracle; prefetch on and off bit-identical.  The workspace holds the side
    state exactly where the split applies."""
    N, H = 3, 3
    spec = ShardSpec(S=N * L, N=N, H=H, d=d, dtype="bf16", mask="causal", B=B, cfg_id=140)
    inp = make_inputs(spec, seed=13, ranks=range(N))
    kb, vb = _blocks(spec, inp)
    side = B * (4 * L * H * d + 2 * 4 * H * L)
    base = cp.cp_attn_workspace_bytes(cp.Desc(B, H, d, N, L, 1, "bf16", "none"))
    assert cp.cp_attn_workspace_bytes(_desc(cp, spec, 1)) >= base + side
    assert cp.cp_attn_workspace_bytes(_desc(cp, spec, 0)) == base      # one step: no split
    for r in range(1, N):
        for fl, name in ((0, "forward"), (cp.CP_RING_REVERSE, "reverse")):
            say(f"[key split] L={L} d={d} B={B} rank {r} {name}")
            q = dev(inp["q"][r], "bf16")
            got = run_rank(cp, spec, r, q, kb, vb, fl | cp.CP_RING_PREFETCH)
            serial = run_rank(cp, spec, r, q, kb, vb, fl)
            for x, y in zip(got, serial):
                assert np.array_equal(x, y)
            ref = oracle.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, "causal")
            _check_all(got, ref, "bf16")


@pytest.mark.parametrize("mask", ["causal", "doc_causal"])
def test_invisible_blocks_are_never_read(cp, mask):
    """Blocks the schedule skips are filled with NaN: outputs stay finite and
    bit-identical to a run with ordinary data there."""
    N, L = 4, 256
    cu = np.asarray([0, 100, 700, 900, 1024], np.int32)
    spec = ShardSpec(S=N * L, N=N, H=2, d=128, dtype="bf16", mask=mask, cfg_id=104,
                     cu_seqlens=cu if mask == "doc_causal" else None)
    r = 3 if mask == "doc_causal" else 1
    inp = make_inputs(spec, seed=4, ranks=[r])
    kb, vb = _blocks(spec, inp)
    q = dev(inp["q"][r], "bf16")
    visited = set(oracle.ring_schedule(N, r, L, mask, spec.cu_seqlens))
    assert len(visited) < N
    say(f"[poison] {mask} rank {r} visits {sorted(visited)}")
    a = run_rank(cp, spec, r, q, kb, vb, cp.CP_RING_PREFETCH)
    kp = [k if j in visited else torch.full_like(k, float("nan")) for j, k in enumerate(kb)]
    vp = [v if j in visited else torch.full_like(v, float("nan")) for j, v in enumerate(vb)]
    b = run_rank(cp, spec, r, q, kp, vp, cp.CP_RING_PREFETCH)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    ref = oracle.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, mask, spec.cu_seqlens)
    _check_all(a, ref, "bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_degenerate_shapes(cp, dtype):
    """L = 1 with N = 1 (one key: O = v_0), L = 1 with N = 5, an odd L with a
    non-default softmax scale."""
    for N, L, H, mask, scale in ((1, 1, 1, "causal", 0.0), (5, 1, 3, "causal", 0.0), (2, 77, 1, "none", 0.3),
                                 (1, 129, 2, "causal", 0.05)):
        say(f"[degenerate] {dtype} N={N} L={L} H={H} {mask} scale={scale}")
        spec = ShardSpec(S=N * L, N=N, H=H, d=64, dtype=dtype, mask=mask, cfg_id=105)
        inp = make_inputs(spec, seed=5, ranks=range(N))
        kb, vb = _blocks(spec, inp)
        for r in range(N):
            got = run_rank(cp, spec, r, dev(inp["q"][r], dtype), kb, vb, cp.CP_RING_PREFETCH, scale=scale)
            ref = oracle.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, mask,
                                        scale=scale if scale > 0 else None)
            _check_all(got, ref, dtype, rounding_floor=(L == 1))
    spec = ShardSpec(S=1, N=1, H=1, d=64, dtype=dtype, mask="causal", cfg_id=106)
    inp = make_inputs(spec, seed=6, ranks=[0])
    kb, vb = _blocks(spec, inp)
    o, m, l, lse = run_rank(cp, spec, 0, dev(inp["q"][0], dtype), kb, vb, 0)
    assert np.allclose(o[0, 0, 0], inp["v"][0][0, 0, 0], atol=1e-2 if dtype == "bf16" else 1e-6)
    assert abs(l[0, 0, 0] - 1.0) < 1e-6


# ----------------------------------------------------------------------------
# full-size workloads, sampled rows


def _full_inputs(spec, seed, blocks):
    q = draw_shard(spec, seed, TENSOR_Q, spec.rank)
    k = {j: draw_shard(spec, seed, TENSOR_K, j) for j in blocks}
    v = {j: draw_shard(spec, seed, TENSOR_V, j) for j in blocks}
    return q, k, v


def _heads(spec, seed):
    rng = np.random.default_rng(seed + 17)
    return sorted({0, spec.H - 1, int(rng.integers(spec.H))})


def _oracle_whole_head(spec, q, k, v, h):
    """The definition for every row of head h of a B = 1 shard, in row chunks
    on a thread pool: O [1, L, 1, d] and m, l, lse [1, 1, L]."""
    blocks = sorted(k)
    K = np.concatenate([k[j][0, :, h, :] for j in blocks]).astype(np.float64)
    V = np.concatenate([v[j][0, :, h, :] for j in blocks]).astype(np.float64)
    c = np.concatenate([np.arange(j * spec.L, (j + 1) * spec.L, dtype=np.int64) for j in blocks])

    def part(rows):
        return oracle.attention_rows(q[0, rows, h, :], K, V, spec.rank * spec.L + rows, c, spec.mask,
                                     spec.cu_seqlens)

    parts = pooled_rows(part, spec.L)
    o = np.concatenate([x[0] for x in parts])[None, :, None, :]
    m, l, lse = (np.concatenate([x[i] for x in parts])[None, None, :] for i in (1, 2, 3))
    return {"o": o, "m": m, "l": l, "lse": lse}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_full_size_rank_forward(cp, cfg):
    """The causal 32K and 128K last-rank shards and the packed-document shard
    at full size, ring prefetch on: one whole head element by element, and in
    every head the first and last row of every 256-row query tile plus rows
    at document boundaries and a seeded random set, against the oracle."""
    spec = standard_configs(seed=0)[cfg]
    blocks = oracle.ring_schedule(spec.N, spec.rank, spec.L, spec.mask, spec.cu_seqlens)
    say(f"[full cfg {cfg}] {spec.name}: blocks {blocks}")
    q, k, v = _full_inputs(spec, 0, blocks)
    kb = [dev(k[j], "bf16") if j in k else None for j in range(spec.N)]
    vb = [dev(v[j], "bf16") if j in v else None for j in range(spec.N)]
    got = run_rank(cp, spec, spec.rank, dev(q, "bf16"), kb, vb, cp.CP_RING_PREFETCH)
    for arr in got:
        assert np.all(np.isfinite(arr))

    h = int(np.random.default_rng(100 + cfg).integers(spec.H))
    say(f"[full cfg {cfg}] oracle: all {spec.L} rows of head {h}")
    ref = _oracle_whole_head(spec, q, k, v, h)
    stats = _check_all(got, ref, "bf16", rows=np.arange(spec.L), heads=[h])
    say(f"[full cfg {cfg}] whole head {h}: {stats}")

    extra = [t * 256 for t in range((spec.L + 255) // 256)] + [min(t * 256 + 255, spec.L - 1)
                                                                for t in range((spec.L + 255) // 256)]
    if spec.cu_seqlens is not None:
        s0 = spec.rank * spec.L
        for x in spec.cu_seqlens:
            if s0 <= x < s0 + spec.L:
                extra += [x - s0 - 1, x - s0, x - s0 + 1]
    rows = sample_rows(spec.L, cfg, n_random=64, extra=extra)
    say(f"[full cfg {cfg}] oracle: {len(rows)} rows x {spec.H} heads")
    per_head = pooled_map(lambda hh: oracle.rank_attention(q, k, v, spec.rank, spec.N, spec.mask, spec.cu_seqlens,
                                                           rows=rows, heads=[hh]), range(spec.H))
    ref = {key: np.concatenate([x[key] for x in per_head], axis=2 if key == "o" else 1) for key in per_head[0]}
    stats = _check_all(got, ref, "bf16", rows=rows, heads=list(range(spec.H)))
    say(f"[full cfg {cfg}] {len(rows)} rows x {spec.H} heads: {stats}")


@pytest.mark.parametrize("nqt", [512, 516])
def test_document_order_at_and_past_its_table(cp, nqt):
    """Under the document mask the host passes a launch's query-tile order
    (by decreasing work) in the launch arguments, for up to 512 query tiles;
    a launch with more tiles runs them in index order.  A 2-block ring of
    ragged shards of exactly 512 and of 516 query tiles (L = 256 nqt - 37),
    one head, documents of 500-9000 tokens, rank 1 with prefetch: sampled
    rows (tile edges, document edges, a seeded set) against the oracle."""
    N, H, d = 2, 1, 64
    L = 256 * nqt - 37
    S = N * L
    rng = np.random.default_rng(41 + nqt)
    pts = [0]
    while pts[-1] < S:
        pts.append(pts[-1] + int(rng.integers(500, 9000)))
    cu = np.asarray(pts[:-1] + [S], np.int32)
    spec = ShardSpec(S=S, N=N, H=H, d=d, dtype="bf16", mask="doc_causal", rank=1, cfg_id=141, cu_seqlens=cu)
    blocks = [0, 1]
    q, k, v = _full_inputs(spec, 0, blocks)
    kb = [dev(k[j], "bf16") for j in blocks]
    vb = [dev(v[j], "bf16") for j in blocks]
    say(f"[document order] {nqt} query tiles, L={L}, {len(cu) - 1} documents")
    got = run_rank(cp, spec, 1, dev(q, "bf16"), kb, vb, cp.CP_RING_PREFETCH)
    extra = [t * 256 for t in range(nqt)][::16] + [x - L for x in cu if L <= x < 2 * L]
    rows = sample_rows(L, nqt, n_random=96, extra=extra)
    ref = oracle.rank_attention(q, k, v, 1, N, "doc_causal", cu, rows=rows, heads=[0])
    stats = _check_all(got, ref, "bf16", rows=rows, heads=[0])
    say(f"[document order] {len(rows)} rows: {stats}")


def test_full_size_partial_merge(cp):
    """Bidirectional 64K over 8 ranks, rank 5, Q x 3: eight PARTIAL_LSE
    blocks, then merge_lse in a seeded shuffled order; sampled rows."""
    spec = standard_configs(seed=0)[4]
    say(f"[full cfg 4] {spec.name}")
    q, k, v = _full_inputs(spec, 0, range(spec.N))
    desc = _desc(cp, spec, spec.rank)
    qd = dev(q, "bf16")
    big, vec = (1, spec.L, spec.H, spec.d), (1, spec.H, spec.L)
    o_parts, lse_parts = [], []
    for j in range(spec.N):
        kd, vd = dev(k[j], "bf16"), dev(v[j], "bf16")
        op = torch.empty(big, device="cuda")
        lp = torch.empty(vec, device="cuda")
        cp.cp_attn_block_partial(desc, j, cp.CP_MODE_PARTIAL_LSE, qd, kd, vd, o_part=op, lse_part=lp)
        o_parts.append(op)
        lse_parts.append(lp)
    order = shuffled_order(0, 4, spec.N)
    out, _, _, lse = _outs(spec)
    cp.cp_attn_merge_lse(desc, o_parts, lse_parts, order, out, lse)
    torch.cuda.synchronize()
    rows = sample_rows(spec.L, 4)
    heads = _heads(spec, 4)
    ref = oracle.rank_attention(q, k, v, spec.rank, spec.N, spec.mask, rows=rows, heads=heads)
    o = host(out)[:, rows][:, :, heads]
    stats = check_o(o, ref["o"], "bf16")
    check_stat(host(lse)[:, heads][:, :, rows], ref["lse"], "bf16", "lse")
    say(f"[full cfg 4] order {order}: {stats}")


# ----------------------------------------------------------------------------
# API corners


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_merge_and_finalize_many_heads(cp, dtype):
    """merge_lse and finalize with B * H = 80000 (batch, head) pairs and a
    4-row shard: their 1-D grids walk (batch, row, head) in memory order, so
    no grid extent bounds B * H.  Checked on sampled heads of both batches."""
    N, L, H, d, B, r = 2, 4, 40000, 64, 2, 1
    spec = ShardSpec(S=N * L, N=N, H=H, d=d, dtype=dtype, mask="none", B=B, cfg_id=108)
    inp = make_inputs(spec, seed=9, ranks=[r])
    desc = _desc(cp, spec, r)
    q = dev(inp["q"][r], dtype)
    kb, vb = _blocks(spec, inp)
    heads = [0, 1, 20011, H - 1]
    ref = oracle.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, "none", heads=heads)
    big, vec = (B, L, H, d), (B, H, L)

    say(f"[many heads] {dtype} partial_lse + merge")
    o_parts, lse_parts = [], []
    for j in range(N):
        op = torch.full(big, float("nan"), device="cuda")
        lp = torch.full(vec, float("nan"), device="cuda")
        cp.cp_attn_block_partial(desc, j, cp.CP_MODE_PARTIAL_LSE, q, kb[j], vb[j], o_part=op, lse_part=lp)
        o_parts.append(op)
        lse_parts.append(lp)
    out, _, _, lse = _outs(spec)
    cp.cp_attn_merge_lse(desc, o_parts, lse_parts, [1, 0], out, lse)
    torch.cuda.synchronize()
    check_o(host(out)[:, :, heads], ref["o"], dtype)
    check_stat(host(lse)[:, heads], ref["lse"], dtype, "lse")
    del o_parts, lse_parts

    say(f"[many heads] {dtype} init/accumulate + finalize")
    st = (torch.zeros(big, device="cuda"), torch.zeros(vec, device="cuda"), torch.zeros(vec, device="cuda"))
    for t, j in enumerate([1, 0]):
        cp.cp_attn_block_partial(desc, j, cp.CP_MODE_INIT if t == 0 else cp.CP_MODE_ACCUMULATE, q, kb[j], vb[j],
                                 state=st)
    out, m, l, lse = _outs(spec)
    cp.cp_attn_finalize(desc, st, out, m, l, lse)
    torch.cuda.synchronize()
    _check_all((host(out)[:, :, heads], host(m)[:, heads], host(l)[:, heads], host(lse)[:, heads]), ref, dtype)


def test_merge_order_null_and_single_part(cp):
    """merge_lse with order = NULL sums in index order (bit-identical to the
    explicit identity order); with one part the output is that part."""
    N, L, H, d = 3, 160, 2, 64
    spec = ShardSpec(S=N * L, N=N, H=H, d=d, dtype="bf16", mask="none", cfg_id=107)
    inp = make_inputs(spec, seed=8, ranks=[1])
    desc = _desc(cp, spec, 1)
    q = dev(inp["q"][1], "bf16")
    big, vec = (1, L, H, d), (1, H, L)
    ops, lps = [], []
    for j in range(N):
        op = torch.empty(big, device="cuda")
        lp = torch.empty(vec, device="cuda")
        cp.cp_attn_block_partial(desc, j, cp.CP_MODE_PARTIAL_LSE, q, dev(inp["k"][j], "bf16"),
                                 dev(inp["v"][j], "bf16"), o_part=op, lse_part=lp)
        ops.append(op)
        lps.append(lp)
    a, la = _outs(spec)[0], torch.empty(vec, device="cuda")
    b, lb = _outs(spec)[0], torch.empty(vec, device="cuda")
    cp.cp_attn_merge_lse(desc, ops, lps, None, a, la)
    cp.cp_attn_merge_lse(desc, ops, lps, [0, 1, 2], b, lb)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    ref = oracle.rank_attention(inp["q"][1], inp["k"], inp["v"], 1, N, "none")
    check_o(host(a), ref["o"], "bf16")
    check_stat(host(la), ref["lse"], "bf16", "lse")
    one, l1 = _outs(spec)[0], torch.empty(vec, device="cuda")
    cp.cp_attn_merge_lse(desc, ops[1:2], lps[1:2], None, one, l1)
    torch.cuda.synchronize()
    # the weight exp(lse_0 - lse) is 1 up to the rounding of lse * log2(e): at most one bf16 ulp apart
    assert torch.allclose(one.float(), ops[1], rtol=2.0 ** -8, atol=1e-6)
    assert torch.allclose(l1, lps[1], rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_invisible_block_through_block_partial(cp, dtype):
    """A block the rank never sees (causal, j > rank), called anyway: every
    row is empty - PARTIAL_LSE gives O = 0 and lse = -inf, INIT gives
    m = -inf, l = 0, O = 0."""
    N, L, H, d = 4, 96, 2, 128
    spec = ShardSpec(S=N * L, N=N, H=H, d=d, dtype=dtype, mask="causal", cfg_id=108)
    inp = make_inputs(spec, seed=9, ranks=[1])
    desc = _desc(cp, spec, 1)
    q = dev(inp["q"][1], dtype)
    k3, v3 = dev(inp["k"][3], dtype), dev(inp["v"][3], dtype)
    big, vec = (1, L, H, d), (1, H, L)
    op = torch.full(big, 7.0, device="cuda")
    lp = torch.full(vec, 7.0, device="cuda")
    cp.cp_attn_block_partial(desc, 3, cp.CP_MODE_PARTIAL_LSE, q, k3, v3, o_part=op, lse_part=lp)
    st = (torch.full(big, 7.0, device="cuda"), torch.full(vec, 7.0, device="cuda"), torch.full(vec, 7.0, device="cuda"))
    cp.cp_attn_block_partial(desc, 3, cp.CP_MODE_INIT, q, k3, v3, state=st)
    torch.cuda.synchronize()
    assert torch.all(op == 0) and torch.all(torch.isneginf(lp))
    assert torch.all(st[0] == 0) and torch.all(torch.isneginf(st[1])) and torch.all(st[2] == 0)


def test_profiler_records_each_launch_and_receive(cp):
    spec = ShardSpec(S=4 * 384, N=4, H=2, d=128, dtype="bf16", mask="causal", cfg_id=109)
    inp = make_inputs(spec, seed=10, ranks=[2])
    kb, vb = _blocks(spec, inp)
    desc = _desc(cp, spec, 2)
    out, m, l, lse = _outs(spec)
    ws = cp.alloc_workspace(desc)
    prof = cp.Profiler(8)
    cs, xs = torch.cuda.Stream(), torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    for _ in range(2):
        cp.cp_attn_rank_forward(desc, dev(inp["q"][2], "bf16"), kb, vb, out, m, l, lse, workspace=ws,
                                compute_stream=cs, copy_stream=xs, flags=cp.CP_RING_PREFETCH, profiler=prof)
    cs.synchronize()
    times = prof.read()
    assert len(times) == 6 and all(t > 0 for t in times)      # rank 2 visits blocks 2, 1, 0 per call
    copies = prof.read_copies()
    assert len(copies) == 4 and all(t > 0 for t in copies)    # blocks 1 and 0 are received per call
    prof.reset()
    assert prof.read() == [] and prof.read_copies() == []
    prof.close()


@pytest.mark.parametrize("N,d,mask", [(24, 64, "none"), (64, 128, "doc_causal")])
def test_many_parts_and_long_ring(cp, N, d, mask):
    """Rings of 24 and of CP_MAX_RING = 64 blocks of 16 tokens (every tile
    ragged): the PARTIAL_LSE partials of all blocks merged in a seeded shuffled
    order (more parts than the merge keeps in registers; under the document
    mask most parts are empty), and the prefetching rank forward over the whole
    ring, both against the oracle."""
    L, H = 16, 2
    spec = ShardSpec(S=N * L, N=N, H=H, d=d, dtype="bf16", mask=mask, cfg_id=108,
                     cu_seqlens=_small_cu(N * L) if mask == "doc_causal" else None)
    r = N // 2
    inp = make_inputs(spec, seed=9, ranks=[r])
    cu_dev = None
    if mask == "doc_causal":
        cu_dev = torch.from_numpy(np.asarray(spec.cu_seqlens, np.int32)).cuda()
    desc = _desc(cp, spec, r, cu_dev)
    q = dev(inp["q"][r], "bf16")
    kb, vb = _blocks(spec, inp)
    big, vec = (1, L, H, d), (1, H, L)
    ops = [torch.full(big, float("nan"), device="cuda") for _ in range(N)]
    lps = [torch.full(vec, float("nan"), device="cuda") for _ in range(N)]
    say(f"[long ring] N={N} d={d} mask={mask}: {N} partials")
    for j in range(N):
        cp.cp_attn_block_partial(desc, j, cp.CP_MODE_PARTIAL_LSE, q, kb[j], vb[j], o_part=ops[j], lse_part=lps[j])
    order = [int(x) for x in np.random.default_rng(N).permutation(N)]
    out = torch.full(big, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(vec, float("nan"), device="cuda")
    cp.cp_attn_merge_lse(desc, ops, lps, order, out, lse)
    torch.cuda.synchronize()
    ref = oracle.rank_attention(inp["q"][r], inp["k"], inp["v"], r, N, mask, spec.cu_seqlens)
    check_o(host(out), ref["o"], "bf16")
    check_stat(host(lse), ref["lse"], "bf16", "lse")
    say(f"[long ring] N={N}: rank forward")
    got = run_rank(cp, spec, r, q, kb, vb, cp.CP_RING_PREFETCH)
    _check_all(got, ref, "bf16")
