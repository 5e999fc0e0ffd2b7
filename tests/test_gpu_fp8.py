"""GPU parity of the FP8 (e4m3) path against the oracle (oracle/fp8.py).

Quantisation is byte work, so its bar is bit-exact: every code and every
float32 (power-of-two) scale equals the oracle's, in both roles (keys and
values; the query, multiplied by the softmax scale times log2(e) first, for
the default and a given softmax scale), on ragged lengths (L not a multiple
of the 256 rows a workgroup covers), both head dims, heads of very different
magnitudes, an all-zero head, and a full-size 128K block (all scales, codes
of sampled rows).

The FP8 shard forward is compared with the oracle's float64 attention on the
dequantised inputs (the oracle quantises the same bf16 draws itself, the
query with its base-2 factor).  The kernel takes P = exp2(x - m_ref) two
ways: exp2 of the logit with the conversion dividing by 2^m_ref, or, when a
reference leaves the range where that is exact, exp2 of x - m_ref; logits
hundreds of units above or below zero drive the second way
(test_fp8_forward_logit_range).  The tolerance follows from the arithmetic of
the kernel:
  * scores: products of two e4m3 values are exact in float32 and are summed
    over at most 128 head dims in float32 (the power-of-two scales are
    exact), so each score, and with it m (the row max), differs from the
    oracle's by float32 rounding of at most 128 * 2^-24 = 2^-17 of the sum of
    the products' magnitudes.  That sum is bounded per row, for every key the
    row sees, by A = scale * sum_d |q_d| max_k |k_d| (the maximum over all
    keys of the supplied blocks, from the dequantised inputs); it can exceed
    |m| many times over (a row of one visible key whose score is near zero).
    Bound: max-abs 2e-3 + 2^-17 A + 2^-20 |m| (the bf16 path's 2e-3; the last
    term covers log2(e) and ln(2) rounded to float32);
  * P = exp(s - m_ref) is rounded to e4m3 before the P V product and l sums
    the same rounded values.  A normal e4m3 value is within 2^-4 (half of the
    3-bit mantissa's ulp) of its argument, relative; over a log-uniform
    spread of P the rms relative error is 2^-4 / sqrt(3) * sqrt(0.541) =
    0.0266.  Hence l: relative error at most 2^-4 plus the values below the
    smallest normal (absolute error <= 2^-10 of the row max each, negligible
    against l >= 1): bound 0.07; lse = m + log l: max-abs 0.07 plus m's bound;
  * O = sum rho(p_k) v_k / sum rho(p_k): the error is
    sum (rho(p_k) - p_k)(v_k - O) / sum rho(p_k), so over many elements its rms
    is about 0.0266 of the rms of O itself: bound rms(err) <= 0.045 rms(O_ref).
    A row with two keys of weights 1 and x errs at most
    2^-4 x / (1 + x)^2 |v_1 - v_0| <= 2^-6 * 9 for |v| <= 4.5: max-abs 0.15;
    mean-abs 1e-2.
A mistake in the operand layouts (a key of P paired with the wrong V row, a
head dim dropped, a scale missed) moves O by about its own size (relative rms
near 1) and m or l far beyond these bounds.
"""
import numpy as np
import pytest

import oracle
import oracle.fp8 as F
from harness.inputs import (TENSOR_K, TENSOR_Q, TENSOR_V, ShardSpec, draw_shard, make_inputs, round_to_bf16,
                            standard_configs)
from tests.gpu_util import dev, host, sample_rows, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_ring_attention_cp_amd as cp
    cp.lib()     # raises if the library is not built: no fallback
    return cp


def _quantize_gpu(cp, x, d, role=None, scale=0.0):
    B, L, H, _ = x.shape
    desc = cp.Desc(B, H, d, 1, L, 0, "bf16", "none", scale=scale)
    codes = torch.empty((B, L, H, d), dtype=torch.uint8, device="cuda")
    scales = torch.full((B, H), float("nan"), device="cuda")
    cp.cp_attn_quantize_fp8(desc, dev(x, "bf16"), codes, scales, role=cp.CP_FP8_KV if role is None else role)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


@pytest.mark.parametrize("role", ["kv", "query", "query_scale"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L", [1, 300, 513])
def test_quantize_bit_exact(cp, d, L, role):
    rng = np.random.default_rng(L + d)
    x = rng.standard_normal((2, L, 4, d)).astype(np.float32) * np.array([1.0, 1e-3, 50.0, 1.0], np.float32)[None, None, :, None]
    x[1, :, 3, :] = 0.0                                   # one all-zero (b, h)
    x[0, 0, 0, :4] = [0.0, -0.0, 1e-30, -1e-30]           # zeros and values far below the smallest code
    x = round_to_bf16(x)
    say(f"[fp8 quantize] L={L} d={d} role={role}")
    sm = 0.3 if role == "query_scale" else 0.0
    c = 1.0 if role == "kv" else F.query_prescale(d, sm)
    codes, scales = _quantize_gpu(cp, x, d, cp.CP_FP8_KV if role == "kv" else cp.CP_FP8_QUERY, sm)
    ref = F.quantize_heads(x, c)
    assert np.array_equal(scales.view(np.uint32), ref["scale"].view(np.uint32)), "scales differ"
    bad = np.argwhere(codes != ref["codes"])
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0].tolist()}: gpu {codes[tuple(bad[0])]:#x} " \
                          f"oracle {ref['codes'][tuple(bad[0])]:#x}"


def test_quantize_full_size_block(cp):
    """One K block of the 128K example (L = 32768, H = 32, d = 128) and the
    same draws as a query: every scale, and the codes of sampled rows."""
    spec = ShardSpec(S=131072, N=4, H=32, d=128, dtype="bf16", mask="causal", cfg_id=3)
    x = draw_shard(spec, 0, TENSOR_K, 2)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 32767], np.random.default_rng(5).integers(0, 32768, 64)]))
    for role in (cp.CP_FP8_KV, cp.CP_FP8_QUERY):
        say(f"[fp8 quantize full] role={role}")
        c = np.float32(1.0) if role == cp.CP_FP8_KV else F.query_prescale(128)
        codes, scales = _quantize_gpu(cp, x, 128, role)
        # the oracle's steps on the whole block for the scales, on the sampled rows for the codes
        amax = np.abs((x * c).astype(np.float32)).max(axis=(1, 3))
        e = F.scale_exponent(amax)
        assert np.array_equal(scales.view(np.uint32), np.exp2(e).astype(np.float32).view(np.uint32)), "scales differ"
        ref = F.quantize_heads(x[:, rows], c)          # codes only: its scales are those of the sampled rows
        y = (x[:, rows] * c).astype(np.float32).astype(np.float64) * np.exp2(-e.astype(np.float64))[:, None, :, None]
        assert np.array_equal(codes[:, rows], F.e4m3_encode(np.clip(y, -448, 448))), "codes of sampled rows differ"
        del ref


# ----------------------------------------------------------------------------
# the shard forward on e4m3 inputs

FP8_TOL = dict(o_max=0.15, o_mean=1e-2, o_rel_rms=0.045, m_abs=2e-3, m_acc=2.0 ** -17, m_rel=2.0 ** -20, l_rel=0.07,
               lse_abs=0.07)


def _product_bound(spec, qz, kz, rows=None, scale=None):
    """A [B, H, rows] (natural-log units): scale * sum_d |q_d| max_k |k_d| over
    the keys of the supplied blocks, a bound on the sum of the magnitudes of
    one score's products, from the dequantised inputs (softmax scale
    1/sqrt(d) unless given)."""
    q = np.abs(F.dequantize_heads(qz["codes"], qz["scale"], F.query_prescale(spec.d, scale)))   # [B, L, H, d]
    if rows is not None:
        q = q[:, rows]
    kmax = np.max([np.abs(F.dequantize_heads(z["codes"], z["scale"])).max(axis=1) for z in kz if z is not None],
                  axis=0)                                                                  # [B, H, d]
    sm = scale if scale else 1.0 / np.sqrt(spec.d)
    return np.einsum("blhd,bhd->bhl", q, kmax) * sm


def _codes_dev(q):
    """oracle codes and scales -> device uint8 codes and float32 scales."""
    return (torch.from_numpy(np.ascontiguousarray(q["codes"])).cuda(),
            torch.from_numpy(np.ascontiguousarray(q["scale"], dtype=np.float32)).cuda())


def _run_fp8(cp, spec, rank, qc, qs, kc, ks, vc, vs, flags):
    cu_dev = None
    if spec.mask == "doc_causal":
        cu_dev = torch.from_numpy(np.asarray(spec.cu_seqlens, np.int32)).cuda()
    d = cp.Desc(spec.B, spec.H, spec.d, spec.N, spec.L, rank, "bf16", spec.mask,
                cu_seqlens=spec.cu_seqlens, cu_seqlens_dev=cu_dev)
    big, vec = (spec.B, spec.L, spec.H, spec.d), (spec.B, spec.H, spec.L)
    out = torch.full(big, float("nan"), dtype=torch.bfloat16, device="cuda")
    m, l, lse = (torch.full(vec, float("nan"), device="cuda") for _ in range(3))
    ws = cp.alloc_workspace(d)
    cs, xs = torch.cuda.Stream(), torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        cp.cp_attn_rank_forward_fp8(d, qc, qs, kc, ks, vc, vs, out, m, l, lse, workspace=ws, compute_stream=cs,
                                    copy_stream=xs, flags=flags)
    cs.synchronize()
    torch.cuda.synchronize()
    return host(out), host(m), host(l), host(lse)


def _check_fp8(got, ref, A, rows=None, heads=None):
    o, m, l, lse = got
    if rows is not None:
        o = o[:, rows][:, :, heads]
        m, l, lse = (x[:, heads][:, :, rows] for x in (m, l, lse))
    t = FP8_TOL
    r = ref["o"]
    assert o.shape == r.shape and np.all(np.isfinite(o)), "o: shape or non-finite"
    err = np.abs(o - r)
    stats = {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
             "rel_rms": float(np.sqrt(np.mean(err ** 2)) / max(np.sqrt(np.mean(r ** 2)), 1e-30))}
    assert stats["max_abs"] <= t["o_max"], f"o: max-abs {stats}"
    assert stats["mean_abs"] <= t["o_mean"], f"o: mean-abs {stats}"
    assert stats["rel_rms"] <= t["o_rel_rms"], f"o: relative rms {stats}"
    ninf = np.isneginf(ref["m"])
    for name, g in (("m", m), ("l", l), ("lse", lse)):
        assert np.array_equal(np.isneginf(g), np.isneginf(ref[name])), f"{name}: -inf pattern differs"
    r_m = ref["m"][~ninf]
    m_bound = t["m_abs"] + t["m_acc"] * A[~ninf] + t["m_rel"] * np.abs(r_m)
    stats["m"] = float(np.max(np.abs(m[~ninf] - r_m) / m_bound, initial=0.0))     # fraction of the bound
    assert stats["m"] <= 1.0, f"m: {stats}"
    stats["l"] = float(np.max(np.abs(l[~ninf] / ref["l"][~ninf] - 1), initial=0.0))
    assert stats["l"] <= t["l_rel"], f"l: {stats}"
    stats["lse"] = float(np.max(np.abs(lse[~ninf] - ref["lse"][~ninf]) / (t["lse_abs"] + m_bound), initial=0.0))
    assert stats["lse"] <= 1.0, f"lse: {stats}"
    return stats


def _quantized_inputs(spec, seed, ranks):
    inp = make_inputs(spec, seed=seed, ranks=ranks)
    c = F.query_prescale(spec.d)
    qz = {r: F.quantize_heads(inp["q"][r], c) for r in ranks}
    kz = [F.quantize_heads(inp["k"][j]) for j in range(spec.N)]
    vz = [F.quantize_heads(inp["v"][j]) for j in range(spec.N)]
    return qz, kz, vz


def _oracle_fp8(spec, rank, qz, kz, vz, rows=None, heads=None):
    return F.fp8_rank_attention(qz["codes"], qz["scale"], [z["codes"] for z in kz], [z["scale"] for z in kz],
                                [z["codes"] for z in vz], [z["scale"] for z in vz], rank, spec.N, spec.mask,
                                spec.cu_seqlens, rows=rows, heads=heads, q_prescale=F.query_prescale(spec.d))


def _small_cu(S):
    pts, x = [0], 0
    for n in (37, 130, 5, 300, 64, 1, 211, 90, 400):
        x += n
        if x >= S:
            break
        pts.append(x)
    return np.asarray(pts + [S], np.int32)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", ["none", "causal", "doc_causal"])
def test_fp8_forward_small_every_rank(cp, d, mask):
    """N = 3 shards of L = 300 (several 256-row query tiles and 64-key tiles,
    ragged tails), B = 2, H = 2: every rank, every output element."""
    N, L, H, B = 3, 300, 2, 2
    spec = ShardSpec(S=N * L, N=N, H=H, d=d, dtype="bf16", mask=mask, B=B, cfg_id=111,
                     cu_seqlens=_small_cu(N * L) if mask == "doc_causal" else None)
    qz, kz, vz = _quantized_inputs(spec, 2, range(N))
    kd = [_codes_dev(z) for z in kz]
    vd = [_codes_dev(z) for z in vz]
    for r in range(N):
        say(f"[fp8 fwd small] d={d} mask={mask} rank={r}")
        qc, qs = _codes_dev(qz[r])
        got = _run_fp8(cp, spec, r, qc, qs, [x[0] for x in kd], [x[1] for x in kd], [x[0] for x in vd],
                       [x[1] for x in vd], cp.CP_RING_PREFETCH)
        stats = _check_fp8(got, _oracle_fp8(spec, r, qz[r], kz, vz), _product_bound(spec, qz[r], kz))
        say(f"   {stats}")


@pytest.mark.parametrize("flags", ["serial", "reverse"])
def test_fp8_forward_ring_variants(cp, flags):
    """Copies on the compute stream, and the reversed ring order: same bound."""
    N, L = 4, 200
    spec = ShardSpec(S=N * L, N=N, H=3, d=128, dtype="bf16", mask="causal", cfg_id=112)
    qz, kz, vz = _quantized_inputs(spec, 3, [N - 1])
    kd = [_codes_dev(z) for z in kz]
    vd = [_codes_dev(z) for z in vz]
    qc, qs = _codes_dev(qz[N - 1])
    fl = 0 if flags == "serial" else cp.CP_RING_PREFETCH | cp.CP_RING_REVERSE
    say(f"[fp8 fwd ring] flags={flags}")
    got = _run_fp8(cp, spec, N - 1, qc, qs, [x[0] for x in kd], [x[1] for x in kd], [x[0] for x in vd],
                   [x[1] for x in vd], fl)
    _check_fp8(got, _oracle_fp8(spec, N - 1, qz[N - 1], kz, vz), _product_bound(spec, qz[N - 1], kz))


@pytest.mark.parametrize("L", [1, 65])
def test_fp8_forward_degenerate(cp, L):
    """One-token and 65-token shards, heads of very different magnitudes and
    an all-zero query head (scale 1, codes 0: uniform weights over the
    visible keys)."""
    N, H = 2, 4
    spec = ShardSpec(S=N * L, N=N, H=H, d=64, dtype="bf16", mask="causal", cfg_id=113)
    inp = make_inputs(spec, seed=4, ranks=range(N))
    mag_q = np.array([1.0, 1e-3, 20.0, 1.0], np.float32)[None, None, :, None]
    mag_k = np.array([1.0, 20.0, 20.0, 1.0], np.float32)[None, None, :, None]   # head 2: scores of std 400
    for r in range(N):
        inp["q"][r] = round_to_bf16(inp["q"][r] * mag_q)
        inp["q"][r][:, :, 3, :] = 0.0
    for j in range(N):
        inp["k"][j] = round_to_bf16(inp["k"][j] * mag_k)
    qz = {r: F.quantize_heads(inp["q"][r], F.query_prescale(spec.d)) for r in range(N)}
    kz = [F.quantize_heads(inp["k"][j]) for j in range(N)]
    vz = [F.quantize_heads(inp["v"][j]) for j in range(N)]
    kd = [_codes_dev(z) for z in kz]
    vd = [_codes_dev(z) for z in vz]
    for r in range(N):
        say(f"[fp8 fwd degenerate] L={L} rank={r}")
        qc, qs = _codes_dev(qz[r])
        got = _run_fp8(cp, spec, r, qc, qs, [x[0] for x in kd], [x[1] for x in kd], [x[0] for x in vd],
                       [x[1] for x in vd], cp.CP_RING_PREFETCH)
        _check_fp8(got, _oracle_fp8(spec, r, qz[r], kz, vz), _product_bound(spec, qz[r], kz))


def test_fp8_forward_given_scale(cp):
    """A softmax scale given in the desc (0.3 instead of 1/sqrt(d)): the query
    is quantised under that desc, with the scale folded into its codes, and
    the forward under the same desc matches the oracle's attention with that
    scale.  N = 2 shards of L = 200, causal, d = 64, H = 2, both ranks."""
    N, L, H, d, sm = 2, 200, 2, 64, 0.3
    spec = ShardSpec(S=N * L, N=N, H=H, d=d, dtype="bf16", mask="causal", cfg_id=115)
    inp = make_inputs(spec, seed=8, ranks=range(N))
    kz = [F.quantize_heads(inp["k"][j]) for j in range(N)]
    vz = [F.quantize_heads(inp["v"][j]) for j in range(N)]
    kd = [_codes_dev(z) for z in kz]
    vd = [_codes_dev(z) for z in vz]
    for r in range(N):
        say(f"[fp8 fwd given scale] rank={r}")
        desc_q = cp.Desc(1, H, d, 1, L, 0, "bf16", "none", scale=sm)
        qc = torch.empty((1, L, H, d), dtype=torch.uint8, device="cuda")
        qs = torch.empty((1, H), device="cuda")
        cp.cp_attn_quantize_fp8(desc_q, dev(inp["q"][r], "bf16"), qc, qs, role=cp.CP_FP8_QUERY)
        c = F.query_prescale(d, sm)
        qz = F.quantize_heads(inp["q"][r], c)
        assert np.array_equal(qc.cpu().numpy(), qz["codes"]), "query codes differ from the oracle's"
        desc = cp.Desc(1, H, d, N, L, r, "bf16", "causal", scale=sm)
        out = torch.full((1, L, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        m, l, lse = (torch.full((1, H, L), float("nan"), device="cuda") for _ in range(3))
        ws = cp.alloc_workspace(desc)
        cs, xs = torch.cuda.Stream(), torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            cp.cp_attn_rank_forward_fp8(desc, qc, qs, [x[0] for x in kd], [x[1] for x in kd], [x[0] for x in vd],
                                        [x[1] for x in vd], out, m, l, lse, workspace=ws, compute_stream=cs,
                                        copy_stream=xs, flags=cp.CP_RING_PREFETCH)
        torch.cuda.synchronize()
        ref = F.fp8_rank_attention(qz["codes"], qz["scale"], [z["codes"] for z in kz], [z["scale"] for z in kz],
                                   [z["codes"] for z in vz], [z["scale"] for z in vz], r, N, "causal", scale=sm,
                                   q_prescale=c)
        A = _product_bound(spec, qz, kz, scale=sm)
        say(f"   {_check_fp8((host(out), host(m), host(l), host(lse)), ref, A)}")


def test_fp8_forward_logit_range(cp):
    """Logits far outside the range where exp2(x) and 2^m_ref are normal
    float32 values, so waves take the subtracting path: head 0 has all
    scores near +400 (m_ref near +560 in base 2), head 1 near -400 (m_ref
    near -560), head 2 has ordinary rows and, in the wave of rows 64-95,
    rows 80 on 20 times larger, and the keys of the second block 20 times
    larger from its row 100 on (global key 230): on rank 1 references leave
    the range in the middle of a row, in a wave that mixes both kinds of
    rows.  N = 2 shards of L = 130, causal, d = 64, every rank."""
    N, L, H, d = 2, 130, 3, 64
    spec = ShardSpec(S=N * L, N=N, H=H, d=d, dtype="bf16", mask="causal", cfg_id=114)
    inp = make_inputs(spec, seed=6, ranks=range(N))
    rng = np.random.default_rng(61)
    for r in range(N):
        q = inp["q"][r]
        q[:, :, 0, :] = np.abs(rng.standard_normal((1, L, d))) * 4 + 4
        q[:, :, 1, :] = np.abs(rng.standard_normal((1, L, d))) * 4 + 4
        q[:, 80:, 2, :] *= 20
        inp["q"][r] = round_to_bf16(q)
    for j in range(N):
        k = inp["k"][j]
        k[:, :, 0, :] = np.abs(rng.standard_normal((1, L, d))) * 4 + 4
        k[:, :, 1, :] = -(np.abs(rng.standard_normal((1, L, d))) * 4 + 4)
        if j == 1:
            k[:, 100:, 2, :] *= 20                 # global keys 230 on
        inp["k"][j] = round_to_bf16(k)
    c = F.query_prescale(d)
    qz = {r: F.quantize_heads(inp["q"][r], c) for r in range(N)}
    kz = [F.quantize_heads(inp["k"][j]) for j in range(N)]
    vz = [F.quantize_heads(inp["v"][j]) for j in range(N)]
    kd = [_codes_dev(z) for z in kz]
    vd = [_codes_dev(z) for z in vz]
    for r in range(N):
        ref = _oracle_fp8(spec, r, qz[r], kz, vz)
        m2 = ref["m"] / np.log(2.0)
        say(f"[fp8 fwd logit range] rank={r}: base-2 row max per head "
            f"{[(float(np.min(m2[0, h])), float(np.max(m2[0, h]))) for h in range(H)]}")
        assert np.min(m2[0, 0]) > 130 and np.max(m2[0, 1]) < -130, "the heads do not reach the subtracting path"
        qc, qs = _codes_dev(qz[r])
        got = _run_fp8(cp, spec, r, qc, qs, [x[0] for x in kd], [x[1] for x in kd], [x[0] for x in vd],
                       [x[1] for x in vd], cp.CP_RING_PREFETCH)
        say(f"   {_check_fp8(got, ref, _product_bound(spec, qz[r], kz))}")


def _quantize_dev(cp, x_dev, spec, role):
    desc = cp.Desc(spec.B, spec.H, spec.d, 1, spec.L, 0, "bf16", "none")
    codes = torch.empty(x_dev.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty((spec.B, spec.H), device="cuda")
    cp.cp_attn_quantize_fp8(desc, x_dev, codes, scales, role=role)
    return codes, scales


@pytest.mark.parametrize("cfg", [3, 5])
def test_fp8_forward_full_size(cp, cfg):
    """The causal 128K last-rank shard and the packed-document shard at full
    size: bf16 draws quantised on the device (codes checked bit-exact against
    the oracle's on the sampled heads), the FP8 ring forward with prefetch,
    sampled rows of three heads against the oracle."""
    spec = standard_configs(seed=0)[cfg]
    blocks = oracle.ring_schedule(spec.N, spec.rank, spec.L, spec.mask, spec.cu_seqlens)
    heads = sorted({0, spec.H - 1, int(np.random.default_rng(cfg + 17).integers(spec.H))})
    say(f"[fp8 full cfg {cfg}] {spec.name}: blocks {blocks}, heads {heads}")
    q = draw_shard(spec, 0, TENSOR_Q, spec.rank)
    c = F.query_prescale(spec.d)
    qc, qs = _quantize_dev(cp, dev(q, "bf16"), spec, cp.CP_FP8_QUERY)
    qz = F.quantize_heads(q[:, :, heads], c)
    assert np.array_equal(qc.cpu().numpy()[:, :, heads], qz["codes"])
    del q
    kc, ks, vc, vs = ([None] * spec.N for _ in range(4))
    kz, vz = [None] * spec.N, [None] * spec.N
    for j in blocks:
        for tid, cs_, ss_, zz in ((TENSOR_K, kc, ks, kz), (TENSOR_V, vc, vs, vz)):
            x = draw_shard(spec, 0, tid, j)
            cs_[j], ss_[j] = _quantize_dev(cp, dev(x, "bf16"), spec, cp.CP_FP8_KV)
            zz[j] = F.quantize_heads(x[:, :, heads])
            del x
            assert np.array_equal(cs_[j].cpu().numpy()[:, :, heads], zz[j]["codes"]), f"codes of block {j}"
    got = _run_fp8(cp, spec, spec.rank, qc, qs, kc, ks, vc, vs, cp.CP_RING_PREFETCH)
    extra = []
    if spec.cu_seqlens is not None:
        s0 = spec.rank * spec.L
        extra = [x - s0 + e for x in spec.cu_seqlens if s0 <= x < s0 + spec.L for e in (-1, 0, 1)]
    rows = sample_rows(spec.L, cfg, extra=extra)
    ref = F.fp8_rank_attention(qz["codes"], qz["scale"], [z["codes"] if z else None for z in kz],
                               [z["scale"] if z else None for z in kz], [z["codes"] if z else None for z in vz],
                               [z["scale"] if z else None for z in vz], spec.rank, spec.N, spec.mask,
                               spec.cu_seqlens, rows=rows, q_prescale=c)
    stats = _check_fp8(got, ref, _product_bound(spec, qz, kz, rows=rows), rows=rows, heads=heads)
    say(f"[fp8 full cfg {cfg}] {len(rows)} rows x {len(heads)} heads: {stats}")
    for arr in got:
        assert np.all(np.isfinite(arr))
