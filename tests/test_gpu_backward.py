"""GPU parity of the backward entry points (cp_attn_bwd_delta,
cp_attn_block_backward, cp_attn_rank_backward) against the fp64 backward
oracle, through the C ABI.

Tolerance for the float32 gradients from bf16 inputs (stated here, applied by
every test below), element by element: a gradient row is one (batch, token,
head) vector over the head dim, and each element must satisfy

    |got - ref| <= 1.5e-2 * rms_row(ref) + 1e-4 * rms(ref) + 1e-2 * |ref|,

with rms_row the RMS of the reference over that element's row and rms(ref)
over the whole compared tensor; in addition the RMS of the error over the
tensor must stay within 5e-3 x rms(ref).  Derivation: the oracle sees the same
bf16-rounded Q, K, V, dO, so the kernel's own error is P and dS rounded to
bf16 (round to nearest even) before their MFMA products, and, end to end, O
rounded to bf16 inside delta.  One such rounding has a relative RMS error of
2^-9 / sqrt(3) = 1.1e-3.  An element of dV_c = sum_p P_pc dO_p carries one
rounding per term, an element of dQ_p or dK_c (sums of dS times K or Q) two;
the terms have independent signs, so the error of an element is about
1.6e-3 x sqrt(sum of its squared terms), which is the scale of its row's RMS
(measured on the GPU: 1.54e-3 to 1.74e-3 of rms(ref) over every tensor of
these tests, and single elements up to 1.05e-2 x rms_row in tensors of
10^5 elements); 1.5e-2 x rms_row is about nine such standard deviations.
The bound is per row,
so a wrong mask or index confined to a few rows of small magnitude still
fails.  The 1e-4 x rms(ref) floor covers rows whose exact gradient is zero
but whose computed one is a rounding residue (a query that sees a single key
has dS = P (dP - delta) = 0 exactly, while the kernel's dP and delta round
differently).  A tensor whose reference is exactly zero (a block no row sees)
must be exactly zero.  delta itself is a plain fp32 sum: relative 1e-5 of the
sum of |terms|.

The backward takes the forward output O as an input (delta = rowsum(dO * O)
of the O handed in), and after a GPU forward that O is bf16.  Its rounding
moves delta_p by up to 2^-9 sum_d |dO_pd O_pd| and dQ_p by scale * delta
error * (P K)_p, the same direction for every element of the row: where one
key dominates a row (the first tokens of a document) this exceeds the row's
own small gradient.  So the end-to-end test compares element by element
against the oracle's block form fed with that same O (its delta), and bounds
the remaining gap to the definition computed from Q, K, V and dO alone by the
RMS check.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle.attention as A
import oracle.backward as G
from context_ring_attention_cp_amd import _binding as B
from context_ring_attention_cp_amd import alloc_workspace
from harness.inputs import ShardSpec, draw_grad, lognormal_cu_seqlens, make_inputs, round_to_bf16, standard_configs
from tests.gpu_util import dev, host, pooled_reduce, say

pytestmark = pytest.mark.gpu

ATOL_ROW, ATOL_TENSOR, RTOL, RMS_REL = 1.5e-2, 1e-4, 1e-2, 5e-3


def check_grad(got: np.ndarray, ref: np.ndarray, what: str) -> dict:
    """The per-element bound of the module header; the last axis is the head
    dim, every other index names one gradient row."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    if not np.any(ref):
        assert not np.any(got), f"{what}: reference is zero, got max {np.max(np.abs(got)):.3e}"
        return {"rms_rel": 0.0, "worst": 0.0}
    err = np.abs(got - ref)
    rms_t = float(np.sqrt(np.mean(ref ** 2)))
    rms_row = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
    bound = ATOL_ROW * rms_row + ATOL_TENSOR * rms_t + RTOL * np.abs(ref)
    ratio = err / bound
    worst = float(ratio.max())
    rms_rel = float(np.sqrt(np.mean(err ** 2)) / rms_t)
    at = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    say(f"  {what}: rms error {rms_rel:.2e} of rms(ref); worst element at {tuple(int(x) for x in at)} "
        f"uses {worst:.2f} of its bound (err {float(err[at]):.2e}, row rms {float(rms_row[at[:-1]][0]):.2e})")
    assert worst <= 1.0, f"{what}: element {at} error {float(err[at]):.3e} > bound {float(bound[at]):.3e}"
    assert rms_rel <= RMS_REL, f"{what}: rms error {rms_rel:.3e} of rms(ref) > {RMS_REL}"
    return {"rms_rel": rms_rel, "worst": worst}


def _zeros(shape, dtype="f32"):
    import torch
    return torch.zeros(shape, dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device="cuda")


def _spec(mask, d, rank, N=3, L=300, H=2, Bt=2, cfg_id=41):
    S = N * L
    cu = lognormal_cu_seqlens(7, cfg_id, S, median=150.0, lo=20, hi=600) if mask == "doc_causal" else None
    return ShardSpec(S=S, N=N, H=H, d=d, dtype="bf16", mask=mask, rank=rank, B=Bt, cu_seqlens=cu, cfg_id=cfg_id)


def _desc(spec, cu_dev=None):
    return B.Desc(spec.B, spec.H, spec.d, spec.N, spec.L, spec.rank, "bf16", spec.mask,
                  cu_seqlens=spec.cu_seqlens, cu_seqlens_dev=cu_dev)


def _cu_dev(spec):
    import torch
    if spec.cu_seqlens is None:
        return None
    return torch.from_numpy(np.asarray(spec.cu_seqlens, np.int32)).to("cuda")


def test_bwd_delta_matches_oracle():
    import torch
    rng = np.random.default_rng(3)
    for d in (64, 128):
        shape = (2, 301, 3, d)
        o = round_to_bf16(rng.standard_normal(shape).astype(np.float32))
        g = round_to_bf16(rng.standard_normal(shape).astype(np.float32))
        desc = B.Desc(2, 3, d, 2, 301, 1, "bf16", "causal")
        delta = torch.full((2, 3, 301), float("nan"), device="cuda")
        B.cp_attn_bwd_delta(desc, dev(o, "bf16"), dev(g, "bf16"), delta)
        torch.cuda.synchronize()
        ref = G.bwd_delta(o, g)
        scale = np.einsum("blhd->bhl", np.abs(o.astype(np.float64) * g))
        err = np.abs(host(delta) - ref)
        assert np.all(err <= 1e-5 * scale + 1e-6), float(np.max(err - 1e-5 * scale))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", ["none", "causal", "doc_causal"])
def test_block_backward_every_rank(mask, d):
    """Each block's dq part, dk_j, dv_j with the oracle's lse and delta as
    inputs (the kernels alone), every rank of a 3-rank ring, ragged L = 300."""
    import torch
    spec0 = _spec(mask, d, 0)
    inp = make_inputs(spec0, 0, ranks=range(spec0.N))
    for rank in range(spec0.N):
        spec = _spec(mask, d, rank)
        say(f"block_backward mask={mask} d={d} rank={rank}")
        q = inp["q"][rank]
        ks = [inp["k"][j] for j in range(spec.N)]
        vs = [inp["v"][j] for j in range(spec.N)]
        do = draw_grad(spec, 0, rank)
        f = A.rank_attention(q, ks, vs, rank, spec.N, mask, spec.cu_seqlens)
        delta = G.bwd_delta(f["o"], do)
        cu_dev = _cu_dev(spec)
        desc = _desc(spec, cu_dev)
        qd, dod = dev(q, "bf16"), dev(do, "bf16")
        lse_d, dl_d = dev(f["lse"], "f32"), dev(delta, "f32")
        big = spec.shard_shape()
        dq = torch.full(big, float("nan"), device="cuda")
        ref_dq = np.zeros(big)
        for j in range(spec.N):
            dk = torch.full(big, float("nan"), device="cuda")
            dv = torch.full(big, float("nan"), device="cuda")
            mode = B.CP_MODE_INIT if j == 0 else B.CP_MODE_ACCUMULATE
            B.cp_attn_block_backward(desc, j, mode, qd, dev(ks[j], "bf16"), dev(vs[j], "bf16"), dod, lse_d, dl_d,
                                     dq, dk, dv)
            torch.cuda.synchronize()
            ref = G.block_backward(q, ks[j], vs[j], do, f["lse"], delta, rank, j, spec.N, mask, spec.cu_seqlens)
            ref_dq += ref["dq"]
            check_grad(host(dk), ref["dk"], f"dk{j} r{rank}")
            check_grad(host(dv), ref["dv"], f"dv{j} r{rank}")
        check_grad(host(dq), ref_dq, f"dq r{rank}")


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("mask,d", [("causal", 128), ("doc_causal", 64), ("none", 128)])
def test_rank_backward_end_to_end(mask, d, reverse):
    """GPU forward (out, lse) then GPU backward: element by element against
    the oracle's block form with the delta of the O handed in, and by RMS
    against the definition's gradient from Q, K, V and dO alone."""
    import torch
    spec0 = _spec(mask, d, 0, cfg_id=43)
    inp = make_inputs(spec0, 1, ranks=range(spec0.N))
    flags = B.CP_RING_REVERSE if reverse else 0
    for rank in (1, spec0.N - 1):
        spec = _spec(mask, d, rank, cfg_id=43)
        say(f"rank_backward mask={mask} d={d} rank={rank} reverse={reverse}")
        q = inp["q"][rank]
        ks = [inp["k"][j] for j in range(spec.N)]
        vs = [inp["v"][j] for j in range(spec.N)]
        do = draw_grad(spec, 1, rank)
        cu_dev = _cu_dev(spec)
        desc = _desc(spec, cu_dev)
        big, vec = spec.shard_shape(), (spec.B, spec.H, spec.L)
        qd = dev(q, "bf16")
        kd = [dev(k, "bf16") for k in ks]
        vd = [dev(v, "bf16") for v in vs]
        out = _zeros(big, "bf16")
        lse = torch.zeros(vec, device="cuda")
        ws = alloc_workspace(desc)
        B.cp_attn_rank_forward(desc, qd, kd, vd, out, lse_out=lse, workspace=ws, flags=flags)
        delta = torch.zeros(vec, device="cuda")
        dq = torch.full(big, float("nan"), device="cuda")
        dks = [torch.full(big, float("nan"), device="cuda") for _ in range(spec.N)]
        dvs = [torch.full(big, float("nan"), device="cuda") for _ in range(spec.N)]
        B.cp_attn_rank_backward(desc, qd, kd, vd, out, dev(do, "bf16"), lse, delta, dq, dks, dvs, flags=flags)
        torch.cuda.synchronize()
        # per element: the oracle's block form with the delta of the O handed in
        f = A.rank_attention(q, ks, vs, rank, spec.N, mask, spec.cu_seqlens)
        delta_in = G.bwd_delta(host(out), do)
        blk = [G.block_backward(q, ks[j], vs[j], do, f["lse"], delta_in, rank, j, spec.N, mask, spec.cu_seqlens)
               for j in range(spec.N)]
        check_grad(host(dq), sum(b["dq"] for b in blk), f"dq r{rank}")
        for j in range(spec.N):
            check_grad(host(dks[j]), blk[j]["dk"], f"dk{j} r{rank}")
            check_grad(host(dvs[j]), blk[j]["dv"], f"dv{j} r{rank}")
        # end to end: the definition's gradient from Q, K, V and dO alone
        ref = G.rank_backward(q, ks, vs, do, rank, spec.N, mask, spec.cu_seqlens)
        for got, r, what in [(dq, ref["dq"], "dq")] + [(dks[j], ref["dk"][j], f"dk{j}") for j in range(spec.N)] + \
                [(dvs[j], ref["dv"][j], f"dv{j}") for j in range(spec.N)]:
            g, rr = host(got), r
            if not np.any(rr):
                assert not np.any(g), f"{what} r{rank}: reference is zero"
                continue
            rel = float(np.sqrt(np.mean((g - rr) ** 2)) / np.sqrt(np.mean(rr ** 2)))
            assert rel <= RMS_REL, f"{what} r{rank}: rms error {rel:.3e} of rms(ref) against the definition"


@pytest.mark.timeout(900)
def test_rank_backward_full_size():
    """The 128K last-rank causal shard (S=131072, N=4, L=32768, H=32, d=128,
    rank 3) in the launch configuration bench.py times: one whole head (dQ of
    all 32768 rows; dK, dV of all keys of the four blocks) against the oracle
    element by element; and, over all blocks and every head, sum_c dK_c = 0
    and sum_c dV_c = sum_q dO_q (the rows of dS sum to zero and the rows of P
    to one)."""
    import torch
    spec = standard_configs(0)[3]
    N, L, H, d = spec.N, spec.L, spec.H, spec.d
    say("full-size backward: generating inputs")
    inp = make_inputs(spec, 0)
    q = inp["q"][spec.rank]
    do = draw_grad(spec, 0, spec.rank)
    desc = _desc(spec)
    big, vec = spec.shard_shape(), (1, H, L)
    qd = dev(q, "bf16")
    kd = [dev(inp["k"][j], "bf16") for j in range(N)]
    vd = [dev(inp["v"][j], "bf16") for j in range(N)]
    dod = dev(do, "bf16")
    out = _zeros(big, "bf16")
    lse = torch.zeros(vec, device="cuda")
    ws = alloc_workspace(desc)
    say("full-size backward: forward")
    copy_stream = torch.cuda.Stream()
    B.cp_attn_rank_forward(desc, qd, kd, vd, out, lse_out=lse, workspace=ws, copy_stream=copy_stream,
                           flags=B.CP_RING_PREFETCH)
    delta = torch.zeros(vec, device="cuda")
    dq = torch.full(big, float("nan"), device="cuda")
    dks = [torch.full(big, float("nan"), device="cuda") for _ in range(N)]
    dvs = [torch.full(big, float("nan"), device="cuda") for _ in range(N)]
    say("full-size backward: backward")
    B.cp_attn_rank_backward(desc, qd, kd, vd, out, dod, lse, delta, dq, dks, dvs)
    torch.cuda.synchronize()
    del ws

    # identities over all blocks, every head
    dk_sum = sum(t.double().sum(dim=1) for t in dks)                 # [1, H, d]
    dk_abs = sum(t.double().abs().sum(dim=1) for t in dks)
    say(f"  sum_c dK_c: max {float((dk_sum.abs() / dk_abs).max()):.2e} of sum |dK|")
    assert torch.all(dk_sum.abs() <= 1e-2 * dk_abs), float((dk_sum.abs() / dk_abs).max())
    dv_sum = sum(t.double().sum(dim=1) for t in dvs)
    do_sum = dod.double().sum(dim=1)
    do_abs = dod.double().abs().sum(dim=1)
    say(f"  sum_c dV_c - sum_q dO_q: max {float(((dv_sum - do_sum).abs() / do_abs).max()):.2e} of sum |dO|")
    assert torch.all((dv_sum - do_sum).abs() <= 1e-2 * do_abs), float(((dv_sum - do_sum).abs() / do_abs).max())

    # one whole head against the definition: dQ of every row, and dK, dV of
    # every key of every block (all rows' contributions, summed over row chunks)
    h = int(np.random.default_rng(11).integers(H))
    K_all = np.concatenate([inp["k"][j][0, :, h, :] for j in range(N)]).astype(np.float64)
    V_all = np.concatenate([inp["v"][j][0, :, h, :] for j in range(N)]).astype(np.float64)
    c_all = np.arange(N * L, dtype=np.int64)
    q_h, do_h = q[0, :, h, :], do[0, :, h, :]
    say(f"full-size backward: oracle over all {L} rows of head {h}")

    def part(rows, acc):
        gq, gk, gv = G.attention_grad_rows(q_h[rows], K_all, V_all, do_h[rows], spec.rank * L + rows, c_all,
                                           "causal")
        if acc is None:
            acc = {"dq": np.zeros((L, d)), "dk": np.zeros((N * L, d)), "dv": np.zeros((N * L, d))}
        acc["dq"][rows] = gq
        acc["dk"] += gk
        acc["dv"] += gv
        return acc

    accs = pooled_reduce(part, L, chunk=256)
    ref_dq = sum(a["dq"] for a in accs)
    ref_dk = sum(a["dk"] for a in accs)
    ref_dv = sum(a["dv"] for a in accs)
    del accs
    check_grad(host(dq[0, :, h, :]), ref_dq, f"dq head {h}")
    for j in range(N):
        check_grad(host(dks[j][0, :, h, :]), ref_dk[j * L:(j + 1) * L], f"dk{j} head {h}")
        check_grad(host(dvs[j][0, :, h, :]), ref_dv[j * L:(j + 1) * L], f"dv{j} head {h}")
