"""GPU parity of the backward entry points (cp_attn_bwd_delta,
cp_attn_block_backward, cp_attn_rank_backward) against the fp64 backward
oracle, through the C ABI.

Tolerance for the float32 gradients from bf16 inputs (stated here, applied by
every test below): over the compared tensor, RMS error <= 5e-3 x RMS of the
reference and max error <= 2e-2 x max |reference|; a tensor whose reference
is exactly zero (a block no row sees) must be exactly zero.  Derivation: the
oracle sees the same bf16-rounded Q, K, V, dO, so the kernel's own error is P
and dS rounded to bf16 (round to nearest even) before their MFMA products,
and, end to end, O rounded to bf16 inside delta.  One such rounding has a
relative RMS error of 2^-9 / sqrt(3) = 1.1e-3; a gradient term carries one
(dV: P) or two (dQ, dK: P inside dS, then dS) of them, about 1.6e-3 RMS, and
summing many terms keeps that ratio.  The bounds are about 3x the expected
RMS and leave room for the tails of the largest entries, while a wrong term
(a dropped delta, scale or mask) moves the error to order 1.  delta itself is
a plain fp32 sum: relative 1e-5 of the sum of |terms|.
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
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

RMS_REL, MAX_REL = 5e-3, 2e-2


def check_grad(got: np.ndarray, ref: np.ndarray, what: str) -> dict:
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    if not np.any(ref):
        assert not np.any(got), f"{what}: reference is zero, got max {np.max(np.abs(got)):.3e}"
        return {"rms_rel": 0.0, "max_rel": 0.0}
    err = got - ref
    rms_rel = float(np.sqrt(np.mean(err ** 2)) / np.sqrt(np.mean(ref ** 2)))
    max_rel = float(np.max(np.abs(err)) / np.max(np.abs(ref)))
    say(f"  {what}: rms error {rms_rel:.2e} of rms(ref), max error {max_rel:.2e} of max|ref|")
    assert rms_rel <= RMS_REL, f"{what}: rms error {rms_rel:.3e} of rms(ref) > {RMS_REL}"
    assert max_rel <= MAX_REL, f"{what}: max error {max_rel:.3e} of max|ref| > {MAX_REL}"
    return {"rms_rel": rms_rel, "max_rel": max_rel}


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
    """GPU forward (out, lse) then GPU backward, against the definition's
    gradient from Q, K, V and dO alone."""
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
        ref = G.rank_backward(q, ks, vs, do, rank, spec.N, mask, spec.cu_seqlens)
        check_grad(host(dq), ref["dq"], f"dq r{rank}")
        for j in range(spec.N):
            check_grad(host(dks[j]), ref["dk"][j], f"dk{j} r{rank}")
            check_grad(host(dvs[j]), ref["dv"][j], f"dv{j} r{rank}")


def test_rank_backward_full_size():
    """The 128K last-rank causal shard (S=131072, N=4, L=32768, H=32, d=128,
    rank 3) in the launch configuration bench.py times: dq of sampled rows and
    dk, dv of the diagonal block's last keys against the oracle exactly; and,
    over all blocks, sum_c dK_c = 0 and sum_c dV_c = sum_q dO_q per head (the
    rows of dS sum to zero and the rows of P to one)."""
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

    K_all = [np.concatenate([inp["k"][j][0, :, h, :] for j in range(N)]).astype(np.float64) for h in (0, H - 1)]
    V_all = [np.concatenate([inp["v"][j][0, :, h, :] for j in range(N)]).astype(np.float64) for h in (0, H - 1)]
    c_all = np.arange(N * L, dtype=np.int64)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, L // 2, L - 129, L - 128, L - 1],
                                     np.random.default_rng(5).integers(0, L, 14)]))
    last = np.arange(L - 48, L)
    for hi, h in enumerate((0, H - 1)):
        say(f"full-size backward: oracle rows, head {h}")
        p = spec.rank * L + rows
        gq, _, _ = G.attention_grad_rows(q[0, rows, h, :], K_all[hi], V_all[hi], do[0, rows, h, :], p, c_all, "causal")
        check_grad(host(dq[0, rows, h, :]), gq, f"dq rows h{h}")
        # the diagonal block's last 48 keys are seen only by the last 48 rows
        p = spec.rank * L + last
        _, gk, gv = G.attention_grad_rows(q[0, last, h, :], K_all[hi], V_all[hi], do[0, last, h, :], p, c_all, "causal")
        key_idx = spec.rank * L + last
        check_grad(host(dks[spec.rank][0, last, h, :]), gk[key_idx], f"dk last keys h{h}")
        check_grad(host(dvs[spec.rank][0, last, h, :]), gv[key_idx], f"dv last keys h{h}")
