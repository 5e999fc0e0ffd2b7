"""The allocation-free rank forward, cp_attn_rank_forward_static, through the
C ABI, against cp_attn_rank_forward with a caller-allocated workspace on the
same inputs.  Both run the same kernels in the same order, so every output
(out, m, l, lse) must be bit-identical.  Three calls in a row share the static
scratch, each on a smaller shard than the one before and with the scratch
holding the previous call's bytes: a 4096-token bf16 causal shard with ring
prefetch (68 MB of the 96 MiB scratch, key-split side state included), a ragged document-masked bf16 shard
at d = 64, and a tiny fp32 shard without prefetch.  A shard whose scratch
would exceed the array is refused with CP_ERR_WORKSPACE before anything is
enqueued.
"""
from __future__ import annotations

import numpy as np
import pytest

from harness.inputs import ShardSpec, make_inputs
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def cp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import context_ring_attention_cp_amd as cp
    cp.lib()     # raises if the library is not built: no fallback
    return cp


CASES = [
    (ShardSpec(S=4 * 4096, N=4, H=8, d=128, dtype="bf16", mask="causal", rank=3, cfg_id=130), 1),
    (ShardSpec(S=3 * 700, N=3, H=3, d=64, dtype="bf16", mask="doc_causal", rank=2, B=2, cfg_id=131,
               cu_seqlens=np.asarray([0, 300, 1111, 1500, 2100], np.int32)), 1),
    (ShardSpec(S=2 * 96, N=2, H=2, d=64, dtype="f32", mask="causal", rank=1, cfg_id=132), 0),
]


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _run(cp, spec, static, flags, q, kb, vb, cu_dev):
    desc = cp.Desc(spec.B, spec.H, spec.d, spec.N, spec.L, spec.rank, spec.dtype, spec.mask,
                   cu_seqlens=spec.cu_seqlens, cu_seqlens_dev=cu_dev)
    dt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    out = torch.full((spec.B, spec.L, spec.H, spec.d), float("nan"), dtype=dt, device="cuda")
    m, l, lse = (torch.full((spec.B, spec.H, spec.L), float("nan"), device="cuda") for _ in range(3))
    cs, xs = torch.cuda.Stream(), torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    if static:
        cp.cp_attn_rank_forward_static(desc, q, kb, vb, out, m, l, lse, compute_stream=cs, copy_stream=xs,
                                       flags=flags)
    else:
        ws = cp.alloc_workspace(desc)
        cp.cp_attn_rank_forward(desc, q, kb, vb, out, m, l, lse, workspace=ws, compute_stream=cs,
                                copy_stream=xs, flags=flags)
    torch.cuda.synchronize()
    return [_bits(t) for t in (out, m, l, lse)]


def test_static_scratch_matches_workspace_forward(cp):
    sizes = []
    for spec, flags in CASES:
        desc = cp.Desc(spec.B, spec.H, spec.d, spec.N, spec.L, spec.rank, spec.dtype, spec.mask,
                       cu_seqlens=spec.cu_seqlens,
                       cu_seqlens_dev=torch.zeros(1, dtype=torch.int32, device="cuda"))
        sizes.append(cp.cp_attn_workspace_bytes(desc))
    assert sizes[0] <= cp.CP_STATIC_SCRATCH_BYTES and sizes[0] > sizes[1] > sizes[2]
    for spec, flags in CASES:
        say(f"[static scratch] {spec.dtype} {spec.mask} N={spec.N} L={spec.L} H={spec.H} d={spec.d} flags={flags}")
        inp = make_inputs(spec, seed=3, ranks=[spec.rank])
        q = dev(inp["q"][spec.rank], spec.dtype)
        kb = [dev(inp["k"][j], spec.dtype) for j in range(spec.N)]
        vb = [dev(inp["v"][j], spec.dtype) for j in range(spec.N)]
        cu_dev = torch.from_numpy(spec.cu_seqlens).cuda() if spec.cu_seqlens is not None else None
        got = _run(cp, spec, True, flags, q, kb, vb, cu_dev)
        ref = _run(cp, spec, False, flags, q, kb, vb, cu_dev)
        for name, a, b in zip(("out", "m", "l", "lse"), got, ref):
            bad = np.argwhere(a != b)
            assert bad.size == 0, f"{name}: {len(bad)} elements differ, first at {bad[0]}"
        out_f = got[0].astype(np.uint32) << 16 if spec.dtype == "bf16" else got[0].astype(np.uint32)
        assert np.all(np.isfinite(out_f.view(np.float32))), "non-finite output"


def test_static_scratch_refuses_oversized_shard(cp):
    spec = ShardSpec(S=4 * 8192, N=4, H=8, d=128, dtype="bf16", mask="causal", rank=3, cfg_id=133)
    desc = cp.Desc(spec.B, spec.H, spec.d, spec.N, spec.L, spec.rank, "bf16", "causal")
    assert cp.cp_attn_workspace_bytes(desc) > cp.CP_STATIC_SCRATCH_BYTES
    x = torch.zeros((1, spec.L, spec.H, spec.d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cp.CpAttnError) as e:
        cp.cp_attn_rank_forward_static(desc, x, [x] * 4, [x] * 4, x, flags=0)
    assert e.value.status == cp.CP_ERR_WORKSPACE and "static scratch" in str(e.value)
