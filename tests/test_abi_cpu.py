"""CPU tests of the C ABI: the library loads, exports every function
include/cpattn.h declares, and its host-only logic (validation, ring
schedule, visible-pair counts, workspace size) behaves as documented.

Every error case below makes exactly one argument invalid, so each call
returns a validation status before the library makes any HIP call; no test
here reaches a kernel launch.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from context_ring_attention_cp_amd import _binding as B
from harness.inputs import lognormal_cu_seqlens

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")

FAKE = 0x7F0000000000          # aligned, non-null; never dereferenced (validation fails first)


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(cp_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = B.lib()
    declared = _declared()
    assert len(declared) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", B._LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (cp_attn_\w+)", out))
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    for f in declared:
        assert hasattr(lib, f)
    assert sorted(B.EXPORTED) == declared


def _desc(**kw):
    base = dict(B=1, H=2, d=128, N=4, L=64, rank=3, dtype="bf16", mask="causal")
    base.update(kw)
    cu = base.pop("cu_seqlens", None)
    cud = base.pop("cu_seqlens_dev", None)
    return B.Desc(cu_seqlens=cu, cu_seqlens_dev=cud, **base)


def _status(fn, *args):
    st = fn(*args)
    assert st != B.CP_ERR_HIP, B.last_error()
    return st


@pytest.mark.parametrize("N", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("mask", ["none", "causal", "doc_causal"])
@pytest.mark.parametrize("reverse", [False, True])
def test_schedule_matches_oracle(N, mask, reverse):
    L = 96
    cu = np.asarray([0, 10, 20, 47, 48, 51, 72, 90, 96, 180, 192, 200, 300, 301], np.int64)
    cu = cu[cu < N * L].tolist() + [N * L]
    cu = np.asarray(cu, np.int32)
    for r in range(N):
        d = _desc(N=N, L=L, rank=r, mask=mask, cu_seqlens=cu if mask == "doc_causal" else None,
                  cu_seqlens_dev=FAKE if mask == "doc_causal" else None)
        got = B.cp_attn_ring_schedule(d, B.CP_RING_REVERSE if reverse else 0)
        want = oracle.ring_schedule(N, r, L, mask, cu, direction="reverse" if reverse else "forward")
        assert got == want, (r, got, want)


def test_schedule_workload_examples():
    d = _desc(N=4, L=32768, rank=3, H=32)
    assert B.cp_attn_ring_schedule(d) == [3, 2, 1, 0]
    assert B.cp_attn_ring_schedule(d, B.CP_RING_REVERSE) == [3, 0, 1, 2]
    d = _desc(N=8, L=8192, rank=5, H=16, mask="none")
    assert B.cp_attn_ring_schedule(d) == [5, 4, 3, 2, 1, 0, 7, 6]
    cu = lognormal_cu_seqlens(0, 5, 131072)
    d = _desc(N=8, L=16384, rank=7, H=32, mask="doc_causal", cu_seqlens=cu, cu_seqlens_dev=FAKE)
    assert B.cp_attn_ring_schedule(d) == oracle.ring_schedule(8, 7, 16384, "doc_causal", cu)


@pytest.mark.parametrize("mask", ["none", "causal", "doc_causal"])
def test_visible_pairs_matches_oracle(mask):
    for N, L in ((1, 7), (3, 33), (4, 256), (8, 16384)):
        cu = lognormal_cu_seqlens(3, 9, N * L, median=max(2, L // 3), sigma=1.0, lo=1, hi=N * L)
        for r in range(N):
            d = _desc(N=N, L=L, rank=r, mask=mask, cu_seqlens=cu if mask == "doc_causal" else None,
                      cu_seqlens_dev=FAKE if mask == "doc_causal" else None)
            assert B.cp_attn_visible_pairs(d) == oracle.visible_pairs(N, L, r, mask, cu), (N, L, r)


def test_workspace_bytes():
    d = _desc(N=4, L=32768, rank=3, H=32)
    elems = 32768 * 32 * 128
    need = 4 * elems * 2 + elems * 4 + 2 * 32 * 32768 * 4
    got = B.cp_attn_workspace_bytes(d)
    assert need <= got <= need + 8 * 256
    assert B.lib().cp_attn_workspace_bytes(_desc(rank=9).ref) == 0
    assert "rank" in B.last_error()


def test_workspace_bytes_key_split():
    """A causal bf16 shard with a step after its diagonal and at most 256
    workgroups in the diagonal launch (query tiles of 256 rows x heads x
    batch) also holds the side state of the diagonal's key split."""
    L, H = 8192, 8
    elems = L * H * 128
    base = 4 * elems * 2 + elems * 4 + 2 * H * L * 4
    side = elems * 4 + 2 * H * L * 4
    got = B.cp_attn_workspace_bytes(_desc(N=4, L=L, rank=3, H=H))
    assert base + side <= got <= base + side + 12 * 256
    for kw in (dict(rank=0), dict(mask="none"), dict(mask="doc_causal", cu_seqlens=[0, 4 * L], cu_seqlens_dev=FAKE),
               dict(H=2 * H), dict(dtype="f32")):
        h = kw.pop("H", H)
        d = _desc(N=4, L=L, rank=kw.pop("rank", 3), H=h, **kw)
        eb = 4 if d.dtype == "f32" else 2
        plain = 4 * elems * eb * h // H + elems * 4 * h // H + 2 * h * L * 4
        assert plain <= B.cp_attn_workspace_bytes(d) <= plain + 8 * 256, kw


BAD_DESCS = [
    (dict(B=0), B.CP_ERR_INVALID_ARG, "B="),
    (dict(H=0), B.CP_ERR_INVALID_ARG, "H="),
    (dict(L=0), B.CP_ERR_INVALID_ARG, "L="),
    (dict(N=0, rank=0), B.CP_ERR_INVALID_ARG, "ring size"),
    (dict(N=65, rank=0), B.CP_ERR_INVALID_ARG, "ring size"),
    (dict(rank=4), B.CP_ERR_INVALID_ARG, "rank"),
    (dict(rank=-1), B.CP_ERR_INVALID_ARG, "rank"),
    (dict(dtype=7), B.CP_ERR_INVALID_ARG, "dtype"),
    (dict(mask=9), B.CP_ERR_INVALID_ARG, "mask"),
    (dict(scale=-1.0), B.CP_ERR_INVALID_ARG, "scale"),
    (dict(scale=float("nan")), B.CP_ERR_INVALID_ARG, "scale"),
    (dict(d=96), B.CP_ERR_UNSUPPORTED, "head dim"),
    (dict(d=256), B.CP_ERR_UNSUPPORTED, "head dim"),
    (dict(L=2 ** 30, N=4), B.CP_ERR_UNSUPPORTED, "int32"),
    (dict(mask="doc_causal"), B.CP_ERR_INVALID_ARG, "cu_seqlens"),
    (dict(mask="doc_causal", cu_seqlens=np.array([0, 100, 256], np.int32)), B.CP_ERR_INVALID_ARG, "cu_seqlens"),
    (dict(mask="doc_causal", cu_seqlens=np.array([1, 100, 256], np.int32), cu_seqlens_dev=FAKE),
     B.CP_ERR_INVALID_ARG, "cu_seqlens[0]"),
    (dict(mask="doc_causal", cu_seqlens=np.array([0, 100, 100, 256], np.int32), cu_seqlens_dev=FAKE),
     B.CP_ERR_INVALID_ARG, "strictly increasing"),
    (dict(mask="doc_causal", cu_seqlens=np.array([0, 100, 255], np.int32), cu_seqlens_dev=FAKE),
     B.CP_ERR_INVALID_ARG, "N*L"),
    (dict(mask="doc_causal", cu_seqlens=np.array([0, 256], np.int32), cu_seqlens_dev=FAKE + 2),
     B.CP_ERR_INVALID_ARG, "aligned"),
]


@pytest.mark.parametrize("kw,status,msg", BAD_DESCS)
def test_desc_validation(kw, status, msg):
    d = _desc(**kw)
    st = _status(B.lib().cp_attn_visible_pairs, d.ref, ctypes.byref(ctypes.c_int64()))
    assert st == status, (st, B.last_error())
    assert msg in B.last_error()
    # the same desc is rejected by the launching entry points before any HIP call
    st = _status(B.lib().cp_attn_block_partial, d.ref, 0, B.CP_MODE_PARTIAL_LSE, FAKE, FAKE, FAKE, None,
                 FAKE, FAKE, None)
    assert st == status
    st = _status(B.lib().cp_attn_finalize, d.ref, None, FAKE, None, None, None, None)
    assert st == status


def test_valid_doc_desc_accepted():
    d = _desc(mask="doc_causal", cu_seqlens=np.array([0, 100, 256], np.int32), cu_seqlens_dev=FAKE)
    assert B.cp_attn_visible_pairs(d) == oracle.visible_pairs(4, 64, 3, "doc_causal", np.array([0, 100, 256]))


def _state(o=FAKE, m=FAKE, l=FAKE):
    return ctypes.byref(B.cp_state(o, m, l))


def test_block_partial_argument_errors():
    lib = B.lib()
    d = _desc()
    cases = [
        ((d.ref, 4, B.CP_MODE_INIT, FAKE, FAKE, FAKE, _state(), None, None, None), "block j"),
        ((d.ref, -1, B.CP_MODE_INIT, FAKE, FAKE, FAKE, _state(), None, None, None), "block j"),
        ((d.ref, 0, 7, FAKE, FAKE, FAKE, None, None, None, None), "mode"),
        ((d.ref, 0, B.CP_MODE_INIT, None, FAKE, FAKE, _state(), None, None, None), "q is NULL"),
        ((d.ref, 0, B.CP_MODE_INIT, FAKE + 8, FAKE, FAKE, _state(), None, None, None), "q is not 16-byte"),
        ((d.ref, 0, B.CP_MODE_INIT, FAKE, None, FAKE, _state(), None, None, None), "k_j"),
        ((d.ref, 0, B.CP_MODE_INIT, FAKE, FAKE, FAKE + 4, _state(), None, None, None), "v_j"),
        ((d.ref, 0, B.CP_MODE_INIT, FAKE, FAKE, FAKE, None, None, None, None), "state is NULL"),
        ((d.ref, 0, B.CP_MODE_ACCUMULATE, FAKE, FAKE, FAKE, _state(o=None), None, None, None), "state->o"),
        ((d.ref, 0, B.CP_MODE_ACCUMULATE, FAKE, FAKE, FAKE, _state(m=FAKE + 2), None, None, None), "state->m"),
        ((d.ref, 0, B.CP_MODE_INIT, FAKE, FAKE, FAKE, _state(), FAKE, None, None), "must be NULL"),
        ((d.ref, 0, B.CP_MODE_PARTIAL_LSE, FAKE, FAKE, FAKE, _state(), FAKE, FAKE, None), "state must be NULL"),
        ((d.ref, 0, B.CP_MODE_PARTIAL_LSE, FAKE, FAKE, FAKE, None, None, FAKE, None), "o_part"),
        ((d.ref, 0, B.CP_MODE_PARTIAL_LSE, FAKE, FAKE, FAKE, None, FAKE, None, None), "lse_part"),
    ]
    for args, msg in cases:
        st = _status(lib.cp_attn_block_partial, *args)
        assert st == B.CP_ERR_INVALID_ARG, (msg, st)
        assert msg in B.last_error(), (msg, B.last_error())


def test_merge_argument_errors():
    lib = B.lib()
    d = _desc()
    P = ctypes.c_void_p
    parts = (P * 3)(FAKE, FAKE + 256, FAKE + 512)
    lses = (P * 3)(FAKE, FAKE + 256, FAKE + 512)
    I3 = ctypes.c_int32 * 3
    cases = [
        ((d.ref, 0, parts, lses, None, FAKE, None, None), "n="),
        ((d.ref, 65, parts, lses, None, FAKE, None, None), "n="),
        ((d.ref, 3, None, lses, None, FAKE, None, None), "NULL"),
        ((d.ref, 3, parts, lses, I3(0, 0, 1), FAKE, None, None), "permutation"),
        ((d.ref, 3, parts, lses, I3(0, 1, 3), FAKE, None, None), "permutation"),
        ((d.ref, 3, parts, lses, None, None, None, None), "out is NULL"),
        ((d.ref, 3, parts, lses, None, FAKE, FAKE + 1, None), "lse_out"),
        ((d.ref, 3, (P * 3)(FAKE, FAKE + 8, FAKE), lses, None, FAKE, None, None), "o_parts"),
    ]
    for args, msg in cases:
        st = _status(lib.cp_attn_merge_lse, *args)
        assert st == B.CP_ERR_INVALID_ARG, (msg, st)
        assert msg in B.last_error(), (msg, B.last_error())


def test_rank_forward_argument_errors():
    lib = B.lib()
    d = _desc()
    P = ctypes.c_void_p
    blocks = (P * 4)(FAKE, FAKE + 256, FAKE + 512, FAKE + 768)
    need = B.cp_attn_workspace_bytes(d)
    S1, S2 = 0x1000, 0x2000     # opaque stream handles, never used (validation fails first)
    cases = [
        ((d.ref, FAKE, blocks, blocks, FAKE, None, None, None, FAKE, need, S1, S2, 8, None),
         B.CP_ERR_INVALID_ARG, "flags"),
        ((d.ref, None, blocks, blocks, FAKE, None, None, None, FAKE, need, S1, S2, 1, None),
         B.CP_ERR_INVALID_ARG, "q is NULL"),
        ((d.ref, FAKE, None, blocks, FAKE, None, None, None, FAKE, need, S1, S2, 1, None),
         B.CP_ERR_INVALID_ARG, "k_blocks"),
        ((d.ref, FAKE, (P * 4)(FAKE, None, FAKE, FAKE), blocks, FAKE, None, None, None, FAKE, need, S1, S2, 1, None),
         B.CP_ERR_INVALID_ARG, "k_blocks[j]"),
        ((d.ref, FAKE, blocks, blocks, FAKE, FAKE + 2, None, None, FAKE, need, S1, S2, 1, None),
         B.CP_ERR_INVALID_ARG, "m_out"),
        ((d.ref, FAKE, blocks, blocks, FAKE, None, None, None, None, need, S1, S2, 1, None),
         B.CP_ERR_WORKSPACE, "workspace is NULL"),
        ((d.ref, FAKE, blocks, blocks, FAKE, None, None, None, FAKE + 16, need, S1, S2, 1, None),
         B.CP_ERR_WORKSPACE, "256-byte"),
        ((d.ref, FAKE, blocks, blocks, FAKE, None, None, None, FAKE, need - 1, S1, S2, 1, None),
         B.CP_ERR_WORKSPACE, "needed"),
        ((d.ref, FAKE, blocks, blocks, FAKE, None, None, None, FAKE, need, S1, S1, 1, None),
         B.CP_ERR_INVALID_ARG, "copy_stream"),
    ]
    for args, status, msg in cases:
        st = _status(lib.cp_attn_rank_forward, *args)
        assert st == status, (msg, st, B.last_error())
        assert msg in B.last_error(), (msg, B.last_error())
    # blocks a causal rank never visits may be NULL: rank 1 of 4 visits 1, 0 only
    d1 = _desc(rank=1)
    st = _status(lib.cp_attn_rank_forward, d1.ref, FAKE, (P * 4)(FAKE, FAKE, None, None), (P * 4)(FAKE, FAKE, None, None),
                 FAKE, None, None, None, FAKE, need - 1, S1, S2, 1, None)
    assert st == B.CP_ERR_WORKSPACE


def test_rank_forward_static_argument_errors():
    """The allocation-free rank forward validates everything, the size of the
    shard's scratch against CP_STATIC_SCRATCH_BYTES included, before its first
    HIP call (these calls fail without a GPU)."""
    lib = B.lib()
    P = ctypes.c_void_p
    blocks = (P * 4)(FAKE, FAKE + 256, FAKE + 512, FAKE + 768)
    S1, S2 = 0x1000, 0x2000
    d = _desc()
    assert B.cp_attn_workspace_bytes(d) <= B.CP_STATIC_SCRATCH_BYTES
    cases = [
        ((d.ref, FAKE, blocks, blocks, FAKE, None, None, None, S1, S2, 8, None), B.CP_ERR_INVALID_ARG, "flags"),
        ((d.ref, None, blocks, blocks, FAKE, None, None, None, S1, S2, 1, None), B.CP_ERR_INVALID_ARG, "q is NULL"),
        ((d.ref, FAKE, blocks, blocks, FAKE, None, None, None, S1, S1, 1, None), B.CP_ERR_INVALID_ARG, "copy_stream"),
    ]
    # the largest bf16 shard that fits, and the next one that does not
    small = _desc(L=4096, H=8)
    big = _desc(L=8192, H=8)
    assert B.cp_attn_workspace_bytes(small) <= B.CP_STATIC_SCRATCH_BYTES < B.cp_attn_workspace_bytes(big)
    cases.append(((big.ref, FAKE, blocks, blocks, FAKE, None, None, None, S1, S2, 1, None), B.CP_ERR_WORKSPACE,
                  "static scratch"))
    for args, status, msg in cases:
        st = _status(lib.cp_attn_rank_forward_static, *args)
        assert st == status, (msg, st, B.last_error())
        assert msg in B.last_error(), (msg, B.last_error())


def test_measure_lds_stream_argument_errors():
    lib = B.lib()
    for args, msg in (((None, 4096, None), "src is NULL"), ((FAKE + 8, 4096, None), "16-byte"),
                      ((FAKE, 0, None), "multiple of 4096"), ((FAKE, 4097, None), "multiple of 4096")):
        assert _status(lib.cp_attn_measure_lds_stream, *args) == B.CP_ERR_INVALID_ARG
        assert msg in B.last_error(), (msg, B.last_error())


def test_host_query_argument_errors():
    lib = B.lib()
    d = _desc()
    buf = (ctypes.c_int32 * 2)()
    cnt = ctypes.c_int32()
    assert _status(lib.cp_attn_ring_schedule, d.ref, 0, buf, 2, ctypes.byref(cnt)) == B.CP_ERR_INVALID_ARG
    assert "capacity" in B.last_error()
    assert _status(lib.cp_attn_ring_schedule, d.ref, 0, buf, 2, None) == B.CP_ERR_INVALID_ARG
    assert _status(lib.cp_attn_ring_schedule, d.ref, 4, buf, 2, ctypes.byref(cnt)) == B.CP_ERR_INVALID_ARG
    assert _status(lib.cp_attn_visible_pairs, d.ref, None) == B.CP_ERR_INVALID_ARG
    assert _status(lib.cp_attn_visible_pairs, None, ctypes.byref(ctypes.c_int64())) == B.CP_ERR_INVALID_ARG
    assert "desc is NULL" in B.last_error()
    h = ctypes.c_void_p()
    assert _status(lib.cp_attn_profiler_create, 0, ctypes.byref(h)) == B.CP_ERR_INVALID_ARG
    assert _status(lib.cp_attn_profiler_reset, None) == B.CP_ERR_INVALID_ARG
    assert _status(lib.cp_attn_profiler_read, None, None, 0, ctypes.byref(cnt)) == B.CP_ERR_INVALID_ARG
    lib.cp_attn_profiler_destroy(None)


def test_status_strings():
    assert B.status_string(0) == "CP_OK"
    assert B.status_string(3) == "CP_ERR_WORKSPACE"
    assert B.status_string(99) == "CP_ERR_UNKNOWN"
    assert B.cp_attn_visible_pairs(_desc()) > 0
    assert B.last_error() == ""


def test_backward_argument_errors():
    d = _desc()
    lib = B.lib()
    F = FAKE
    P = ctypes.c_void_p
    blk = (P * 4)(F, F + 256, F + 512, F + 768)
    bad = (P * 4)(F, F + 256, None, F + 768)
    cases_block = [
        ((d.ref, 4, B.CP_MODE_INIT, F, F, F, F, F, F, F, F, F, None), B.CP_ERR_INVALID_ARG, "block j"),
        ((d.ref, 0, B.CP_MODE_PARTIAL_LSE, F, F, F, F, F, F, F, F, F, None), B.CP_ERR_INVALID_ARG, "INIT or ACCUMULATE"),
        ((d.ref, 0, B.CP_MODE_INIT, None, F, F, F, F, F, F, F, F, None), B.CP_ERR_INVALID_ARG, "q is NULL"),
        ((d.ref, 0, B.CP_MODE_INIT, F, F, F, F + 8, F, F, F, F, F, None), B.CP_ERR_INVALID_ARG, "d_o is not 16-byte"),
        ((d.ref, 0, B.CP_MODE_INIT, F, F, F, F, None, F, F, F, F, None), B.CP_ERR_INVALID_ARG, "lse is NULL"),
        ((d.ref, 0, B.CP_MODE_INIT, F, F, F, F, F, F + 2, F, F, F, None), B.CP_ERR_INVALID_ARG, "delta"),
        ((d.ref, 0, B.CP_MODE_INIT, F, F, F, F, F, F, F + 4, F, F, None), B.CP_ERR_INVALID_ARG, "dq"),
        ((d.ref, 0, B.CP_MODE_INIT, F, F, F, F, F, F, F, None, F, None), B.CP_ERR_INVALID_ARG, "dk_j"),
        ((d.ref, 0, B.CP_MODE_INIT, F, F, F, F, F, F, F, F, None, None), B.CP_ERR_INVALID_ARG, "dv_j"),
    ]
    for args, status, msg in cases_block:
        assert _status(lib.cp_attn_block_backward, *args) == status, (args, B.last_error())
        assert msg in B.last_error(), (msg, B.last_error())
    # f32 descs are refused by every backward entry point
    f = _desc(dtype="f32")
    assert _status(lib.cp_attn_bwd_delta, f.ref, F, F, F, None) == B.CP_ERR_UNSUPPORTED
    assert "bf16" in B.last_error()
    assert _status(lib.cp_attn_block_backward, f.ref, 0, B.CP_MODE_INIT, F, F, F, F, F, F, F, F, F,
                   None) == B.CP_ERR_UNSUPPORTED
    assert _status(lib.cp_attn_rank_backward, f.ref, F, blk, blk, F, F, F, F, F, blk, blk, 0,
                   None) == B.CP_ERR_UNSUPPORTED
    # delta
    assert _status(lib.cp_attn_bwd_delta, d.ref, None, F, F, None) == B.CP_ERR_INVALID_ARG
    assert _status(lib.cp_attn_bwd_delta, d.ref, F, F, F + 1, None) == B.CP_ERR_INVALID_ARG
    # rank driver
    cases_rank = [
        ((d.ref, F, blk, blk, F, F, F, F, F, blk, blk, B.CP_RING_PREFETCH, None), "flags"),
        ((d.ref, F, None, blk, F, F, F, F, F, blk, blk, 0, None), "NULL"),
        ((d.ref, F, blk, blk, F, F, F, F, F, bad, blk, 0, None), "dk_blocks[j]"),
        ((d.ref, F, blk, blk, F, F, F, F, F, blk, bad, 0, None), "dv_blocks[j]"),
        ((d.ref, F, bad, blk, F, F, F, F, F, blk, blk, 0, None), "k_blocks[j]"),
        ((d.ref, F, blk, blk, None, F, F, F, F, blk, blk, 0, None), "o is NULL"),
        ((d.ref, F, blk, blk, F, F, F, None, F, blk, blk, 0, None), "delta"),
    ]
    for args, msg in cases_rank:
        assert _status(lib.cp_attn_rank_backward, *args) == B.CP_ERR_INVALID_ARG, (msg, B.last_error())
        assert msg in B.last_error(), (msg, B.last_error())


def test_ulysses_workspace_bytes():
    """Q, K, V and the output of the whole sequence for H/N heads."""
    d = _desc(N=4, L=32768, rank=3, H=32)
    piece = 1 * 131072 * 8 * 128 * 2
    assert B.cp_attn_ulysses_workspace_bytes(d) == 4 * piece
    d32 = _desc(N=3, L=100, rank=0, H=6, dtype="f32", d=64)
    piece = 300 * 2 * 64 * 4
    assert 4 * piece <= B.cp_attn_ulysses_workspace_bytes(d32) <= 4 * (piece + 255)
    assert B.lib().cp_attn_ulysses_workspace_bytes(_desc(N=4, H=6).ref) == 0
    assert "multiple of N" in B.last_error()


def test_ulysses_argument_errors():
    lib = B.lib()
    d = _desc(N=4, H=8)
    P = ctypes.c_void_p
    sh = (P * 4)(FAKE, FAKE + 256, FAKE + 512, FAKE + 768)
    need = B.cp_attn_ulysses_workspace_bytes(d)
    S1 = 0x1000
    cases = [
        ((_desc(N=4, H=6).ref, sh, sh, sh, sh, None, None, None, FAKE, need, S1), B.CP_ERR_INVALID_ARG, "multiple of N"),
        ((d.ref, None, sh, sh, sh, None, None, None, FAKE, need, S1), B.CP_ERR_INVALID_ARG, "NULL"),
        ((d.ref, sh, sh, sh, None, None, None, None, FAKE, need, S1), B.CP_ERR_INVALID_ARG, "NULL"),
        ((d.ref, sh, (P * 4)(FAKE, FAKE, None, FAKE), sh, sh, None, None, None, FAKE, need, S1),
         B.CP_ERR_INVALID_ARG, "k_shards[i]"),
        ((d.ref, sh, sh, sh, (P * 4)(FAKE, FAKE + 8, FAKE, FAKE), None, None, None, FAKE, need, S1),
         B.CP_ERR_INVALID_ARG, "o_shards[i] is not 16-byte aligned"),
        ((d.ref, sh, sh, sh, sh, None, None, FAKE + 2, FAKE, need, S1), B.CP_ERR_INVALID_ARG, "lse_out"),
        ((d.ref, sh, sh, sh, sh, None, None, None, None, need, S1), B.CP_ERR_WORKSPACE, "workspace is NULL"),
        ((d.ref, sh, sh, sh, sh, None, None, None, FAKE + 16, need, S1), B.CP_ERR_WORKSPACE, "256-byte"),
        ((d.ref, sh, sh, sh, sh, None, None, None, FAKE, need - 1, S1), B.CP_ERR_WORKSPACE, "needed"),
        ((_desc(N=4, H=8, d=96).ref, sh, sh, sh, sh, None, None, None, FAKE, need, S1), B.CP_ERR_UNSUPPORTED, "head dim"),
    ]
    for args, status, msg in cases:
        st = _status(lib.cp_attn_ulysses_forward, *args)
        assert st == status, (msg, st, B.last_error())
        assert msg in B.last_error(), (msg, B.last_error())


def test_quantize_fp8_argument_errors():
    lib = B.lib()
    d = _desc()
    S1 = 0x1000
    KV, QR = B.CP_FP8_KV, B.CP_FP8_QUERY
    cases = [
        ((_desc(dtype="f32").ref, FAKE, KV, FAKE, FAKE, S1), B.CP_ERR_UNSUPPORTED, "bf16"),
        ((d.ref, FAKE, 2, FAKE, FAKE, S1), B.CP_ERR_INVALID_ARG, "unknown FP8 role 2"),
        ((d.ref, FAKE, -1, FAKE, FAKE, S1), B.CP_ERR_INVALID_ARG, "unknown FP8 role -1"),
        ((d.ref, None, QR, FAKE, FAKE, S1), B.CP_ERR_INVALID_ARG, "x is NULL"),
        ((d.ref, FAKE, KV, None, FAKE, S1), B.CP_ERR_INVALID_ARG, "codes is NULL"),
        ((d.ref, FAKE, QR, FAKE + 4, FAKE, S1), B.CP_ERR_INVALID_ARG, "8-byte"),
        ((d.ref, FAKE, KV, FAKE, None, S1), B.CP_ERR_INVALID_ARG, "scales is NULL"),
        ((d.ref, FAKE, QR, FAKE, FAKE + 2, S1), B.CP_ERR_INVALID_ARG, "scales is not 4-byte"),
    ]
    for args, status, msg in cases:
        st = _status(lib.cp_attn_quantize_fp8, *args)
        assert st == status, (msg, st, B.last_error())
        assert msg in B.last_error(), (msg, B.last_error())


def test_header_constants_match_binding():
    """The #define'd flags and roles of include/cpattn.h have the binding's values."""
    import re
    text = open(HEADER).read()
    defs = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define (CP_[A-Z0-9_]+) (-?\d+)\b", text)}
    for name in ("CP_RING_PREFETCH", "CP_RING_REVERSE", "CP_MAX_RING", "CP_FP8_KV", "CP_FP8_QUERY"):
        assert defs[name] == getattr(B, name), name


def test_rank_forward_fp8_argument_errors():
    lib = B.lib()
    d = _desc()
    P = ctypes.c_void_p
    blocks = (P * 4)(FAKE, FAKE + 256, FAKE + 512, FAKE + 768)
    scales = (P * 4)(FAKE + 1024, FAKE + 1280, FAKE + 1536, FAKE + 1792)
    need = B.cp_attn_workspace_bytes(d)
    S1, S2 = 0x1000, 0x2000

    def call(desc=d, q=FAKE, qs=FAKE, kb=blocks, ks=scales, vb=blocks, vs=scales, out=FAKE, m=None, ws=FAKE,
             nbytes=need, cs=S1, xs=S2, flags=1):
        return _status(lib.cp_attn_rank_forward_fp8, desc.ref, q, qs, kb, ks, vb, vs, out, m, None, None, ws,
                       nbytes, cs, xs, flags, None)

    cases = [
        (dict(desc=_desc(dtype="f32")), B.CP_ERR_UNSUPPORTED, "bf16"),
        (dict(qs=None), B.CP_ERR_INVALID_ARG, "q_scale is NULL"),
        (dict(qs=FAKE + 2), B.CP_ERR_INVALID_ARG, "q_scale"),
        (dict(ks=None), B.CP_ERR_INVALID_ARG, "k_scales/v_scales is NULL"),
        (dict(vs=None), B.CP_ERR_INVALID_ARG, "k_scales/v_scales is NULL"),
        (dict(ks=(P * 4)(FAKE, None, FAKE, FAKE)), B.CP_ERR_INVALID_ARG, "k_scales[j]"),
        (dict(vs=(P * 4)(FAKE, FAKE, FAKE + 2, FAKE)), B.CP_ERR_INVALID_ARG, "v_scales[j]"),
        (dict(q=None), B.CP_ERR_INVALID_ARG, "q is NULL"),
        (dict(flags=8), B.CP_ERR_INVALID_ARG, "flags"),
        (dict(m=FAKE + 2), B.CP_ERR_INVALID_ARG, "m_out"),
        (dict(nbytes=need - 1), B.CP_ERR_WORKSPACE, "needed"),
        (dict(xs=S1), B.CP_ERR_INVALID_ARG, "copy_stream"),
    ]
    for kw, status, msg in cases:
        st = call(**kw)
        assert st == status, (msg, st, B.last_error())
        assert msg in B.last_error(), (msg, B.last_error())
    # scales of blocks a causal rank never visits may be NULL: rank 1 of 4 visits 1, 0 only
    d1 = _desc(rank=1)
    st = call(desc=d1, ks=(P * 4)(FAKE, FAKE, None, None), vs=(P * 4)(FAKE, FAKE, None, None),
              kb=(P * 4)(FAKE, FAKE, None, None), vb=(P * 4)(FAKE, FAKE, None, None), nbytes=need - 1)
    assert st == B.CP_ERR_WORKSPACE
