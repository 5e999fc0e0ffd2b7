"""ctypes binding of libcpattn (argument marshalling only).

Every function here has the name of the C entry point it calls and does no
arithmetic of the method: it checks tensor placement, dtype, shape and
contiguity, turns torch tensors into device pointers and torch streams into
hipStream_t handles, and raises ``CpAttnError`` on a non-OK status.  The
library must be built (``python -m context_ring_attention_cp_amd.build``);
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcpattn.so")

CP_OK, CP_ERR_INVALID_ARG, CP_ERR_UNSUPPORTED, CP_ERR_WORKSPACE, CP_ERR_HIP = range(5)
CP_MASK_NONE, CP_MASK_CAUSAL, CP_MASK_DOC_CAUSAL = 0, 1, 2
CP_F32, CP_BF16 = 0, 1
CP_MODE_INIT, CP_MODE_ACCUMULATE, CP_MODE_PARTIAL_LSE = 0, 1, 2
CP_RING_PREFETCH, CP_RING_REVERSE = 1, 2
CP_MAX_RING = 64
CP_FP8_KV, CP_FP8_QUERY = 0, 1
CP_STATIC_SCRATCH_BYTES = 96 << 20

MASKS = {"none": CP_MASK_NONE, "causal": CP_MASK_CAUSAL, "doc_causal": CP_MASK_DOC_CAUSAL}
DTYPES = {"f32": CP_F32, "bf16": CP_BF16}

EXPORTED = [
    "cp_attn_block_partial", "cp_attn_merge_lse", "cp_attn_finalize", "cp_attn_workspace_bytes",
    "cp_attn_rank_forward", "cp_attn_ring_schedule", "cp_attn_visible_pairs",
    "cp_attn_profiler_create", "cp_attn_profiler_reset", "cp_attn_profiler_read",
    "cp_attn_profiler_destroy", "cp_attn_status_string", "cp_attn_last_error",
    "cp_attn_bwd_delta", "cp_attn_block_backward", "cp_attn_rank_backward",
    "cp_attn_ulysses_workspace_bytes", "cp_attn_ulysses_forward", "cp_attn_quantize_fp8",
    "cp_attn_rank_forward_fp8", "cp_attn_rank_forward_static", "cp_attn_profiler_read_copies",
    "cp_attn_measure_lds_stream",
]


class CpAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


class cp_attn_desc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32), ("N", ctypes.c_int32),
        ("L", ctypes.c_int64), ("rank", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("mask", ctypes.c_int32), ("ndocs", ctypes.c_int32),
        ("cu_seqlens", ctypes.POINTER(ctypes.c_int32)), ("cu_seqlens_dev", ctypes.c_void_p),
        ("scale", ctypes.c_float),
    ]


class cp_state(ctypes.Structure):
    _fields_ = [("o", ctypes.c_void_p), ("m", ctypes.c_void_p), ("l", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libcpattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: run `python -m context_ring_attention_cp_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, f32p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        dp = ctypes.POINTER(cp_attn_desc)
        sp = ctypes.POINTER(cp_state)
        L.cp_attn_block_partial.argtypes = [dp, i32, i32, vp, vp, vp, sp, f32p, f32p, vp]
        L.cp_attn_merge_lse.argtypes = [dp, i32, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                        ctypes.POINTER(i32), vp, f32p, vp]
        L.cp_attn_finalize.argtypes = [dp, sp, vp, f32p, f32p, f32p, vp]
        L.cp_attn_workspace_bytes.argtypes = [dp]
        L.cp_attn_workspace_bytes.restype = ctypes.c_size_t
        L.cp_attn_rank_forward.argtypes = [dp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, f32p, f32p,
                                           f32p, vp, ctypes.c_size_t, vp, vp, i32, vp]
        L.cp_attn_rank_forward_static.argtypes = [dp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, f32p, f32p,
                                                  f32p, vp, vp, i32, vp]
        L.cp_attn_ring_schedule.argtypes = [dp, i32, ctypes.POINTER(i32), i32, ctypes.POINTER(i32)]
        L.cp_attn_visible_pairs.argtypes = [dp, ctypes.POINTER(i64)]
        L.cp_attn_profiler_create.argtypes = [i32, ctypes.POINTER(vp)]
        L.cp_attn_profiler_reset.argtypes = [vp]
        L.cp_attn_profiler_read.argtypes = [vp, ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(i32)]
        L.cp_attn_profiler_read_copies.argtypes = [vp, ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(i32)]
        L.cp_attn_measure_lds_stream.argtypes = [vp, ctypes.c_size_t, vp]
        L.cp_attn_profiler_destroy.argtypes = [vp]
        L.cp_attn_profiler_destroy.restype = None
        L.cp_attn_bwd_delta.argtypes = [dp, vp, vp, f32p, vp]
        L.cp_attn_block_backward.argtypes = [dp, i32, i32, vp, vp, vp, vp, f32p, f32p, f32p, f32p, f32p, vp]
        L.cp_attn_rank_backward.argtypes = [dp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, f32p, f32p,
                                            f32p, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp]
        L.cp_attn_ulysses_workspace_bytes.argtypes = [dp]
        L.cp_attn_ulysses_workspace_bytes.restype = ctypes.c_size_t
        L.cp_attn_ulysses_forward.argtypes = [dp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                              ctypes.POINTER(vp), f32p, f32p, f32p, vp, ctypes.c_size_t, vp]
        L.cp_attn_quantize_fp8.argtypes = [dp, vp, ctypes.c_int32, vp, f32p, vp]
        L.cp_attn_rank_forward_fp8.argtypes = [dp, vp, f32p, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                               ctypes.POINTER(vp), ctypes.POINTER(vp), vp, f32p, f32p, f32p, vp,
                                               ctypes.c_size_t, vp, vp, i32, vp]
        L.cp_attn_status_string.argtypes = [i32]
        L.cp_attn_status_string.restype = ctypes.c_char_p
        L.cp_attn_last_error.argtypes = []
        L.cp_attn_last_error.restype = ctypes.c_char_p
        for name in EXPORTED:
            f = getattr(L, name)
            if f.restype is ctypes.c_int:   # default: cp_status as int32
                f.restype = ctypes.c_int32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().cp_attn_status_string(int(status)).decode()


def last_error() -> str:
    return lib().cp_attn_last_error().decode()


def _check(status: int) -> None:
    if status != CP_OK:
        raise CpAttnError(status, last_error())


class Desc:
    """Python owner of a cp_attn_desc and of the host cu_seqlens it points to.

    ``cu_seqlens_dev`` is a device int32 tensor; the Desc holds a reference
    to it, so it lives as long as the Desc (kernels enqueued with the Desc read
    it asynchronously).
    """

    def __init__(self, B: int, H: int, d: int, N: int, L: int, rank: int, dtype: str = "bf16",
                 mask: str = "causal", cu_seqlens: Optional[np.ndarray] = None,
                 cu_seqlens_dev=None, scale: float = 0.0):
        self._cu = None
        self.c = cp_attn_desc()
        self.c.B, self.c.H, self.c.d, self.c.N, self.c.L, self.c.rank = B, H, d, N, L, rank
        self.c.dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
        self.c.mask = MASKS[mask] if isinstance(mask, str) else int(mask)
        self.c.scale = float(scale)
        if cu_seqlens is not None:
            self._cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
            self.c.cu_seqlens = self._cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
            self.c.ndocs = int(self._cu.shape[0] - 1)
        self._cu_dev = cu_seqlens_dev
        if cu_seqlens_dev is not None:
            self.c.cu_seqlens_dev = _ptr(cu_seqlens_dev)
        self.dtype = dtype
        self.mask = mask

    @property
    def ref(self):
        return ctypes.byref(self.c)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return int(t.data_ptr())


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _check_tensor(t, name: str, shape, dtype) -> None:
    import torch
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _io_dtype(desc: Desc):
    import torch
    return torch.bfloat16 if desc.c.dtype == CP_BF16 else torch.float32


def _shapes(desc: Desc):
    c = desc.c
    return (c.B, c.L, c.H, c.d), (c.B, c.H, c.L)


def cp_attn_block_partial(desc: Desc, j: int, mode: int, q, k_j, v_j, state=None, o_part=None,
                          lse_part=None, stream=None) -> None:
    import torch
    big, vec = _shapes(desc)
    dt = _io_dtype(desc)
    for n, t in (("q", q), ("k_j", k_j), ("v_j", v_j)):
        _check_tensor(t, n, big, dt)
    st_ref = None
    if state is not None:
        o, m, l = state
        _check_tensor(o, "state.o", big, torch.float32)
        _check_tensor(m, "state.m", vec, torch.float32)
        _check_tensor(l, "state.l", vec, torch.float32)
        st = cp_state(_ptr(o), _ptr(m), _ptr(l))
        st_ref = ctypes.byref(st)
    _check_tensor(o_part, "o_part", big, torch.float32)
    _check_tensor(lse_part, "lse_part", vec, torch.float32)
    _check(lib().cp_attn_block_partial(desc.ref, int(j), int(mode), _ptr(q), _ptr(k_j), _ptr(v_j), st_ref,
                                       _ptr(o_part), _ptr(lse_part), _stream(stream)))


def cp_attn_merge_lse(desc: Desc, o_parts: Sequence, lse_parts: Sequence, order: Optional[Sequence[int]],
                      out, lse_out=None, stream=None) -> None:
    import torch
    big, vec = _shapes(desc)
    n = len(o_parts)
    if len(lse_parts) != n:
        raise ValueError("o_parts and lse_parts differ in length")
    for t in o_parts:
        _check_tensor(t, "o_parts[j]", big, torch.float32)
    for t in lse_parts:
        _check_tensor(t, "lse_parts[j]", vec, torch.float32)
    _check_tensor(out, "out", big, _io_dtype(desc))
    _check_tensor(lse_out, "lse_out", vec, torch.float32)
    op = (ctypes.c_void_p * n)(*[_ptr(t) for t in o_parts])
    lp = (ctypes.c_void_p * n)(*[_ptr(t) for t in lse_parts])
    od = None if order is None else (ctypes.c_int32 * n)(*[int(x) for x in order])
    _check(lib().cp_attn_merge_lse(desc.ref, n, op, lp, od, _ptr(out), _ptr(lse_out), _stream(stream)))


def cp_attn_finalize(desc: Desc, state, out, m_out=None, l_out=None, lse_out=None, stream=None) -> None:
    import torch
    big, vec = _shapes(desc)
    o, m, l = state
    _check_tensor(o, "state.o", big, torch.float32)
    _check_tensor(m, "state.m", vec, torch.float32)
    _check_tensor(l, "state.l", vec, torch.float32)
    _check_tensor(out, "out", big, _io_dtype(desc))
    for n, t in (("m_out", m_out), ("l_out", l_out), ("lse_out", lse_out)):
        _check_tensor(t, n, vec, torch.float32)
    st = cp_state(_ptr(o), _ptr(m), _ptr(l))
    _check(lib().cp_attn_finalize(desc.ref, ctypes.byref(st), _ptr(out), _ptr(m_out), _ptr(l_out),
                                  _ptr(lse_out), _stream(stream)))


def cp_attn_workspace_bytes(desc: Desc) -> int:
    n = int(lib().cp_attn_workspace_bytes(desc.ref))
    if n == 0:
        raise CpAttnError(CP_ERR_INVALID_ARG, last_error())
    return n


def cp_attn_rank_forward(desc: Desc, q, k_blocks: Sequence, v_blocks: Sequence, out, m_out=None, l_out=None,
                         lse_out=None, workspace=None, compute_stream=None, copy_stream=None,
                         flags: int = CP_RING_PREFETCH, profiler: Optional["Profiler"] = None) -> None:
    import torch
    big, vec = _shapes(desc)
    dt = _io_dtype(desc)
    N = desc.c.N
    if len(k_blocks) != N or len(v_blocks) != N:
        raise ValueError(f"need N={N} K and V block entries (None for blocks that are never visited)")
    _check_tensor(q, "q", big, dt)
    for t in list(k_blocks) + list(v_blocks):
        _check_tensor(t, "k/v block", big, dt)
    _check_tensor(out, "out", big, dt)
    for n, t in (("m_out", m_out), ("l_out", l_out), ("lse_out", lse_out)):
        _check_tensor(t, n, vec, torch.float32)
    if workspace is None or not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise ValueError("workspace must be a device tensor")
    kp = (ctypes.c_void_p * N)(*[_ptr(t) for t in k_blocks])
    vp = (ctypes.c_void_p * N)(*[_ptr(t) for t in v_blocks])
    cs = _stream(compute_stream)
    xs = _stream(copy_stream) if copy_stream is not None else cs
    _check(lib().cp_attn_rank_forward(desc.ref, _ptr(q), kp, vp, _ptr(out), _ptr(m_out), _ptr(l_out),
                                      _ptr(lse_out), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), cs, xs, int(flags),
                                      profiler.handle if profiler is not None else None))


def cp_attn_rank_forward_static(desc: Desc, q, k_blocks: Sequence, v_blocks: Sequence, out, m_out=None,
                                l_out=None, lse_out=None, compute_stream=None, copy_stream=None,
                                flags: int = CP_RING_PREFETCH, profiler: Optional["Profiler"] = None) -> None:
    """cp_attn_rank_forward with the library's static scratch as workspace."""
    import torch
    big, vec = _shapes(desc)
    dt = _io_dtype(desc)
    N = desc.c.N
    if len(k_blocks) != N or len(v_blocks) != N:
        raise ValueError(f"need N={N} K and V block entries (None for blocks that are never visited)")
    _check_tensor(q, "q", big, dt)
    for t in list(k_blocks) + list(v_blocks):
        _check_tensor(t, "k/v block", big, dt)
    _check_tensor(out, "out", big, dt)
    for n, t in (("m_out", m_out), ("l_out", l_out), ("lse_out", lse_out)):
        _check_tensor(t, n, vec, torch.float32)
    kp = (ctypes.c_void_p * N)(*[_ptr(t) for t in k_blocks])
    vp = (ctypes.c_void_p * N)(*[_ptr(t) for t in v_blocks])
    cs = _stream(compute_stream)
    xs = _stream(copy_stream) if copy_stream is not None else cs
    _check(lib().cp_attn_rank_forward_static(desc.ref, _ptr(q), kp, vp, _ptr(out), _ptr(m_out), _ptr(l_out),
                                             _ptr(lse_out), cs, xs, int(flags),
                                             profiler.handle if profiler is not None else None))


def cp_attn_measure_lds_stream(src, stream=None) -> None:
    """Read the bytes of the device tensor `src` once through the global -> LDS
    fetch (a measurement helper: calibrates HBM byte counters)."""
    nbytes = src.numel() * src.element_size()
    _check(lib().cp_attn_measure_lds_stream(_ptr(src), nbytes, _stream(stream)))


def cp_attn_ulysses_workspace_bytes(desc: Desc) -> int:
    n = int(lib().cp_attn_ulysses_workspace_bytes(desc.ref))
    if n == 0:
        raise CpAttnError(CP_ERR_INVALID_ARG, last_error())
    return n


def cp_attn_ulysses_forward(desc: Desc, q_shards: Sequence, k_shards: Sequence, v_shards: Sequence,
                            o_shards: Sequence, m_out=None, l_out=None, lse_out=None, workspace=None,
                            stream=None) -> None:
    import torch
    c = desc.c
    big = (c.B, c.L, c.H, c.d)
    N = c.N
    vec = (c.B, c.H // N if N else 0, c.L * N)
    dt = _io_dtype(desc)
    if not (len(q_shards) == len(k_shards) == len(v_shards) == len(o_shards) == N):
        raise ValueError(f"need N={N} entries in q_shards, k_shards, v_shards and o_shards")
    for t in list(q_shards) + list(k_shards) + list(v_shards) + list(o_shards):
        _check_tensor(t, "shard", big, dt)
    for n, t in (("m_out", m_out), ("l_out", l_out), ("lse_out", lse_out)):
        _check_tensor(t, n, vec, torch.float32)
    if workspace is None or not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise ValueError("workspace must be a device tensor")
    arr = lambda ts: (ctypes.c_void_p * N)(*[_ptr(t) for t in ts])  # noqa: E731
    _check(lib().cp_attn_ulysses_forward(desc.ref, arr(q_shards), arr(k_shards), arr(v_shards), arr(o_shards),
                                         _ptr(m_out), _ptr(l_out), _ptr(lse_out), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)))


def cp_attn_quantize_fp8(desc: Desc, x, codes, scales, stream=None, role: int = CP_FP8_KV) -> None:
    """x: bf16 [B, L, H, d]; codes: uint8 [B, L, H, d]; scales: float32 [B, H];
    role CP_FP8_KV (keys, values) or CP_FP8_QUERY (the query, with the
    softmax's base-2 factor folded in, as cp_attn_rank_forward_fp8 expects)."""
    import torch
    c = desc.c
    big = (c.B, c.L, c.H, c.d)
    _check_tensor(x, "x", big, torch.bfloat16)
    _check_tensor(codes, "codes", big, torch.uint8)
    _check_tensor(scales, "scales", (c.B, c.H), torch.float32)
    if codes is None or scales is None:
        raise ValueError("codes and scales are required")
    _check(lib().cp_attn_quantize_fp8(desc.ref, _ptr(x), int(role), _ptr(codes), _ptr(scales), _stream(stream)))


def cp_attn_rank_forward_fp8(desc: Desc, q, q_scale, k_blocks: Sequence, k_scales: Sequence, v_blocks: Sequence,
                             v_scales: Sequence, out, m_out=None, l_out=None, lse_out=None, workspace=None,
                             compute_stream=None, copy_stream=None, flags: int = CP_RING_PREFETCH,
                             profiler: Optional["Profiler"] = None) -> None:
    """q, k/v blocks: uint8 e4m3 codes [B, L, H, d]; scales float32 [B, H]; out bf16."""
    import torch
    c = desc.c
    big, vec = _shapes(desc)
    N = c.N
    if not (len(k_blocks) == len(v_blocks) == len(k_scales) == len(v_scales) == N):
        raise ValueError(f"need N={N} entries in k_blocks, k_scales, v_blocks and v_scales")
    _check_tensor(q, "q", big, torch.uint8)
    _check_tensor(q_scale, "q_scale", (c.B, c.H), torch.float32)
    for t in list(k_blocks) + list(v_blocks):
        _check_tensor(t, "k/v block", big, torch.uint8)
    for t in list(k_scales) + list(v_scales):
        _check_tensor(t, "k/v scale", (c.B, c.H), torch.float32)
    _check_tensor(out, "out", big, torch.bfloat16)
    for n, t in (("m_out", m_out), ("l_out", l_out), ("lse_out", lse_out)):
        _check_tensor(t, n, vec, torch.float32)
    if workspace is None or not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise ValueError("workspace must be a device tensor")
    arr = lambda ts: (ctypes.c_void_p * N)(*[_ptr(t) for t in ts])  # noqa: E731
    cs = _stream(compute_stream)
    xs = _stream(copy_stream) if copy_stream is not None else cs
    _check(lib().cp_attn_rank_forward_fp8(desc.ref, _ptr(q), _ptr(q_scale), arr(k_blocks), arr(k_scales),
                                          arr(v_blocks), arr(v_scales), _ptr(out), _ptr(m_out), _ptr(l_out),
                                          _ptr(lse_out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          cs, xs, int(flags), profiler.handle if profiler is not None else None))


def cp_attn_bwd_delta(desc: Desc, o, d_o, delta, stream=None) -> None:
    import torch
    big, vec = _shapes(desc)
    _check_tensor(o, "o", big, torch.bfloat16)
    _check_tensor(d_o, "d_o", big, torch.bfloat16)
    _check_tensor(delta, "delta", vec, torch.float32)
    _check(lib().cp_attn_bwd_delta(desc.ref, _ptr(o), _ptr(d_o), _ptr(delta), _stream(stream)))


def cp_attn_block_backward(desc: Desc, j: int, mode: int, q, k_j, v_j, d_o, lse, delta, dq, dk_j, dv_j,
                           stream=None) -> None:
    import torch
    big, vec = _shapes(desc)
    for n, t in (("q", q), ("k_j", k_j), ("v_j", v_j), ("d_o", d_o)):
        _check_tensor(t, n, big, torch.bfloat16)
    for n, t in (("lse", lse), ("delta", delta)):
        _check_tensor(t, n, vec, torch.float32)
    for n, t in (("dq", dq), ("dk_j", dk_j), ("dv_j", dv_j)):
        _check_tensor(t, n, big, torch.float32)
    _check(lib().cp_attn_block_backward(desc.ref, int(j), int(mode), _ptr(q), _ptr(k_j), _ptr(v_j), _ptr(d_o),
                                        _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk_j), _ptr(dv_j),
                                        _stream(stream)))


def cp_attn_rank_backward(desc: Desc, q, k_blocks: Sequence, v_blocks: Sequence, o, d_o, lse, delta, dq,
                          dk_blocks: Sequence, dv_blocks: Sequence, flags: int = 0, stream=None) -> None:
    import torch
    big, vec = _shapes(desc)
    N = desc.c.N
    if not (len(k_blocks) == len(v_blocks) == len(dk_blocks) == len(dv_blocks) == N):
        raise ValueError(f"need N={N} entries in k_blocks, v_blocks, dk_blocks and dv_blocks")
    for n, t in (("q", q), ("o", o), ("d_o", d_o)):
        _check_tensor(t, n, big, torch.bfloat16)
    for t in list(k_blocks) + list(v_blocks):
        _check_tensor(t, "k/v block", big, torch.bfloat16)
    for n, t in (("lse", lse), ("delta", delta)):
        _check_tensor(t, n, vec, torch.float32)
    _check_tensor(dq, "dq", big, torch.float32)
    for t in list(dk_blocks) + list(dv_blocks):
        _check_tensor(t, "dk/dv block", big, torch.float32)
    kp = (ctypes.c_void_p * N)(*[_ptr(t) for t in k_blocks])
    vp = (ctypes.c_void_p * N)(*[_ptr(t) for t in v_blocks])
    dkp = (ctypes.c_void_p * N)(*[_ptr(t) for t in dk_blocks])
    dvp = (ctypes.c_void_p * N)(*[_ptr(t) for t in dv_blocks])
    _check(lib().cp_attn_rank_backward(desc.ref, _ptr(q), kp, vp, _ptr(o), _ptr(d_o), _ptr(lse), _ptr(delta),
                                       _ptr(dq), dkp, dvp, int(flags), _stream(stream)))


def cp_attn_ring_schedule(desc: Desc, flags: int = 0):
    cap = CP_MAX_RING
    buf = (ctypes.c_int32 * cap)()
    cnt = ctypes.c_int32(0)
    _check(lib().cp_attn_ring_schedule(desc.ref, int(flags), buf, cap, ctypes.byref(cnt)))
    return [int(buf[i]) for i in range(cnt.value)]


def cp_attn_visible_pairs(desc: Desc) -> int:
    out = ctypes.c_int64(0)
    _check(lib().cp_attn_visible_pairs(desc.ref, ctypes.byref(out)))
    return int(out.value)


class Profiler:
    """Per-launch timer of the rank forward's attention kernels and ring receives."""

    def __init__(self, capacity: int):
        h = ctypes.c_void_p(None)
        _check(lib().cp_attn_profiler_create(int(capacity), ctypes.byref(h)))
        self.handle = h.value
        self.capacity = capacity

    def reset(self) -> None:
        _check(lib().cp_attn_profiler_reset(self.handle))

    def read(self):
        buf = (ctypes.c_float * self.capacity)()
        cnt = ctypes.c_int32(0)
        _check(lib().cp_attn_profiler_read(self.handle, buf, self.capacity, ctypes.byref(cnt)))
        return [float(buf[i]) for i in range(cnt.value)]

    def read_copies(self):
        buf = (ctypes.c_float * self.capacity)()
        cnt = ctypes.c_int32(0)
        _check(lib().cp_attn_profiler_read_copies(self.handle, buf, self.capacity, ctypes.byref(cnt)))
        return [float(buf[i]) for i in range(cnt.value)]

    def close(self) -> None:
        if self.handle:
            lib().cp_attn_profiler_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass
