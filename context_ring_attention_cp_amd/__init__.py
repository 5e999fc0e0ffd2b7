"""MI355X-native context-parallel ring attention, one rank's shard.

Python binding of libcpattn (HIP kernels for gfx950 behind a C ABI, declared
in include/cpattn.h).  The binding only marshals arguments; every step of the
computation runs in the library's kernels.
"""
from ._binding import (  # noqa: F401
    CP_BF16, CP_ERR_HIP, CP_ERR_INVALID_ARG, CP_ERR_UNSUPPORTED, CP_ERR_WORKSPACE, CP_F32, CP_FP8_KV, CP_FP8_QUERY,
    CP_MASK_CAUSAL,
    CP_MASK_DOC_CAUSAL, CP_MASK_NONE, CP_MAX_RING, CP_MODE_ACCUMULATE, CP_MODE_INIT, CP_MODE_PARTIAL_LSE,
    CP_OK, CP_RING_PREFETCH, CP_RING_REVERSE, CP_STATIC_SCRATCH_BYTES, EXPORTED, CpAttnError, Desc, Profiler, cp_attn_block_backward,
    cp_attn_block_partial, cp_attn_bwd_delta, cp_attn_finalize, cp_attn_measure_lds_stream, cp_attn_merge_lse, cp_attn_quantize_fp8,
    cp_attn_rank_backward, cp_attn_rank_forward, cp_attn_rank_forward_fp8, cp_attn_rank_forward_static, cp_attn_ring_schedule,
    cp_attn_ulysses_forward, cp_attn_ulysses_workspace_bytes, cp_attn_visible_pairs, cp_attn_workspace_bytes,
    last_error, lib, status_string,
)


def alloc_workspace(desc: Desc):
    """A device byte tensor of cp_attn_workspace_bytes(desc) (256-byte aligned by the allocator)."""
    import torch
    return torch.empty(cp_attn_workspace_bytes(desc), dtype=torch.uint8, device="cuda")


def alloc_ulysses_workspace(desc: Desc):
    """A device byte tensor of cp_attn_ulysses_workspace_bytes(desc)."""
    import torch
    return torch.empty(cp_attn_ulysses_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
