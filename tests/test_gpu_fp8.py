"""GPU parity of the FP8 (e4m3) path against the oracle (oracle/fp8.py).

Quantisation is byte work, so its bar is bit-exact: every code and every
float32 scale equals the oracle's, on ragged lengths (L not a multiple of
the 256 rows a workgroup covers), both head dims, heads of very different
magnitudes, an all-zero head, and a full-size 128K block (all scales, codes
of sampled rows).
"""
import numpy as np
import pytest

import oracle.fp8 as F
from harness.inputs import TENSOR_K, ShardSpec, draw_shard
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


def _quantize_gpu(cp, x, d):
    B, L, H, _ = x.shape
    desc = cp.Desc(B, H, d, 1, L, 0, "bf16", "none")
    codes = torch.empty((B, L, H, d), dtype=torch.uint8, device="cuda")
    scales = torch.full((B, H), float("nan"), device="cuda")
    cp.cp_attn_quantize_fp8(desc, dev(x, "bf16"), codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("L", [1, 300, 513])
def test_quantize_bit_exact(cp, d, L):
    rng = np.random.default_rng(L + d)
    x = rng.standard_normal((2, L, 4, d)).astype(np.float32) * np.array([1.0, 1e-3, 50.0, 1.0], np.float32)[None, None, :, None]
    x[1, :, 3, :] = 0.0                                   # one all-zero (b, h)
    x[0, 0, 0, :4] = [0.0, -0.0, 1e-30, -1e-30]           # zeros and values far below the smallest code
    from harness.inputs import round_to_bf16
    x = round_to_bf16(x)
    say(f"[fp8 quantize] L={L} d={d}")
    codes, scales = _quantize_gpu(cp, x, d)
    ref = F.quantize_heads(x)
    assert np.array_equal(scales.view(np.uint32), ref["scale"].view(np.uint32)), "scales differ"
    bad = np.argwhere(codes != ref["codes"])
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0].tolist()}: gpu {codes[tuple(bad[0])]:#x} " \
                          f"oracle {ref['codes'][tuple(bad[0])]:#x}"


def test_quantize_full_size_block(cp):
    """One K block of the 128K example (L = 32768, H = 32, d = 128)."""
    spec = ShardSpec(S=131072, N=4, H=32, d=128, dtype="bf16", mask="causal", cfg_id=3)
    x = draw_shard(spec, 0, TENSOR_K, 2)
    codes, scales = _quantize_gpu(cp, x, 128)
    amax = np.abs(x).max(axis=(1, 3))
    ref_scale = (amax / np.float32(448)).astype(np.float32)
    assert np.array_equal(scales.view(np.uint32), ref_scale.view(np.uint32)), "scales differ"
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 32767], np.random.default_rng(5).integers(0, 32768, 64)]))
    inv = (np.float32(448) / amax).astype(np.float32)
    y = np.clip(x[:, rows] * inv[:, None, :, None], -448, 448).astype(np.float32)
    ref_codes = F.e4m3_encode(y)
    assert np.array_equal(codes[:, rows], ref_codes), "codes of sampled rows differ"
