"""CPU oracle for the FP8 (e4m3) variant of one rank's shard.

TEST INFRASTRUCTURE ONLY.  This module is the correctness reference for the
HIP library's FP8 entry points.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call it; the
product path never does.  It shares no code with the HIP path (it imports
numpy, the standard library and the forward oracle).

What the pages fix: the compassingai.com context-parallelism page notes that
the bytes CP moves depend on whether the exchanged blocks are compressed or
sent in FP8 (section "通訊量分析"), and that FlashAttention-3 computes
attention in FP8 (section "技術演進史").  They fix no format or scaling; the
readings below are this library's choices:

* format: OCP FP8 E4M3 (1 sign bit, 4 exponent bits with bias 7, 3 mantissa
  bits, largest finite value 448, no infinities), the format of the
  matrix-core FP8 inputs on MI355X;
* scaling: one scale per (batch, head) and tensor block, a power of two.
  With y = float32(x * c), where c = 1 for keys and values and, for the
  query, c is the softmax scale times log2(e) in float32 (``query_prescale``),
  amax is the largest |y| over the block's tokens and head dim and
  scale = 2^e, e the smallest integer >= -126 with amax <= 448 * 2^e
  (e = 0 when amax = 0); the code of x is the e4m3 value nearest to
  y * 2^-e (at most 448 in magnitude by the choice of e), ties to the even
  code, and it stands for decode(code) * scale / c.  Powers of two are what
  the matrix core's block-scale operands apply exactly, and with c folded
  into the query the products of query and key codes come out as base-2
  logits;
* attention: the forward of the shard (oracle ``attention.rank_attention``)
  on the dequantised Q, K and V, computed in float64.  The GPU kernel also
  rounds P to e4m3 for the P V product; that is an approximation of this
  definition, covered by the parity tolerance (as the bf16 kernel's rounding
  of P to bf16 is).

Functions: ``e4m3_values`` (the value table), ``e4m3_decode``,
``e4m3_encode`` (nearest value, ties to even, over the finite codes),
``query_prescale`` (c of the query), ``scale_exponent`` (e of an amax),
``quantize_heads`` (scale and codes of a [B, L, H, d] block),
``dequantize_heads``, ``fp8_rank_attention``.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from . import attention as fwd

__all__ = ["E4M3_MAX", "LOG2E", "e4m3_values", "e4m3_decode", "e4m3_encode", "query_prescale", "scale_exponent",
           "quantize_heads", "dequantize_heads", "fp8_rank_attention"]

E4M3_MAX = 448.0
LOG2E = 1.4426950408889634        # log2(e), rounded to float32 where it is used


def e4m3_values() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    out = np.empty(256)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            out[c] = np.nan
            continue
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        out[c] = -v if s else v
    return out


_VALUES = e4m3_values()
_POS = _VALUES[:0x7F]                 # codes 0x00 .. 0x7E: 0 .. 448, increasing


def e4m3_decode(codes) -> np.ndarray:
    return _VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Code of the e4m3 value nearest to x (|x| <= 448), ties to the even
    code (the code whose mantissa's last bit is 0); the sign bit is x's."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX) or np.any(np.isnan(x)):
        raise ValueError("e4m3_encode takes finite |x| <= 448 (clamp first)")
    ax = np.abs(x)
    hi = np.searchsorted(_POS, ax, side="left")          # first code with value >= |x|
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = ax - _POS[lo]
    d_hi = _POS[hi] - ax
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(ax == _POS[hi], hi, code)             # exact values
    # the sign bit follows x, also when the magnitude rounds to 0 (-0 is 0x80)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def query_prescale(d: int, scale: Optional[float] = None) -> np.float32:
    """c of the query: float32(s * float32(log2 e)), with s = float32(scale),
    or float32(1 / float32(sqrt(d))) when scale is None or not positive; each
    operation rounded to float32."""
    if scale is None or scale <= 0:
        s = np.float32(1) / np.sqrt(np.float32(d))
    else:
        s = np.float32(scale)
    return np.float32(np.float32(s) * np.float32(LOG2E))


def scale_exponent(amax) -> np.ndarray:
    """e of each amax: the smallest integer >= -126 with amax <= 448 * 2^e
    (0 where amax == 0), found by counting up from -126; the comparisons are
    exact in float64."""
    a = np.asarray(amax, dtype=np.float64)
    out = np.zeros(a.shape, dtype=np.int64)
    for idx, v in np.ndenumerate(a):
        if v > 0:
            e = -126
            while v > E4M3_MAX * 2.0 ** e:
                e += 1
            out[idx] = e
    return out


def quantize_heads(x, prescale=1.0) -> Dict[str, np.ndarray]:
    """Scale and codes of a block x [B, L, H, d] (float32 values, e.g. the
    bf16 inputs) multiplied by ``prescale`` (c): per (b, h) amax of
    y = float32(x * c) over tokens and head dim; returns ``codes``
    [B, L, H, d] uint8 and ``scale`` [B, H] float32 (2^e)."""
    x = np.asarray(x, dtype=np.float32)
    y = (x * np.float32(prescale)).astype(np.float32)      # one float32 rounding (none when c = 1)
    amax = np.abs(y).max(axis=(1, 3))                      # [B, H], exact
    e = scale_exponent(amax)
    scale = np.exp2(e.astype(np.float64)).astype(np.float32)
    z = y.astype(np.float64) * np.exp2(-e.astype(np.float64))[:, None, :, None]   # exact
    z = np.clip(z, -E4M3_MAX, E4M3_MAX)
    return {"codes": e4m3_encode(z), "scale": scale}


def dequantize_heads(codes, scale, prescale=1.0) -> np.ndarray:
    """float64 values decode(code) * scale / c, [B, L, H, d]."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[:, None, :, None] / float(prescale)


def fp8_rank_attention(q_codes, q_scale, k_codes: Sequence, k_scales: Sequence, v_codes: Sequence,
                       v_scales: Sequence, rank: int, N: int, mask: str, cu_seqlens=None,
                       scale: Optional[float] = None, rows=None, heads=None,
                       q_prescale=1.0) -> Dict[str, np.ndarray]:
    """The shard's forward on the dequantised inputs (float64), the query's
    codes standing for decode * q_scale / q_prescale; blocks not supplied
    (None) must be invisible to the shard, as in ``rank_attention``."""
    q = dequantize_heads(q_codes, q_scale, q_prescale)
    ks = {j: dequantize_heads(k_codes[j], k_scales[j]) for j in range(N) if k_codes[j] is not None}
    vs = {j: dequantize_heads(v_codes[j], v_scales[j]) for j in range(N) if v_codes[j] is not None}
    return fwd.rank_attention(q, ks, vs, rank, N, mask, cu_seqlens, scale, rows=rows, heads=heads)
