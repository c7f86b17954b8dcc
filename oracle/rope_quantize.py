"""CPU oracle for the MLA RoPE + FP8 quantize producer (test infrastructure only).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg do.  It shares no code with the HIP library.

What it computes follows the MATE documentation of mla_rope_quantize_fp8
(the MATE native sparse-MLA API page, "RoPE and FP8 quantization"; the MATE
FlashInfer-compatibility wrapper page, same section):

  R1  rotary embedding of the 64-value RoPE tails of q (per head) and k, in
      float32, with the cosine / sine of the token's position taken from a
      [max_seq_len, 64] cache (columns 0..31 cosines, 32..63 sines); is_neox
      rotates the two contiguous 32-value halves, otherwise adjacent
      even/odd pairs;
  R2  per-tensor quantization: every value of q (its 512-value latent and its
      rotated tail) times quant_scale_q, every value of k times
      quant_scale_kv, then cast to FP8 E4M3.

Readings taken where the pages are silent:
  * pair i (i = 0..31) -- values (i, i + 32) for is_neox, (2i, 2i + 1)
    otherwise -- turns by the angle of cache column i:
        a' = a cos_i - b sin_i,   b' = b cos_i + a sin_i;
  * "the rotary arithmetic in float32" is taken as each product, sum and
    the scale multiplication rounded to float32 on its own (no fused
    multiply-add), so the float32 value each code is cast from is fixed;
  * the cast rounds to the nearest finite E4M3 value, ties to the even code,
    and saturates: magnitudes beyond 448, infinities included, become +-448;
    zero keeps its sign;
  * a NaN value is cast to a NaN code (OCP E4M3: 0x7F or 0xFF; this oracle
    writes 0x7F, and which of the two a NaN becomes is not part of the
    result), so a bad activation is not turned into a large finite key;
  * a position outside [0, max_seq_len) is the caller's error (the library
    writes NaN codes for that token's rotated tails).
"""
from __future__ import annotations

import numpy as np

from .bsr_attention import e4m3fn_decode

__all__ = ["e4m3fn_encode", "rope_fp32", "mla_rope_quantize_fp8"]

# the 127 non-negative finite E4M3 values, code order (0x00 .. 0x7E), increasing
_POS_VALUES = e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3fn_encode(values) -> np.ndarray:
    """R2: float values -> E4M3 codes (uint8): nearest finite value, ties to the even
    code, magnitudes above 448 (and infinities) saturated to 448, the sign bit from the
    value's sign; NaN -> the NaN code 0x7F."""
    v = np.asarray(values, dtype=np.float64)
    nan = np.isnan(v)
    mag = np.minimum(np.abs(np.where(nan, 0.0, v)), _POS_VALUES[-1])
    hi = np.clip(np.searchsorted(_POS_VALUES, mag, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    return np.where(nan, np.uint8(0x7F), code).astype(np.uint8)


def rope_fp32(x, cos, sin, is_neox: bool) -> np.ndarray:
    """R1: rotate the last axis (64 values) of x by per-row angles.

    x: float32 (..., 64); cos, sin: float32 broadcastable to (..., 32).  Every
    product and sum is a float32 operation of its own."""
    x = np.asarray(x, dtype=np.float32)
    cos = np.asarray(cos, dtype=np.float32)
    sin = np.asarray(sin, dtype=np.float32)
    if x.shape[-1] != 64:
        raise ValueError("the RoPE tail has 64 values")
    if is_neox:
        a, b = x[..., :32], x[..., 32:]
    else:
        a, b = x[..., 0::2], x[..., 1::2]
    a_rot = (a * cos) - (b * sin)
    b_rot = (b * cos) + (a * sin)
    out = np.empty_like(x)
    if is_neox:
        out[..., :32], out[..., 32:] = a_rot, b_rot
    else:
        out[..., 0::2], out[..., 1::2] = a_rot, b_rot
    return out


def mla_rope_quantize_fp8(q_rope, k_rope, q_nope, k_nope, cos_sin_cache, pos_ids, is_neox: bool = True,
                          quant_scale_q: float = 1.0, quant_scale_kv: float = 1.0):
    """R1 + R2.  q_rope (nnz, H, 64), k_rope (nnz, 64), q_nope (nnz, H, 512), k_nope
    (nnz, 512): float32 arrays holding the BF16 inputs' values; cos_sin_cache
    (max_seq_len, 64) float32 (the values of an FP32 or BF16 cache); pos_ids (nnz,).
    Returns the E4M3 codes (q_rope_out, k_rope_out, q_nope_out, k_nope_out) as uint8."""
    cache = np.asarray(cos_sin_cache, dtype=np.float32)
    pos = np.asarray(pos_ids, dtype=np.int64)
    if cache.ndim != 2 or cache.shape[1] != 64:
        raise ValueError("cos_sin_cache must be (max_seq_len, 64)")
    if ((pos < 0) | (pos >= cache.shape[0])).any():
        raise ValueError("positions must lie in [0, max_seq_len)")
    cos, sin = cache[pos, :32], cache[pos, 32:]
    sq, skv = np.float32(quant_scale_q), np.float32(quant_scale_kv)
    q_rot = rope_fp32(q_rope, cos[:, None, :], sin[:, None, :], is_neox)
    k_rot = rope_fp32(k_rope, cos, sin, is_neox)
    return (e4m3fn_encode(q_rot * sq), e4m3fn_encode(k_rot * skv),
            e4m3fn_encode(np.asarray(q_nope, dtype=np.float32) * sq),
            e4m3fn_encode(np.asarray(k_nope, dtype=np.float32) * skv))
