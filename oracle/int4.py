"""4-bit KV-cache encoding (test infrastructure; see package doc).

The pages say only that the method composes with 4-bit KV-cache quantization
(xllm-io review, section 五 量化组合; paperlayer summary, section 1
Compatibility); they give no scheme. The workload fixes per-token, per-head,
per-32-channel fp16 scale and zero-point. The reading used here, step by step,
for each group x[0..31] of one token and one head (values upcast to float32):

  mn = min x, mx = max x
  s  = fp16_round((mx - mn) / 15)          float32 subtract and IEEE divide
  z  = fp16_round(mn)                      the zero-point is an fp16 offset
  c  = clamp(rint((x - f32(z)) / f32(s)), 0, 15)   rint ties to even; c = 0 if s == 0
  x^ = fma(c, f32(s), f32(z))              one rounding to float32

The codes are integer decisions taken in float32, the precision the GPU
quantiser uses, so both sides must agree bit for bit. Packing: byte b of a
token's 64-byte row holds channel 2b in the low nibble and channel 2b+1 in the
high nibble.
"""
from __future__ import annotations

import numpy as np

GROUP = 32


def quantize_int4_g32(x):
    """x [..., D] (float values, D % 32 == 0) -> (codes u8 [..., D], s f16 [..., D/32],
    z f16 [..., D/32]). Codes are unpacked (one per channel)."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    if D % GROUP:
        raise ValueError("head_dim must be a multiple of 32")
    g = x.reshape(x.shape[:-1] + (D // GROUP, GROUP))
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    s16 = ((mx - mn) / np.float32(15.0)).astype(np.float32).astype(np.float16)
    z16 = mn.astype(np.float16)
    s32 = s16.astype(np.float32)[..., None]
    z32 = z16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (g - z32).astype(np.float32) / s32
    c = np.clip(np.rint(t), 0.0, 15.0)
    c = np.where(s32 == 0, 0.0, c)
    codes = c.astype(np.uint8).reshape(x.shape)
    return codes, s16, z16


def dequantize_int4_g32(codes, s16, z16) -> np.ndarray:
    """x^ = fma(c, s, z) in float32, one rounding: the exact product-sum is
    formed in float64 (a 4-bit times an 11-bit significand plus an fp16 value
    is exact there) and rounded once to float32."""
    codes = np.asarray(codes)
    D = codes.shape[-1]
    c = codes.reshape(codes.shape[:-1] + (D // GROUP, GROUP)).astype(np.float64)
    exact = c * np.asarray(s16, np.float64)[..., None] + np.asarray(z16, np.float64)[..., None]
    return exact.astype(np.float32).reshape(codes.shape)


def pack_nibbles(codes) -> np.ndarray:
    """[..., D] codes in 0..15 -> [..., D/2] bytes, even channel in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = codes[..., 0::2]
    hi = codes[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out
