"""Asymmetric group quantizer with fp16 scale and zero point.

Technical review of arXiv 2606.08382, section 6.1 (eq. 14 and the text before
it): the leading channels of the retained latent are stored at 4 bits and the
rest at 3 bits; the quality experiments use a 20:80 split and the community
checkpoint card a `top_fraction=0.25` recipe.  The pages do not give the
quantizer's arithmetic.  Readings taken (all emulated bit-for-bit here in IEEE
float32 / float16, so that the GPU packer can match it exactly):

* a group is up to 32 consecutive channels of one token inside one precision
  block (groups never straddle the 4-bit / 3-bit boundary);
* lo = min, hi = max of the group (exact in float32);
* zero z = fp16(lo) rounded toward -inf;
* scale s = fp16(fp32(fp32(hi - z) / L)) rounded toward +inf, L = 2^bits - 1;
* code = clamp(rint_half_even(fp32(fp32(x - z) / s)), 0, L); s == 0 gives 0;
* dequantized value x_hat = z + s * code (evaluated in float64 here).

Directed rounding guarantees z <= lo and z + L*s >= hi up to float32 rounding,
hence |x - x_hat| <= s/2 up to that rounding.
"""

from __future__ import annotations

import numpy as np


def _f16_step(bits: np.ndarray, down: bool) -> np.ndarray:
    """Move fp16 bit patterns one representable value down (or up)."""
    bits = bits.astype(np.uint16)
    neg = (bits & 0x8000) != 0
    mag = bits & 0x7FFF
    out = bits.copy()
    if down:
        # positive non-zero: magnitude - 1; zero (either sign): -min_denormal;
        # negative: magnitude + 1
        out = np.where(~neg & (mag != 0), bits - 1, out)
        out = np.where(mag == 0, np.uint16(0x8001), out)
        out = np.where(neg & (mag != 0), bits + 1, out)
    else:
        out = np.where(~neg, bits + 1, out)
        out = np.where(neg & (mag != 0), bits - 1, out)
        out = np.where(neg & (mag == 0), np.uint16(0x0001), out)
    return out.astype(np.uint16)


def fp16_round_down(x: np.ndarray) -> np.ndarray:
    """float32 -> fp16 bits, rounded toward -inf."""
    x = np.asarray(x, dtype=np.float32)
    h = x.astype(np.float16)
    bits = h.view(np.uint16)
    over = h.astype(np.float32) > x
    return np.where(over, _f16_step(bits, True), bits).astype(np.uint16)


def fp16_round_up(x: np.ndarray) -> np.ndarray:
    """float32 -> fp16 bits, rounded toward +inf."""
    x = np.asarray(x, dtype=np.float32)
    h = x.astype(np.float16)
    bits = h.view(np.uint16)
    under = h.astype(np.float32) < x
    return np.where(under, _f16_step(bits, False), bits).astype(np.uint16)


def f16(bits: np.ndarray) -> np.ndarray:
    """fp16 bit patterns -> float32 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def quantize(x: np.ndarray, bits: int):
    """Quantize groups along the last axis.

    x: float32 [..., n] (one group per leading index).
    Returns codes uint8 [..., n], scale fp16 bits [...], zero fp16 bits [...].
    """
    x = np.asarray(x, dtype=np.float32)
    levels = np.float32((1 << bits) - 1)
    lo = x.min(axis=-1)
    hi = x.max(axis=-1)
    zbits = fp16_round_down(lo)
    zf = f16(zbits)
    s32 = (hi - zf).astype(np.float32) / levels
    sbits = fp16_round_up(s32.astype(np.float32))
    sf = f16(sbits)
    num = (x - zf[..., None]).astype(np.float32)
    safe = np.where(sf == 0, np.float32(1), sf)
    q = np.rint((num / safe[..., None]).astype(np.float32))
    q = np.clip(q, 0, levels)
    q = np.where((sf == 0)[..., None], np.float32(0), q)
    return q.astype(np.uint8), sbits, zbits


def dequantize(codes: np.ndarray, sbits: np.ndarray, zbits: np.ndarray):
    """x_hat = z + s * code in float64 (scale/zero broadcast over the group)."""
    s = f16(sbits).astype(np.float64)
    z = f16(zbits).astype(np.float64)
    return z[..., None] + s[..., None] * codes.astype(np.float64)
