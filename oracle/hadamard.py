"""Block-wise Walsh-Hadamard rotation of the latent channels.

Technical review of arXiv 2606.08382, section 6.1: the retained channels are
split into an outlier block (the leading, high-precision channels) and an
inlier block, each rotated independently; eq. 13 states Z U^T = (Z H)(H^T U^T)
with H H^T = I, so the down-projection side absorbs H and the up-projection
side absorbs H^T.

The pages do not say how a block whose width is not a power of two is rotated.
Reading taken: a block of n channels uses I_{n/m} (x) H_m, with H_m the
normalised Sylvester-Hadamard matrix and m the largest power of two dividing n
(keys: 8 + 3x8 channels; values: 256 + 3x256, or 64 + 3x64 for the GQA shape).

The stored latent is defined as the float32 fast transform below (butterfly
strides 1, 2, 4, ..., each (a, b) -> (a + b, a - b) rounded to float32, then
one float32 multiply by the float32 value nearest 1/sqrt(m)), so that the
packed cache is reproducible to the bit.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def sylvester(m: int) -> np.ndarray:
    """Normalised Sylvester-Hadamard matrix H_m (float64), H_m H_m^T = I."""
    assert m >= 1 and m & (m - 1) == 0
    h = np.ones((1, 1))
    while h.shape[0] < m:
        h = np.block([[h, h], [h, -h]])
    return h / math.sqrt(m)


def pow2_block(n: int) -> int:
    """Largest power of two dividing n."""
    return n & -n


def block_matrix(n: int) -> np.ndarray:
    """I_{n/m} (x) H_m for a precision block of n channels (float64)."""
    m = pow2_block(n)
    return np.kron(np.eye(n // m), sylvester(m))


def rotation_matrix(n_hi: int, n_lo: int) -> np.ndarray:
    """Rotation of one latent vector: hi block then lo block, block-diagonal."""
    r = np.zeros((n_hi + n_lo, n_hi + n_lo))
    r[:n_hi, :n_hi] = block_matrix(n_hi)
    r[n_hi:, n_hi:] = block_matrix(n_lo)
    return r


def inv_sqrt_f32(m: int) -> np.float32:
    """The float32 value nearest to 1/sqrt(m) (checked exactly)."""
    c = np.float32(1.0 / math.sqrt(m))
    # exact check: c is within half an ulp of 1/sqrt(m), i.e. the neighbours
    # of c are farther; compare squares as rationals.
    fc = Fraction(float(c))
    up = Fraction(float(np.nextafter(c, np.float32(2))))
    dn = Fraction(float(np.nextafter(c, np.float32(0))))
    target2 = Fraction(1, m)
    mid_up2 = ((fc + up) / 2) ** 2
    mid_dn2 = ((fc + dn) / 2) ** 2
    assert mid_dn2 <= target2 <= mid_up2, "1/sqrt(m) rounding check failed"
    return c


def fwht_f32(x: np.ndarray, m: int) -> np.ndarray:
    """Float32 fast Walsh-Hadamard transform in consecutive blocks of m along
    the last axis (the definition of a stored rotated latent)."""
    y = np.array(x, dtype=np.float32, copy=True)
    n = y.shape[-1]
    assert n % m == 0
    shp = y.shape
    y = y.reshape(-1, n // m, m)
    h = 1
    while h < m:
        v = y.reshape(y.shape[0], y.shape[1], m // (2 * h), 2, h)
        a = v[:, :, :, 0, :].copy()
        b = v[:, :, :, 1, :].copy()
        v[:, :, :, 0, :] = a + b
        v[:, :, :, 1, :] = a - b
        h *= 2
    y = y * inv_sqrt_f32(m)
    return y.reshape(shp).astype(np.float32)


def rotate_latent_f32(z: np.ndarray, n_hi: int) -> np.ndarray:
    """Rotate float32 latents [..., n_hi + n_lo] block-wise (stored form)."""
    z = np.asarray(z, dtype=np.float32)
    n_lo = z.shape[-1] - n_hi
    out = np.empty_like(z)
    out[..., :n_hi] = fwht_f32(z[..., :n_hi], pow2_block(n_hi))
    out[..., n_hi:] = fwht_f32(z[..., n_hi:], pow2_block(n_lo))
    return out
