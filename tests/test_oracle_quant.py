"""Pins for the oracle's quantizer and rotation (CPU only).

Quantizer: technical review of arXiv 2606.08382, section 6.1 (4-bit leading
channels, 3-bit rest); rotation: same section, eq. 13.  The pins are the
hand-derived examples under tests/golden/, an exhaustive search over all fp16
values for the directed rounding, the round-trip bound |x - x_hat| <= s/2, and
the orthogonality and matrix form of the Walsh-Hadamard transform.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import hadamard, quant

GOLD = os.path.join(os.path.dirname(__file__), "golden")

_ALL_F16 = np.arange(0x10000, dtype=np.uint16)
_F16_VALS = _ALL_F16.view(np.float16).astype(np.float64)
_FINITE = np.isfinite(_F16_VALS)


def _brute_down(x):
    """Largest finite fp16 value <= x, by exhaustive search (value only)."""
    ok = _FINITE & (_F16_VALS <= float(x))
    return _F16_VALS[ok].max()


def _brute_up(x):
    ok = _FINITE & (_F16_VALS >= float(x))
    return _F16_VALS[ok].min()


def test_golden_quantizer_examples():
    ex = json.load(open(os.path.join(GOLD, "quantizer_examples.json")))["examples"]
    for e in ex:
        x = np.array(e["x"], np.float32)
        codes, s, z = quant.quantize(x[None], e["bits"])
        assert int(z[0]) == int(e["zero"], 16), e
        assert int(s[0]) == int(e["scale"], 16), e
        assert codes[0].tolist() == e["codes"], e


def test_directed_rounding_matches_exhaustive_search():
    rng = np.random.default_rng(1)
    xs = np.concatenate([
        rng.standard_normal(400) * 10.0 ** rng.integers(-9, 4, 400),
        rng.uniform(-1, 1, 200) * 6e-5,           # subnormal fp16 range
        np.array([0.0, -0.0, 1.0, -1.0, 0.1, 65504.0, -65504.0, 6.1e-5]),
    ]).astype(np.float32)
    down = quant.f16(quant.fp16_round_down(xs)).astype(np.float64)
    up = quant.f16(quant.fp16_round_up(np.abs(xs))).astype(np.float64)
    for x, d, u in zip(xs, down, up):
        assert d == _brute_down(x), x
        assert u == _brute_up(abs(x)), x


def _groups(rng, n_groups, width):
    base = rng.standard_normal((n_groups, width))
    scale = 10.0 ** rng.uniform(-3, 1.5, (n_groups, 1))
    shift = rng.standard_normal((n_groups, 1)) * scale * 3
    x = base * scale + shift
    x[:5, 3] *= 40.0                               # outliers
    return x.astype(np.float32)


@pytest.mark.parametrize("bits,width", [(4, 8), (3, 24), (4, 32), (3, 32)])
def test_round_trip_bound_and_code_range(bits, width):
    rng = np.random.default_rng(bits * 100 + width)
    x = _groups(rng, 3000, width)
    codes, s, z = quant.quantize(x, bits)
    assert codes.max() <= (1 << bits) - 1
    xh = quant.dequantize(codes, s, z)
    sf = quant.f16(s).astype(np.float64)
    err = np.abs(x.astype(np.float64) - xh)
    bound = sf[:, None] / 2 * (1 + 2.0 ** -18)
    assert np.all(err <= bound)
    # zero point never above the group minimum, top level reaches the max
    zf = quant.f16(z).astype(np.float64)
    assert np.all(zf <= x.min(axis=1))
    top = zf + ((1 << bits) - 1) * sf
    mx = x.max(axis=1).astype(np.float64)
    assert np.all(top >= mx - np.abs(mx) * 2.0 ** -20 - 1e-30)


@pytest.mark.parametrize("bits", [3, 4])
def test_requantize_is_identity(bits):
    rng = np.random.default_rng(7 + bits)
    x = _groups(rng, 500, 32)
    codes, s, z = quant.quantize(x, bits)
    xh = quant.dequantize(codes, s, z).astype(np.float32)
    zf = quant.f16(z)[:, None]
    sf = quant.f16(s)[:, None]
    again = np.clip(np.rint(((xh - zf).astype(np.float32) / sf).astype(np.float32)),
                    0, (1 << bits) - 1)
    assert np.array_equal(again.astype(np.uint8), codes)


@pytest.mark.parametrize("bits", [3, 4])
def test_every_code_reached_by_a_ramp(bits):
    L = (1 << bits) - 1
    x = (np.arange(L + 1, dtype=np.float32) * np.float32(0.25) - 1)[None]
    codes, s, z = quant.quantize(x, bits)
    assert codes[0].tolist() == list(range(L + 1))


def test_constant_groups():
    # fp16-representable constant: scale 0, all codes 0, exact reconstruction
    x = np.full((3, 8), 1.5, np.float32)
    x[1] = -0.25
    x[2] = 0.0
    codes, s, z = quant.quantize(x, 4)
    assert np.all(s == 0) and np.all(codes == 0)
    assert np.array_equal(quant.dequantize(codes, s, z), x.astype(np.float64))
    # non-representable constant: tiny positive scale, within s/2
    y = np.full((1, 24), 0.1, np.float32)
    codes, s, z = quant.quantize(y, 3)
    assert s[0] != 0
    err = abs(quant.dequantize(codes, s, z)[0, 0] - np.float64(np.float32(0.1)))
    assert err <= quant.f16(s)[0] / 2


# -------------------------------------------------------------- Hadamard --

@pytest.mark.parametrize("m", [1, 2, 8, 64, 256])
def test_sylvester_orthonormal(m):
    h = hadamard.sylvester(m)
    assert np.allclose(h @ h.T, np.eye(m), atol=1e-15, rtol=0)
    assert np.allclose(np.abs(h), 1 / math.sqrt(m), atol=1e-16, rtol=0)
    assert np.array_equal(h, h.T)


def test_inv_sqrt_constants_are_nearest_floats():
    for m, hexv in [(8, 0x3EB504F3), (32, 0x3E3504F3), (128, 0x3DB504F3),
                    (256, 0x3D800000), (64, 0x3E000000)]:
        c = hadamard.inv_sqrt_f32(m)
        assert int(np.float32(c).view(np.uint32)) == hexv
        err = abs(Fraction(float(c)) ** 2 - Fraction(1, m))
        assert err < Fraction(1, m) * Fraction(1, 2 ** 22)


@pytest.mark.parametrize("m", [8, 64, 256])
def test_fwht_matches_matrix_and_unit_vectors(m):
    rng = np.random.default_rng(m)
    x = rng.standard_normal((50, 3 * m)).astype(np.float32)
    y = hadamard.fwht_f32(x, m)
    ref = x.astype(np.float64) @ np.kron(np.eye(3), hadamard.sylvester(m))
    tol = math.log2(m) * 2.0 ** -23 * np.abs(x).sum(axis=1, keepdims=True) + 1e-30
    assert np.all(np.abs(y - ref) <= tol)
    # unit vectors map to the rows of H exactly when 1/sqrt(m) is a power of 2
    if m in (64, 256):
        e = np.eye(m, dtype=np.float32)
        assert np.array_equal(hadamard.fwht_f32(e, m).astype(np.float64),
                              hadamard.sylvester(m))


def test_fwht_is_an_involution_up_to_rounding():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((20, 256)).astype(np.float32)
    back = hadamard.fwht_f32(hadamard.fwht_f32(x, 256), 256)
    assert np.allclose(back, x, atol=1e-5, rtol=0)


def test_block_rotation_structure_and_eq13():
    """Eq. 13: Z U^T = (Z H)(H^T U^T) for the block-diagonal rotation."""
    r = hadamard.rotation_matrix(8, 24)
    assert np.allclose(r @ r.T, np.eye(32), atol=1e-15)
    assert np.all(r[:8, 8:] == 0) and np.all(r[8:, :8] == 0)
    assert np.all(r[8:16, 16:] == 0)           # lo block is I_3 (x) H_8
    assert hadamard.pow2_block(24) == 8 and hadamard.pow2_block(768) == 256
    rng = np.random.default_rng(3)
    z = rng.standard_normal((40, 32))
    u = rng.standard_normal((128, 32))
    assert np.allclose((z @ r) @ (u @ r).T, z @ u.T, atol=1e-12, rtol=0)
    rv = hadamard.rotation_matrix(256, 768)
    assert np.allclose(rv @ rv.T, np.eye(1024), atol=1e-14)


def test_rotate_latent_matches_block_matrix():
    rng = np.random.default_rng(9)
    z = rng.standard_normal((10, 1024)).astype(np.float32)
    got = hadamard.rotate_latent_f32(z, 256)
    ref = z.astype(np.float64) @ hadamard.rotation_matrix(256, 768)
    assert np.allclose(got, ref, atol=1e-5, rtol=0)
