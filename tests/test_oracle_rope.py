"""Pins for the oracle's rotary position embedding (CPU).

Technical review of arXiv 2606.08382, section 5.3 ("keys are harder"):
pre-RoPE latent keys are kept and reconstruction, rotation and scoring are
fused at runtime (Algorithm 2, steps 4b-4c).  The RoPE variant is the
half-split pairing of LLaMA-family models (channel i with i + d_h/2, angle
pos * theta^(-2i/d_h)).  Pinned by:
* position 0 is the identity; a hand-placed example fixes the pairing and
  the frequency of each pair (an interleaved pairing or a wrong exponent
  fails it);
* each rotation preserves norms and rotations compose additively
  (R_p R_q = R_{p+q});
* scores depend on positions only through j - t (shift invariance);
* decode with RoPE equals a scalar-loop implementation (math.cos/sin per
  pair) on tiny shapes, with GQA;
* rope_theta = 0 is the unrotated oracle;
* chunked causal prefill with RoPE: a scalar-loop implementation on a tiny
  shape (query i at position ctx + i sees positions 0 .. ctx + i), and each
  prefill row equals the RoPE decode of the same query over the prefix it
  sees.
"""

import math

import numpy as np
import pytest

from oracle import attention as oa
from oracle import cache as oc


def test_position_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((5, 16))
    assert np.array_equal(oa.rope(x, 0, 10000.0), x)


def test_hand_placed_pairing_and_frequencies():
    base, p = 100.0, 3.0
    e0 = np.array([1.0, 0.0, 0.0, 0.0])
    e1 = np.array([0.0, 1.0, 0.0, 0.0])
    e3 = np.array([0.0, 0.0, 0.0, 1.0])
    assert np.allclose(oa.rope(e0, p, base), [math.cos(p), 0, math.sin(p), 0], atol=1e-15)
    w = p * base ** -0.5                       # pair 1: theta^(-2/4)
    assert np.allclose(oa.rope(e1, p, base), [0, math.cos(w), 0, math.sin(w)], atol=1e-15)
    assert np.allclose(oa.rope(e3, p, base), [0, -math.sin(w), 0, math.cos(w)], atol=1e-15)


def test_rotation_is_orthogonal_and_composes():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 32))
    for p, q in ((5, 9), (1000, 31000), (0, 77)):
        y = oa.rope(x, p, 10000.0)
        assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
        assert np.allclose(oa.rope(y, q, 10000.0), oa.rope(x, p + q, 10000.0), atol=1e-9)


def test_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for t, j, shift in ((10, 3, 1000), (32767, 0, -32767), (5, 5, 123456)):
        a = oa.rope(q, t, 500000.0) @ oa.rope(k, j, 500000.0)
        b = oa.rope(q, t + shift, 500000.0) @ oa.rope(k, j + shift, 500000.0)
        assert abs(a - b) <= 1e-9 * (1 + abs(a))


def _rot_scalar(v, pos, theta):
    d = len(v)
    h = d // 2
    out = list(v)
    for i in range(h):
        a = pos * theta ** (-2.0 * i / d)
        c, s = math.cos(a), math.sin(a)
        out[i] = v[i] * c - v[i + h] * s
        out[i + h] = v[i] * s + v[i + h] * c
    return out


@pytest.mark.parametrize("hq,hkv,t", [(2, 2, 9), (4, 2, 40), (2, 1, 1)])
def test_decode_with_rope_brute_force(hq, hkv, t):
    rng = np.random.default_rng(t)
    d, rk, rv, theta, scale = 6, 3, 5, 100.0, 0.7
    c = oc.Cache(1, hkv, rk, rv, 64, "f32")
    zk = rng.standard_normal((1, t, hkv, rk)).astype(np.float32)
    zv = rng.standard_normal((1, t, rv)).astype(np.float32)
    c.append(zk, zv, 0, t)
    bk = rng.standard_normal((hkv, d, rk))
    bv = rng.standard_normal((hkv * d, rv))
    q = rng.standard_normal((1, hq, d))
    out = oa.decode(c, t, q, bk, bv, scale, hq, rotate=False, rope_theta=theta)
    g = hq // hkv
    for h in range(hq):
        kv = h // g
        qr = _rot_scalar(list(q[0, h]), t - 1, theta)
        sc = []
        for j in range(t):
            k = [sum(float(zk[0, j, kv, r]) * bk[kv, i, r] for r in range(rk)) for i in range(d)]
            kr = _rot_scalar(k, j, theta)
            sc.append(scale * sum(a * b for a, b in zip(qr, kr)))
        m = max(sc)
        e = [math.exp(x - m) for x in sc]
        for i in range(d):
            v = sum(e[j] * sum(float(zv[0, j, r]) * bv[kv * d + i, r] for r in range(rv))
                    for j in range(t)) / sum(e)
            assert abs(v - out[0, h, i]) <= 1e-12 * max(1.0, abs(v))


def test_rope_theta_zero_is_the_unrotated_oracle():
    rng = np.random.default_rng(3)
    c = oc.Cache(1, 2, 4, 6, 64, "f32")
    c.append(rng.standard_normal((1, 30, 2, 4)).astype(np.float32),
             rng.standard_normal((1, 30, 6)).astype(np.float32), 0, 30)
    bk, bv = rng.standard_normal((2, 8, 4)), rng.standard_normal((16, 6))
    q = rng.standard_normal((1, 2, 8))
    a = oa.decode(c, 30, q, bk, bv, 0.5, 2, rotate=False)
    b = oa.decode(c, 30, q, bk, bv, 0.5, 2, rotate=False, rope_theta=0.0)
    assert np.array_equal(a, b)
    r = oa.decode(c, 30, q, bk, bv, 0.5, 2, rotate=False, rope_theta=10000.0)
    assert np.abs(r - a).max() > 1e-3      # and RoPE does change the result


@pytest.mark.parametrize("hq,hkv,ctx,c", [(2, 2, 5, 4), (4, 2, 0, 6), (2, 1, 9, 3)])
def test_causal_prefill_with_rope_brute_force(hq, hkv, ctx, c):
    rng = np.random.default_rng(ctx * 7 + c)
    d, rk, rv, theta, scale = 6, 3, 5, 50.0, 0.6
    t = ctx + c
    cache = oc.Cache(1, hkv, rk, rv, 64, "f32")
    zk = rng.standard_normal((1, t, hkv, rk)).astype(np.float32)
    zv = rng.standard_normal((1, t, rv)).astype(np.float32)
    cache.append(zk, zv, 0, t)
    bk = rng.standard_normal((hkv, d, rk))
    bv = rng.standard_normal((hkv * d, rv))
    q = rng.standard_normal((c, hq, d))
    out = oa.causal_attention(cache, ctx, q, bk, bv, scale, hq, False, rope_theta=theta)
    g = hq // hkv
    for i in range(c):
        for h in range(hq):
            kv = h // g
            qr = _rot_scalar(list(q[i, h]), ctx + i, theta)
            sc = []
            for j in range(ctx + i + 1):
                k = [sum(float(zk[0, j, kv, r]) * bk[kv, e, r] for r in range(rk))
                     for e in range(d)]
                kr = _rot_scalar(k, j, theta)
                sc.append(scale * sum(a * b for a, b in zip(qr, kr)))
            m = max(sc)
            ex = [math.exp(x - m) for x in sc]
            for e in range(d):
                v = sum(ex[j] * sum(float(zv[0, j, r]) * bv[kv * d + e, r] for r in range(rv))
                        for j in range(ctx + i + 1)) / sum(ex)
                assert abs(v - out[i, h, e]) <= 1e-12 * max(1.0, abs(v))


def test_prefill_rows_with_rope_equal_rope_decode():
    rng = np.random.default_rng(11)
    hq, hkv, d, rk, rv, ctx, c, theta = 4, 2, 8, 4, 6, 37, 29, 10000.0
    cache = oc.Cache(1, hkv, rk, rv, 128, "f32")
    cache.append(rng.standard_normal((1, ctx + c, hkv, rk)).astype(np.float32),
                 rng.standard_normal((1, ctx + c, rv)).astype(np.float32), 0, ctx + c)
    bk, bv = rng.standard_normal((hkv, d, rk)), rng.standard_normal((hkv * d, rv))
    q = rng.standard_normal((c, hq, d))
    rows = [0, 1, 13, 28]
    out = oa.causal_attention(cache, ctx, q, bk, bv, 0.4, hq, False, rows=rows,
                              rope_theta=theta)
    for ri, i in enumerate(rows):
        dec = oa.decode(cache, ctx + i + 1, q[i][None], bk, bv, 0.4, hq, False,
                        rope_theta=theta)
        assert np.allclose(out[ri], dec[0], atol=1e-12)
    plain = oa.causal_attention(cache, ctx, q, bk, bv, 0.4, hq, False, rows=rows)
    assert np.abs(plain - out).max() > 1e-3
