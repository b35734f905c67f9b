"""Pins for per-head key ranks in the oracle's unquantized caches (CPU).

Technical review of arXiv 2606.08382, section 4 / Fig. 2: the learned key
ranks differ per head; eq. 15 sums the per-head ranks in the cache size.
Pinned by: uniform ranks give the bytes of the plain layout; a hand-derived
byte position for ragged ranks; the cache size of eq. 15; and decode with
ragged ranks equals decode of a uniform-rank cache whose extra channels are
zero (a head of rank r uses only its first r latent channels and factor
columns).
"""

import math

import numpy as np
import pytest

from oracle import attention as oa
from oracle import cache as oc


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_uniform_ranks_give_the_plain_layout(kind):
    rng = np.random.default_rng(0)
    zk = rng.standard_normal((2, 70, 4, 16)).astype(np.float32)
    zv = rng.standard_normal((2, 70, 64)).astype(np.float32)
    a = oc.Cache(2, 4, 16, 64, 128, kind)
    b = oc.Cache(2, 4, 16, 64, 128, kind, key_ranks=[16] * 4)
    a.append(zk, zv, 0, 70)
    b.append(zk, zv, 0, 70)
    for k in a.buf:
        assert np.array_equal(a.buf[k], b.buf[k])


def test_hand_derived_position_with_ragged_ranks():
    # B=2, ranks [8, 16], fp32, one tile: element (b=1, head 1, token 3,
    # channel 9) sits at 64*(1*24 + 8) + (0*2 + 1)*512 + 3*8 + 1 = 2585
    c = oc.Cache(2, 2, 16, 32, 64, "f32", key_ranks=[8, 16])
    zk = np.zeros((2, 4, 2, 16), np.float32)
    zk[1, 3, 1, 9] = 7.0
    zk[0, 2, 0, 12] = 5.0          # past head 0's rank: not stored
    c.append(zk, np.zeros((2, 4, 32), np.float32), 0, 4)
    f = c.buf["key"].view(np.float32)
    assert f.size == 2 * 64 * 24
    assert f[2585] == 7.0 and np.count_nonzero(f) == 1
    lat = c.key_latents(1, 4)
    assert lat[3, 1, 9] == 7.0 and np.count_nonzero(lat) == 1


def test_cache_size_is_eq15_sum_of_head_ranks():
    sz = oc.layout(3, 4, 64, 256, 640, "bf16", key_ranks=[8, 64, 24, 40])
    assert sz["key"] == 3 * 640 * (8 + 64 + 24 + 40) * 2
    assert sz["value"] == 3 * 640 * 256 * 2


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_ragged_ranks_equal_zero_padded_uniform(kind):
    rng = np.random.default_rng(1)
    ranks = [8, 24, 16, 32]
    B, H, Hq, d, R, T = 2, 4, 8, 16, 64, 150
    zk = rng.standard_normal((B, T, H, 32)).astype(np.float32)
    zv = rng.standard_normal((B, T, R)).astype(np.float32)
    ragged = oc.Cache(B, H, 32, R, 192, kind, key_ranks=ranks)
    ragged.append(zk, zv, 0, T)
    zk0 = zk.copy()
    for g, r in enumerate(ranks):
        zk0[:, :, g, r:] = 0.0
    uni = oc.Cache(B, H, 32, R, 192, kind)
    uni.append(zk0, zv, 0, T)
    bk = rng.standard_normal((H, d, 32))
    bv = rng.standard_normal((H * d, R))
    q = rng.standard_normal((B, Hq, d))
    a = oa.decode(ragged, T, q, bk, bv, 1 / math.sqrt(d), Hq, False)
    b = oa.decode(uni, T, q, bk, bv, 1 / math.sqrt(d), Hq, False)
    assert np.allclose(a, b, atol=1e-12, rtol=0)
    # the factor columns past a head's rank play no part
    bk2 = bk.copy()
    for g, r in enumerate(ranks):
        bk2[g, :, r:] = 1e3
    assert np.allclose(oa.decode(ragged, T, q, bk2, bv, 1 / math.sqrt(d), Hq, False), a,
                       atol=1e-12, rtol=0)
