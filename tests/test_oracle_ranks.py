"""Pins for per-head key ranks in the oracle's caches (CPU).

Technical review of arXiv 2606.08382, section 4 / Fig. 2: the learned key
ranks differ per head; eq. 15 sums the per-head ranks in the cache size.
Pinned by: uniform ranks give the bytes of the plain layout; a hand-derived
byte position for ragged ranks; the cache size of eq. 15; and decode with
ragged ranks equals decode of a uniform-rank cache whose extra channels are
zero (a head of rank r uses only its first r latent channels and factor
columns).

Quantized (q43) caches keep each head's 32-channel key tile and zero the
channels past its rank (section 6.2: rank rounding to a supported kernel
tile, the padding term of eq. 15).  Pinned by: the tile sizes do not change;
input in the padded channels never reaches the bytes; without rotation the
padded channels read back within half a quantization step of zero; and
decode equals decode of an fp32 cache with the same ragged ranks that holds
the q43 cache's own read-out, unrotated (so nothing in the padded channels,
nor any factor column past a rank, reaches a score).
"""

import math

import numpy as np
import pytest

from oracle import attention as oa
from oracle import cache as oc
from oracle import hadamard


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


Q_RANKS = [8, 24, 16, 32]


def _q43_pair(rotate, lo_bits=3, seed=2):
    rng = np.random.default_rng(seed)
    B, H, R, T = 2, 4, 256, 150
    zk = rng.standard_normal((B, T, H, 32)).astype(np.float32)
    zv = rng.standard_normal((B, T, R)).astype(np.float32) * 0.5
    c = oc.Cache(B, H, 32, R, 192, "q43", rotate, key_ranks=Q_RANKS, lo_bits=lo_bits)
    c.append(zk, zv, 0, T)
    return c, zk, zv


def test_q43_ranks_keep_the_tile_layout():
    for lob in (3, 4):
        assert oc.layout(2, 4, 32, 256, 192, "q43", key_ranks=Q_RANKS, lo_bits=lob) == \
            oc.layout(2, 4, 32, 256, 192, "q43", lo_bits=lob)


@pytest.mark.parametrize("rotate", [False, True])
def test_q43_input_past_a_rank_never_reaches_the_bytes(rotate):
    c, zk, zv = _q43_pair(rotate)
    zk0 = zk.copy()
    for g, r in enumerate(Q_RANKS):
        zk0[:, :, g, r:] = 0.0
    # a uniform-rank cache fed the zero-padded latents stores the same bytes
    u = oc.Cache(2, 4, 32, 256, 192, "q43", rotate)
    u.append(zk0, zv, 0, 150)
    for k in c.buf:
        assert np.array_equal(c.buf[k], u.buf[k]), k
    # and a cache whose ranks are all 32 stores the unpadded latents
    full = oc.Cache(2, 4, 32, 256, 192, "q43", rotate, key_ranks=[32] * 4)
    full.append(zk, zv, 0, 150)
    plain = oc.Cache(2, 4, 32, 256, 192, "q43", rotate)
    plain.append(zk, zv, 0, 150)
    for k in full.buf:
        assert np.array_equal(full.buf[k], plain.buf[k]), k


def test_q43_padded_channels_read_back_near_zero():
    """Without rotation a padded channel is a zero in its token's 3-bit
    group: its read-out is within half of that group's step of 0."""
    c, _, _ = _q43_pair(False)
    lat = c.key_latents(1, 150)
    _, km, _, _ = c._q_views()
    scale_lo = km[1].reshape(4, -1, 4)[:, :150, 2].view(np.float16).astype(np.float64)
    for g, r in enumerate(Q_RANKS):
        if r < 32:
            dev_ = np.abs(lat[:, g, r:]).max(axis=1)
            assert np.all(dev_ <= scale_lo[g] / 2 * (1 + 2 ** -10)), g


@pytest.mark.parametrize("rotate,lo_bits", [(True, 3), (False, 3), (True, 4)])
def test_q43_ranks_equal_fp32_ranks_on_the_read_out(rotate, lo_bits):
    c, _, _ = _q43_pair(rotate, lo_bits)
    B, H, Hq, d, R, T = 2, 4, 8, 16, 256, 150
    rk_rot = hadamard.rotation_matrix(8, 24) if rotate else np.eye(32)
    rv_rot = hadamard.rotation_matrix(64, 192) if rotate else np.eye(R)
    f = oc.Cache(B, H, 32, R, 192, "f32", key_ranks=Q_RANKS)
    zk = np.stack([c.key_latents(b, T) @ rk_rot for b in range(B)]).astype(np.float32)
    zv = np.stack([c.value_latents(b, T) @ rv_rot for b in range(B)]).astype(np.float32)
    f.append(zk, zv, 0, T)
    rng = np.random.default_rng(3)
    bk = rng.standard_normal((H, d, 32))
    for g, r in enumerate(Q_RANKS):
        bk[g, :, r:] = 1e3 * rng.standard_normal((d, 32 - r))   # columns that do not exist
    bv = rng.standard_normal((H * d, R))
    q = rng.standard_normal((B, Hq, d)) * 2
    s = 1 / math.sqrt(d)
    a = oa.decode(c, T, q, bk, bv, s, Hq, rotate)
    b = oa.decode(f, T, q, bk, bv, s, Hq, False)
    # the fp32 cache rounds the read-out to float32
    assert np.allclose(a, b, atol=1e-5 * np.abs(b).max(), rtol=0)
