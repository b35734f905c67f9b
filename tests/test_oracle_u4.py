"""Pins for the oracle's uniform 4-bit cache (lo_bits = 4; CPU).

The technical review of arXiv 2606.08382 measures its speed with a 4-bit
latent cache (section 6.1 after eq. 14; section 8).  Same precision blocks,
groups and rotation as the 4/3-bit cache, every group at 4 bits.  Pinned by:
hand-derived byte positions of single codes (key nibble planes, value runs),
unpack(pack) = id, the eq. 15 size with 4 bits per channel, the element-wise
read-out bound with 4-bit scales, and an unquantized-cache comparison
(uniform 4-bit is closer to the exact latents than 4/3-bit).
"""

import math

import numpy as np

import synth
from oracle import attention as oa
from oracle import cache as oc
from oracle import hadamard, quant


def test_key_nibble_planes_hand_derived():
    # code 0xB for token 5, channel 19 -> plane 2 (channels 16..23), nibble 3:
    # byte 2*256 + 4*5 + 1 (bits 12..15 = high nibble of byte 1 of the word)
    codes = np.zeros((1, 64, 32), np.uint8)
    codes[0, 5, 19] = 0xB
    blob = oc.pack_key_tiles(codes, lo_bits=4)[0]
    want = np.zeros(1024, np.uint8)
    want[512 + 4 * 5 + 1] = 0xB0
    assert np.array_equal(blob, want)
    assert np.array_equal(oc.unpack_key_tiles(blob[None], 4), codes)


def test_value_runs_hand_derived():
    # R_v = 128: group 3 (channels 96..127, 4-bit with lo_bits 4) starts at
    # byte 3 * 1024; token 37 = half 1, u = 5: word 0, bit 16*(5%2) + 4*(5//2)
    # = 24; channel 100 = c 4: run at (32*1 + 4) * 16 bytes into the group
    codes = np.zeros((1, 64, 128), np.uint8)
    codes[0, 37, 100] = 0x9
    blob = oc.pack_value_tiles(codes, lo_bits=4)[0]
    want = np.zeros(32 * 128, np.uint8)
    want[3 * 1024 + 36 * 16 + 3] = 0x09       # bit 24 = byte 3, low nibble
    assert np.array_equal(blob, want)
    assert np.array_equal(oc.unpack_value_tiles(blob[None], 128, 4), codes)


def test_pack_unpack_roundtrip_and_size():
    rng = np.random.default_rng(0)
    k = rng.integers(0, 16, (5, 64, 32)).astype(np.uint8)
    v = rng.integers(0, 16, (3, 64, 256)).astype(np.uint8)
    assert np.array_equal(oc.unpack_key_tiles(oc.pack_key_tiles(k, 4), 4), k)
    assert np.array_equal(oc.unpack_value_tiles(oc.pack_value_tiles(v, 4), 256, 4), v)
    lay = oc.layout(16, 32, 32, 1024, 32768, "q43", lo_bits=4)
    payload = 16 * 32768 * 4 // 8 * (32 * 32 + 1024)        # eq. 15, 4 bits
    meta = 16 * 32768 * (32 * 2 + 1024 // 32) * 4
    assert lay["key"] + lay["value"] == payload
    assert lay["key_meta"] + lay["value_meta"] == meta
    assert sum(lay.values()) == 16 * 32768 * 1408


def test_readout_within_half_a_4bit_step():
    w = synth.WORKLOADS["l2_q4"].replace(batch=1, n_q_heads=4, n_kv_heads=4,
                                         value_rank=256)
    zk, zv = synth.batch_latents(w, 0, 100)
    c = oc.Cache.for_workload(w, max_tokens=128, fill=0xFF)
    c.append(zk, zv, 0, 100)
    rk = hadamard.rotate_latent_f32(zk, 8)[0]
    rv = hadamard.rotate_latent_f32(zv, 64)[0]
    kh = quant.quantize(rk[..., :8], 4)
    kl = quant.quantize(rk[..., 8:], 4)
    got = c.key_latents(0, 100)
    s = np.concatenate([np.repeat(quant.f16(kh[1])[..., None], 8, -1),
                        np.repeat(quant.f16(kl[1])[..., None], 24, -1)], -1)
    assert np.all(np.abs(got - rk) <= s / 2 * (1 + 2.0 ** -18))
    vq = quant.quantize(rv.reshape(100, 8, 32), 4)
    sv = np.repeat(quant.f16(vq[1]), 32, axis=-1).reshape(100, 256)
    assert np.all(np.abs(c.value_latents(0, 100) - rv) <= sv / 2 * (1 + 2.0 ** -18))


def test_uniform_4bit_halves_the_trailing_block_error():
    """The trailing block's step is range/15 instead of range/7: its mean
    read-out error falls by about half; the leading block is unchanged."""
    base = synth.WORKLOADS["l2_q43"].replace(batch=1, n_q_heads=8, n_kv_heads=8,
                                             value_rank=256)
    zk, zv = synth.batch_latents(base, 0, 256)
    rk = hadamard.rotate_latent_f32(zk, 8)[0]
    rv = hadamard.rotate_latent_f32(zv, 64)[0]
    err = {}
    for lob in (3, 4):
        c = oc.Cache(1, 8, 32, 256, 256, "q43", rotate=True, lo_bits=lob)
        c.append(zk, zv, 0, 256)
        ek = np.abs(c.key_latents(0, 256) - rk)
        ev = np.abs(c.value_latents(0, 256) - rv)
        err[lob] = (ek[..., :8].mean(), ek[..., 8:].mean(), ev[:, :64].mean(), ev[:, 64:].mean())
    assert err[4][0] == err[3][0] and err[4][2] == err[3][2]
    assert err[4][1] < 0.6 * err[3][1] and err[4][3] < 0.6 * err[3][3]
