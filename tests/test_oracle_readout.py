"""Pins for the oracle's latent projection and its quantized read-out (CPU).

* project_latents is Algorithm 2, step 1 of the technical review of arXiv
  2606.08382 (project the hidden state into latent keys and values), in the
  row-vector convention of eq. 2: Z = X A, the key columns of A laid out
  [D][Hkv * r_k] with KV head g owning columns g r_k .. g r_k + r_k - 1.
  Pinned by scalar loops on a tiny shape and by the placement of one
  hand-chosen element (a transposed A or a reshape in the wrong order puts
  it elsewhere).
* The quantized read-out (unpack + dequantize, section 6.1, eq. 13 and 14)
  of a rotated 4/3-bit cache is pinned element by element: every entry is
  exactly zero + scale * code of its own group (scale and zero the fp16
  values the quantizer chose for that token and group) and lies within
  (s/2)(1 + 2^-18) of the rotated latent it stores.  A group index off by
  one, a swapped scale and zero, or a token shifted by one fails both.
Each pin is also run against planted mistakes in a copy of the oracle, to
show that it catches them.
"""

import numpy as np
import pytest

import synth
from oracle import attention as oa
from oracle import cache as oc
from oracle import hadamard, quant


# ------------------------------------------------------- projection pins --

def _check_projection(project):
    """Raise AssertionError unless `project` is Z = X A with the key columns
    split per KV head."""
    rng = np.random.default_rng(11)
    c, d, hkv, rk, rv = 3, 5, 2, 3, 4
    x = rng.standard_normal((c, d)).astype(np.float32)
    ak = rng.standard_normal((d, hkv * rk)).astype(np.float32)
    av = rng.standard_normal((d, rv)).astype(np.float32)
    zk, zv = project(x, ak, av, hkv, rk)
    assert zk.shape == (c, hkv, rk) and zv.shape == (c, rv)
    for i in range(c):
        for g in range(hkv):
            for r in range(rk):
                want = sum(float(x[i, k]) * float(ak[k, g * rk + r]) for k in range(d))
                assert abs(float(zk[i, g, r]) - want) <= 1e-6 * max(1.0, abs(want))
        for r in range(rv):
            want = sum(float(x[i, k]) * float(av[k, r]) for k in range(d))
            assert abs(float(zv[i, r]) - want) <= 1e-6 * max(1.0, abs(want))
    # one hand-placed element: row 1 of X is e_3, A_key[3, g=1, r=2] = 7,
    # so latent (token 1, KV head 1, channel 2) is 7 and every other key
    # latent of token 1 is 0
    x = np.zeros((c, d), np.float32)
    x[1, 3] = 1.0
    ak = np.zeros((d, hkv * rk), np.float32)
    ak[3, 1 * rk + 2] = 7.0
    zk, _ = project(x, ak, np.zeros((d, rv), np.float32), hkv, rk)
    want = np.zeros((c, hkv, rk))
    want[1, 1, 2] = 7.0
    assert np.array_equal(zk, want)


def test_project_latents_pinned():
    _check_projection(oa.project_latents)


def _transposed_a(x, a_key, a_value, n_kv_heads, key_rank):
    # A read as [Hkv * r_k][D] reinterpreted: the columns come out permuted
    zk = np.asarray(x, np.float64) @ np.asarray(a_key, np.float64).reshape(
        -1, a_key.shape[0]).T.reshape(a_key.shape)
    zv = np.asarray(x, np.float64) @ np.asarray(a_value, np.float64)
    return (zk.astype(np.float32).reshape(x.shape[0], n_kv_heads, key_rank),
            zv.astype(np.float32))


def _head_major_reshape(x, a_key, a_value, n_kv_heads, key_rank):
    # columns taken channel-major instead of head-major
    zk, zv = oa.project_latents(x, a_key, a_value, n_kv_heads, key_rank)
    return zk.reshape(x.shape[0], key_rank, n_kv_heads).transpose(0, 2, 1), zv


@pytest.mark.parametrize("mutant", [_transposed_a, _head_major_reshape])
def test_projection_pin_catches_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        _check_projection(mutant)


# --------------------------------------------------------- read-out pins --

def _rotated_q43_cache(seq_len=150, value_rank=256, seed=3):
    w = synth.WORKLOADS["l2_q43"].replace(batch=2, n_q_heads=4, n_kv_heads=4,
                                          value_rank=value_rank, seed=seed)
    zk, zv = synth.batch_latents(w, 0, seq_len)
    cache = oc.Cache(2, 4, 32, value_rank, 256, "q43", rotate=True, fill=0xFF)
    cache.append(zk, zv, 0, seq_len)
    return cache, zk, zv


def _expected_groups(zk, zv, value_rank):
    """Rotated latents and, per entry, the fp16 scale / zero / code the
    quantizer chose for its own group (keys: channels 0-7 and 8-31 of a head;
    values: 32-channel groups, the leading quarter at 4 bits)."""
    rk_rot = hadamard.rotate_latent_f32(zk, 8)
    rv_rot = hadamard.rotate_latent_f32(zv, value_rank // 4)
    kh = quant.quantize(rk_rot[..., :8], 4)
    kl = quant.quantize(rk_rot[..., 8:], 3)
    kcode = np.concatenate([kh[0], kl[0]], axis=-1)
    ks = np.concatenate([np.repeat(kh[1][..., None], 8, -1),
                         np.repeat(kl[1][..., None], 24, -1)], axis=-1)
    kz = np.concatenate([np.repeat(kh[2][..., None], 8, -1),
                         np.repeat(kl[2][..., None], 24, -1)], axis=-1)
    b, t = zv.shape[:2]
    groups = rv_rot.reshape(b, t, value_rank // 32, 32)
    n4 = value_rank // 4 // 32
    v4 = quant.quantize(groups[:, :, :n4], 4)
    v3 = quant.quantize(groups[:, :, n4:], 3)
    vcode = np.concatenate([v4[0], v3[0]], axis=2).reshape(b, t, value_rank)
    vs = np.repeat(np.concatenate([v4[1], v3[1]], axis=2), 32, axis=-1)
    vz = np.repeat(np.concatenate([v4[2], v3[2]], axis=2), 32, axis=-1)
    return rk_rot, rv_rot, (kcode, ks, kz), (vcode, vs, vz)


def _check_readout(key_latents, value_latents, seq_len=150, value_rank=256):
    cache, zk, zv = _rotated_q43_cache(seq_len, value_rank)
    rk_rot, rv_rot, kq, vq = _expected_groups(zk, zv, value_rank)
    for b in range(2):
        for got, rot, (code, s, z) in (
                (key_latents(cache, b, seq_len), rk_rot[b], tuple(a[b] for a in kq)),
                (value_latents(cache, b, seq_len), rv_rot[b], tuple(a[b] for a in vq))):
            sf = quant.f16(s).astype(np.float64)
            zf = quant.f16(z).astype(np.float64)
            assert got.shape == rot.shape
            # exactly the dequantized value of the entry's own group
            assert np.array_equal(got, zf + sf * code.astype(np.float64))
            # and within half a step of the rotated latent it stores
            bound = sf / 2 * (1 + 2.0 ** -18)
            assert np.all(np.abs(got - rot.astype(np.float64)) <= bound)


def test_q43_readout_pinned_elementwise():
    _check_readout(oc.Cache.key_latents, oc.Cache.value_latents)
    _check_readout(oc.Cache.key_latents, oc.Cache.value_latents, seq_len=64,
                   value_rank=512)


def _value_group_shifted(cache, b, seq_len):
    """Read-out with the scale / zero of the next group (off by one)."""
    x = oc.Cache.value_latents(cache, b, seq_len)
    g = cache.rv // 32
    _, _, vb, vm = cache._q_views()
    nt = (seq_len + 63) // 64
    codes = oc.unpack_value_tiles(vb[b, :nt], cache.rv).reshape(nt * 64, g, 32)[:seq_len]
    s = np.roll(np.transpose(vm[b, :nt, 0], (0, 2, 1)).reshape(nt * 64, g), 1, axis=1)[:seq_len]
    z = np.roll(np.transpose(vm[b, :nt, 1], (0, 2, 1)).reshape(nt * 64, g), 1, axis=1)[:seq_len]
    return quant.dequantize(codes, s, z).reshape(x.shape)


def _key_scale_zero_swapped(cache, b, seq_len):
    """Read-out taking the hi group's zero as its scale and vice versa."""
    kb, km, _, _ = cache._q_views()
    nt = (seq_len + 63) // 64
    codes = oc.unpack_key_tiles(kb[b, :, :nt].reshape(-1, 832)).reshape(
        cache.H, nt * 64, 32)[:, :seq_len]
    meta = km[b, :, :nt].reshape(cache.H, nt * 64, 4)[:, :seq_len]
    hi = quant.dequantize(codes[..., :8], meta[..., 1], meta[..., 0])
    lo = quant.dequantize(codes[..., 8:], meta[..., 2], meta[..., 3])
    return np.transpose(np.concatenate([hi, lo], axis=-1), (1, 0, 2))


def _token_shifted(cache, b, seq_len):
    """Read-out one token late."""
    x = oc.Cache.key_latents(cache, b, seq_len + 1)
    return x[1:]


@pytest.mark.parametrize("mutant", ["value_group", "key_meta", "token"])
def test_readout_pin_catches_planted_mistakes(mutant):
    k, v = oc.Cache.key_latents, oc.Cache.value_latents
    if mutant == "value_group":
        v = _value_group_shifted
    elif mutant == "key_meta":
        k = _key_scale_zero_swapped
    else:
        k = _token_shifted
    with pytest.raises(AssertionError):
        _check_readout(k, v)
