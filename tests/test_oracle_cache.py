"""Pins for the oracle's packed cache format and size formulas (CPU only).

The format itself is our own (the pages fix none); it is pinned by
hand-derived byte positions (tests/golden/format_examples.json), single-bit
exhaustive placement, bijectivity, and the sizes the pages' formulas give
(technical review of arXiv 2606.08382, eq. 1, eq. 14, eq. 15, eq. 16).
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import cache as oc
from oracle import sizes

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _key_codes(rng, n):
    c = rng.integers(0, 8, (n, 64, 32)).astype(np.uint8)
    c[:, :, :8] = rng.integers(0, 16, (n, 64, 8))
    return c


def _value_codes(rng, n, rv):
    c = rng.integers(0, 8, (n, 64, rv)).astype(np.uint8)
    c[:, :, :rv // 4] = rng.integers(0, 16, (n, 64, rv // 4))
    return c


def test_golden_byte_positions():
    ex = json.load(open(os.path.join(GOLD, "format_examples.json")))["examples"]
    for e in ex:
        if e["kind"] == "value":
            rv = e["value_rank"]
            codes = np.zeros((1, 64, rv), np.uint8)
            codes[0, e["token"], e["channel"]] = e["code"]
            blob = oc.pack_value_tiles(codes)[0]
            back = oc.unpack_value_tiles(blob[None], rv)
        else:
            codes = np.zeros((1, 64, 32), np.uint8)
            codes[0, e["token"], e["channel"]] = e["code"]
            blob = oc.pack_key_tiles(codes)[0]
            back = oc.unpack_key_tiles(blob[None])
        want = np.zeros_like(blob)
        for k, v in e["bytes"].items():
            want[int(k)] = v
        assert np.array_equal(blob, want), (e, np.nonzero(blob))
        assert np.array_equal(back, codes)


def test_pack_unpack_are_inverse():
    rng = np.random.default_rng(0)
    k = _key_codes(rng, 7)
    assert np.array_equal(oc.unpack_key_tiles(oc.pack_key_tiles(k)), k)
    for rv in (128, 256, 1024):
        v = _value_codes(rng, 3, rv)
        assert np.array_equal(oc.unpack_value_tiles(oc.pack_value_tiles(v), rv), v)
    # and bytes -> codes -> bytes is identity on random bytes (dense format)
    kb = rng.integers(0, 256, (4, 832)).astype(np.uint8)
    assert np.array_equal(oc.pack_key_tiles(oc.unpack_key_tiles(kb)), kb)
    vb = rng.integers(0, 256, (2, 26 * 256)).astype(np.uint8)
    assert np.array_equal(oc.pack_value_tiles(oc.unpack_value_tiles(vb, 256)), vb)


def test_every_bit_has_exactly_one_owner():
    """Setting one code bit sets exactly one stored bit, and all stored bits
    are covered (the format is dense: no padding bits)."""
    seen = np.zeros(832 * 8, np.int32)
    for t in range(64):
        for ch in range(32):
            for k in range(4 if ch < 8 else 3):
                c = np.zeros((1, 64, 32), np.uint8)
                c[0, t, ch] = 1 << k
                bits = np.unpackbits(oc.pack_key_tiles(c)[0])
                assert bits.sum() == 1
                seen += bits
    assert np.all(seen == 1)
    rv = 128
    seen = np.zeros(26 * rv * 8, np.int32)
    for t in range(64):
        for ch in range(0, rv, 5):
            for k in range(4 if ch < rv // 4 else 3):
                c = np.zeros((1, 64, rv), np.uint8)
                c[0, t, ch] = 1 << k
                bits = np.unpackbits(oc.pack_value_tiles(c)[0])
                assert bits.sum() == 1
                seen += bits
    assert seen.max() == 1


# the buffers start as random bytes, read out as (meaningless, often NaN)
# latents on purpose
@pytest.mark.filterwarnings("ignore:invalid value encountered in cast")
@pytest.mark.parametrize("kind", ["f32", "bf16", "q43"])
def test_append_touches_only_its_tokens(kind):
    w = synth.WORKLOADS["l2_q43"].replace(batch=2, n_q_heads=4, n_kv_heads=4,
                                          value_rank=256, cache=kind,
                                          rotate=(kind == "q43"), seq_len=200)
    rng = np.random.default_rng(1)
    c = oc.Cache.for_workload(w, fill=0)
    for key in c.buf:
        c.buf[key][:] = rng.integers(0, 256, c.buf[key].size)
    before_k = c.key_latents(0, 192).copy() if kind != "q43" else None
    zk, zv = synth.batch_latents(w, 70, 45)
    c2 = oc.Cache.for_workload(w)
    for key in c.buf:
        c2.buf[key][:] = c.buf[key]
    c2.append(zk, zv, 70, 45)
    if kind == "q43":
        for b in range(2):
            kb0 = oc.unpack_key_tiles(c._q_views()[0][b].reshape(-1, 832))
            kb1 = oc.unpack_key_tiles(c2._q_views()[0][b].reshape(-1, 832))
            kb0 = kb0.reshape(4, -1, 32)
            kb1 = kb1.reshape(4, -1, 32)
            keep = np.ones(kb0.shape[1], bool)
            keep[70:115] = False
            assert np.array_equal(kb0[:, keep], kb1[:, keep])
            v0 = oc.unpack_value_tiles(c._q_views()[2][b], 256).reshape(-1, 256)
            v1 = oc.unpack_value_tiles(c2._q_views()[2][b], 256).reshape(-1, 256)
            assert np.array_equal(v0[keep], v1[keep])
            m0 = c._q_views()[3][b]
            m1 = c2._q_views()[3][b]
            mk = np.ones(m0.shape[0] * 64, bool)
            mk[70:115] = False
            a0 = np.transpose(m0, (0, 3, 1, 2)).reshape(-1, 2, 8)
            a1 = np.transpose(m1, (0, 3, 1, 2)).reshape(-1, 2, 8)
            assert np.array_equal(a0[mk], a1[mk])
    else:
        after = c2.key_latents(0, 192)
        keep = np.ones(192, bool)
        keep[70:115] = False
        assert np.array_equal(before_k[keep], after[keep], equal_nan=True)
        assert np.array_equal(c.value_latents(1, 192)[keep],
                              c2.value_latents(1, 192)[keep], equal_nan=True)
    # appended tokens read back as stored values (fp32 exact / bf16 rounded)
    got = c2.key_latents(1, 115)[70:115]
    if kind == "f32":
        assert np.array_equal(got, zk[1].astype(np.float64))
    elif kind == "bf16":
        assert np.allclose(got, zk[1], rtol=2 ** -8, atol=0)


def test_cache_sizes_match_eq15_and_eq1():
    """Metric workload: 16 x 32768 tokens, 32 KV heads x r_k 32 + R_v 1024."""
    w = synth.WORKLOADS["l2_q43"]
    lay = oc.layout(w.batch, w.n_kv_heads, w.key_rank, w.value_rank,
                    w.seq_len, w.cache)
    payload = lay["key"] + lay["value"]
    meta = lay["key_meta"] + lay["value_meta"]
    bbar = sizes.mean_bits(Fraction(1, 4), 4, 3)            # 25:75 split
    assert bbar == Fraction(13, 4)
    eq15 = sizes.latent_payload_bytes(w.batch, w.seq_len, bbar,
                                      [[w.key_rank] * w.n_kv_heads],
                                      [w.value_rank])
    assert payload == eq15 == 436207616                    # no padding term
    assert meta == sizes.metadata_bytes(w.batch, w.seq_len, 2 * w.n_kv_heads,
                                        w.value_rank // 32) == 201326592
    assert payload + meta == 16 * 32768 * 1216
    dense = sizes.dense_kv_bytes(w.batch, w.seq_len, 1, w.n_kv_heads,
                                 w.head_dim, 16)
    assert dense == 8589934592
    # eq. 14 at the 25 % retained fraction with the 25:75 bit split
    assert dense / payload == sizes.payload_compression(Fraction(1, 4), bbar)
    assert float(dense / payload) == pytest.approx(19.6923, abs=1e-4)
    # GQA workload: eq. 1 counts KV heads, not query heads
    g = synth.WORKLOADS["l3_gqa_q43"]
    lg = oc.layout(g.batch, g.n_kv_heads, g.key_rank, g.value_rank, g.seq_len,
                   g.cache)
    assert sum(lg.values()) == g.batch * g.seq_len * 304


def test_page_printed_numbers():
    pn = json.load(open(os.path.join(GOLD, "page_numbers.json")))
    e = pn["eq14_mean_bits"]
    assert sizes.mean_bits(Fraction(e["frac_hi"]), e["bits_hi"], e["bits_lo"]) \
        == Fraction(e["value"])
    for key in ("eq14_compression_rho_025", "eq14_compression_rho_04"):
        e = pn[key]
        assert sizes.payload_compression(Fraction(e["rho"]), Fraction(e["bbar"])) \
            == Fraction(e["value"])
    e = pn["eq16_compressed_fraction"]
    assert Fraction(1, 4) * Fraction(16, 5) / 16 == Fraction(e["value"])
    e = pn["eq16_protected_fraction"]
    f = sizes.protected_fraction(e["layers"], e["protected"], Fraction(e["compressed"]))
    assert f == Fraction(e["value"])
    assert round(float(1 / f), 2) == e["inverse_approx"]
    # eq. 1 worked by hand: B=1, T=1, L=1, h_kv=1, d_h=1, 16 bits -> K and V
    assert sizes.dense_kv_bytes(1, 1, 1, 1, 1, 16) == 4


def test_plain_layout_byte_positions():
    """bf16 cache, B=2, Hkv=3, r_k=16, R_v=64, T_max=192 (3 tiles): one key
    and one value element placed by hand.
    key (b=1, h=2, t=70, c=13): tile 1, token 6, chunk 1, channel-in-chunk 5
      element ((((1*3 + 2)*3 + 1)*2 + 1)*64 + 6)*8 + 5 = 16949 -> byte 33898
    value (b=1, t=70, ch=45): tile 1, group 1, channel-in-group 13, block 0,
      token-in-block 6
      element ((((1*3 + 1)*2 + 1)*8 + 0)*32 + 13)*8 + 6 = 18542 -> byte 37084
    1.5 is bf16 0x3FC0 (little-endian bytes C0 3F); -2.25 is 0xC010."""
    c = oc.Cache(2, 3, 16, 64, 192, "bf16")
    zk = np.zeros((2, 1, 3, 16), np.float32)
    zv = np.zeros((2, 1, 64), np.float32)
    zk[1, 0, 2, 13] = 1.5
    zv[1, 0, 45] = -2.25
    c.append(zk, zv, 70, 1)
    kb, vb = c.buf["key"], c.buf["value"]
    assert list(kb[33898:33900]) == [0xC0, 0x3F]
    assert list(vb[37084:37086]) == [0x10, 0xC0]
    assert np.count_nonzero(kb) == 2 and np.count_nonzero(vb) == 2
    # the same positions in an fp32 cache hold 4-byte elements
    c = oc.Cache(2, 3, 16, 64, 192, "f32")
    c.append(zk, zv, 70, 1)
    assert c.buf["key"][16949 * 4:16949 * 4 + 4].view(np.float32)[0] == 1.5
    assert c.buf["value"][18542 * 4:18542 * 4 + 4].view(np.float32)[0] == -2.25
