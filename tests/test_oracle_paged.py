"""Pins for the oracle's paged and ragged caches (CPU).

A paged pool with the identity table is the contiguous cache; a permuted
table moves whole tiles and nothing else; a ragged length decodes each
sequence exactly as a plain decode of that length does; appends land in the
page the table names.  (The model card's vLLM integration stores the cache
in KV blocks; the pages fix no block format, so these pins tie the paged
forms to the contiguous cache, which the other oracle pins already fix.)
"""

import math

import numpy as np

import synth
from oracle import attention as oa
from oracle import cache as oc
from oracle import paged


def _setup(seed=0, B=3, T=192, seq=150, rope=0.0):
    w = synth.WORKLOADS["l2_q43"].replace(batch=B, n_q_heads=4, n_kv_heads=4,
                                          value_rank=256, seed=seed)
    c = oc.Cache.for_workload(w, max_tokens=T)
    zk, zv = synth.batch_latents(w, 0, seq)
    c.append(zk, zv, 0, seq)
    bk, bv = synth.factors(w)
    q = synth.queries(w) * 4
    return w, c, bk, bv, q


def _permuted_pool(c, rng):
    nt = c.nt
    perm = rng.permutation(c.B * nt)
    table = perm.reshape(c.B, nt)
    pool = oc.Cache(c.B, c.H, c.rk, c.rv, c.T, "q43", c.rotate, fill=0xAB)
    for b in range(c.B):
        one = oc.Cache(1, c.H, c.rk, c.rv, c.T, "q43", c.rotate)
        for k in one.buf:
            n = one.buf[k].size
            one.buf[k][:] = c.buf[k][b * n:(b + 1) * n]
        paged.scatter(pool, table, b, one)
    return pool, table


def test_identity_table_is_the_contiguous_cache():
    w, c, bk, bv, q = _setup()
    table = np.arange(c.B * c.nt).reshape(c.B, c.nt)
    s = 1 / math.sqrt(w.head_dim)
    ref = oa.decode(c, 150, q, bk, bv, s, 4, True)
    got = paged.decode_paged(c, table, [150] * 3, q, bk, bv, s, 4, True)
    assert np.array_equal(got, ref)


def test_permuted_pages_move_whole_tiles_only():
    w, c, bk, bv, q = _setup(seed=1)
    pool, table = _permuted_pool(c, np.random.default_rng(2))
    s = 1 / math.sqrt(w.head_dim)
    assert np.array_equal(paged.decode_paged(pool, table, [150] * 3, q, bk, bv, s, 4, True),
                          oa.decode(c, 150, q, bk, bv, s, 4, True))
    for b in range(3):
        g = paged.gather(pool, table, b, c.nt)
        for k in g.buf:
            n = g.buf[k].size
            assert np.array_equal(g.buf[k], c.buf[k][b * n:(b + 1) * n])


def test_ragged_rows_are_plain_decodes_of_their_lengths():
    w, c, bk, bv, q = _setup(seed=3)
    pool, table = _permuted_pool(c, np.random.default_rng(4))
    s = 1 / math.sqrt(w.head_dim)
    lens = [150, 1, 77]
    got = paged.decode_paged(pool, table, lens, q, bk, bv, s, 4, True, rope_theta=1e4)
    for b, n in enumerate(lens):
        ref = oa.decode(c, n, q, bk, bv, s, 4, True, batches=[b], rope_theta=1e4)
        assert np.array_equal(got[b], ref[0])
    assert not np.allclose(got[0], got[2])
    zero = paged.decode_paged(pool, table, [0, 5, 5], q, bk, bv, s, 4, True)
    assert np.array_equal(zero[0], np.zeros_like(zero[0]))


def test_paged_append_lands_in_the_named_page():
    w, c, bk, bv, q = _setup(seed=5)
    pool, table = _permuted_pool(c, np.random.default_rng(6))
    rng = np.random.default_rng(7)
    zk = rng.standard_normal((3, 4, 32)).astype(np.float32)
    zv = rng.standard_normal((3, 256)).astype(np.float32)
    pos = [150, 63, 64]
    paged.append_paged(pool, table, pos, zk, zv)
    for b in range(3):
        one = oc.Cache(1, c.H, c.rk, c.rv, c.T, "q43", c.rotate)
        for k in one.buf:
            n = one.buf[k].size
            one.buf[k][:] = c.buf[k][b * n:(b + 1) * n]
        one.append(zk[b][None, None], zv[b][None, None], pos[b], 1)
        g = paged.gather(pool, table, b, c.nt)
        for k in g.buf:
            assert np.array_equal(g.buf[k], one.buf[k]), (b, k)


def test_paged_prefill_is_plain_prefill_per_sequence():
    """Chunked prefill over a permuted pool: each sequence's output and bytes
    equal the plain prefill of that sequence's contiguous cache (the chunk
    crosses a tile boundary; the identity table gives the contiguous cache's
    own result)."""
    w, c, bk, bv, q = _setup(seed=8, seq=100)
    pool, table = _permuted_pool(c, np.random.default_rng(9))
    rng = np.random.default_rng(10)
    C = 50
    zk = rng.standard_normal((3, C, 4, 32)).astype(np.float32)
    zv = (rng.standard_normal((3, C, 256)) * 0.3).astype(np.float32)
    qc = rng.standard_normal((3, C, 4, w.head_dim)) * 4 / math.sqrt(w.head_dim)
    s = 1 / math.sqrt(w.head_dim)
    got = paged.prefill_paged(pool, table, 100, zk, zv, qc, bk, bv, s, 4, True)
    for b in range(3):
        one = oc.Cache(1, c.H, c.rk, c.rv, c.T, "q43", c.rotate)
        for k in one.buf:
            n = one.buf[k].size
            one.buf[k][:] = c.buf[k][b * n:(b + 1) * n]
        one.append(zk[b:b + 1], zv[b:b + 1], 100, C)
        ref = oa.causal_attention(one, 100, qc[b], bk, bv, s, 4, True)
        assert np.array_equal(got[b], ref)
        g = paged.gather(pool, table, b, c.nt)
        for k in g.buf:
            assert np.array_equal(g.buf[k], one.buf[k]), (b, k)
    # identity table: the contiguous cache prefilled in place
    c2 = oc.Cache(3, c.H, c.rk, c.rv, c.T, "q43", c.rotate)
    for k in c.buf:
        c2.buf[k][:] = c.buf[k]
    ident = np.arange(3 * c.nt).reshape(3, c.nt)
    got2 = paged.prefill_paged(c2, ident, 100, zk, zv, qc, bk, bv, s, 4, True)
    assert np.array_equal(got2, got)
