"""Paged and ragged 4/3-bit caches (vLLM-style KV blocks), written from the
definition: a pool of pages, each one 64-token tile of every KV head (the
tile of the packed format in cache.py), and a page table mapping tile t of
sequence b to its page.  The contiguous cache is the pool with
page(b, t) = b * NT + t.  Every operation gathers a sequence's pages into a
one-sequence contiguous cache, applies the plain operation there, and (for
writes) scatters the pages back -- no other arithmetic.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).
"""

from __future__ import annotations

import numpy as np

from . import attention, cache as oc


def _tile_views(c):
    """The four buffers of a q43 cache viewed as [pages, bytes per page]."""
    n = c.B * c.nt
    return {k: c.buf[k].reshape(n, -1) for k in ("key", "key_meta", "value", "value_meta")}


def gather(pool, table, b, n_tiles):
    """One-sequence contiguous cache whose tile t is pool page table[b][t],
    t < n_tiles."""
    assert pool.kind == "q43"
    c = oc.Cache(1, pool.H, pool.rk, pool.rv, n_tiles * oc.TT, "q43", pool.rotate,
                 key_ranks=pool.kr, lo_bits=pool.lob)
    src, dst = _tile_views(pool), _tile_views(c)
    for t in range(n_tiles):
        for k in src:
            dst[k][t] = src[k][table[b][t]]
    return c


def scatter(pool, table, b, seq_cache):
    """Write the tiles of a one-sequence cache back to their pool pages."""
    src, dst = _tile_views(seq_cache), _tile_views(pool)
    for t in range(seq_cache.nt):
        for k in src:
            dst[k][table[b][t]] = src[k][t]


def append_paged(pool, table, positions, z_key, z_value):
    """One token per sequence b at positions[b]: z_key [B, Hkv, r_k],
    z_value [B, R_v] (technical review of arXiv 2606.08382, Algorithm 2,
    step 3, per sequence)."""
    for b, pos in enumerate(positions):
        n_tiles = pos // oc.TT + 1
        c = gather(pool, table, b, n_tiles)
        c.append(np.asarray(z_key[b], np.float32)[None, None],
                 np.asarray(z_value[b], np.float32)[None, None], int(pos), 1)
        scatter(pool, table, b, c)


def decode_paged(pool, table, seq_lens, q, bk, bv, sm_scale, n_q_heads, rotate,
                 batches=None, rope_theta=0.0):
    """Row b: plain decode of sequence b over its first seq_lens[b] tokens
    (its own query position seq_lens[b] - 1 with rotary keys).  A length of
    0 gives a zero row.  out [len(batches), Hq, d_h] float64."""
    q = np.asarray(q, np.float64)
    batches = range(len(seq_lens)) if batches is None else batches
    out = np.zeros((len(batches), n_q_heads, q.shape[-1]))
    for bi, b in enumerate(batches):
        n = int(seq_lens[b])
        if n == 0:
            continue
        c = gather(pool, table, b, (n + oc.TT - 1) // oc.TT)
        out[bi] = attention.decode(c, n, q[b:b + 1], bk, bv, sm_scale, n_q_heads,
                                   rotate, rope_theta=rope_theta)[0]
    return out


def prefill_paged(pool, table, ctx_len, z_key, z_value, q, bk, bv, sm_scale,
                  n_q_heads, rotate, rows=None, heads=None, rope_theta=0.0):
    """Chunked causal prefill of every sequence b of a paged pool: the
    chunk's latents z_key [B, C, Hkv, r_k], z_value [B, C, R_v] are appended
    at [ctx_len, ctx_len + C) of sequence b's pages (technical review of
    arXiv 2606.08382, Algorithm 2 step 3), then query i of q [B, C, Hq, d_h]
    (absolute position ctx_len + i) attends to positions 0 .. ctx_len + i of
    the stored cache.  Returns out [B, len(rows), len(heads), d_h] float64."""
    z_key = np.asarray(z_key, np.float32)
    z_value = np.asarray(z_value, np.float32)
    n = z_key.shape[1]
    n_tiles = (ctx_len + n + oc.TT - 1) // oc.TT
    outs = []
    for b in range(z_key.shape[0]):
        c = gather(pool, table, b, n_tiles)
        c.append(z_key[b:b + 1], z_value[b:b + 1], ctx_len, n)
        outs.append(attention.causal_attention(c, ctx_len, q[b], bk, bv, sm_scale,
                                               n_q_heads, rotate, rows, heads,
                                               rope_theta=rope_theta))
        scatter(pool, table, b, c)
    return np.stack(outs)
