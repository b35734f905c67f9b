"""Plain float64 attention over the dequantized, reconstructed cache.

Definitions followed (technical review of arXiv 2606.08382):
* eq. 2 (section 2.2), row-vector convention: the reconstructed keys of KV
  head g are K_g = Z_k,g B_key[g]^T and the reconstructed values are
  V = Z_v B_value^T, V_g being its g-th block of head_dim columns
  (section 5.3, eq. 12 left-hand side: p_h (Z_V U_h^T));
* eq. 13 (section 6.1): with rotated stored latents Z H the factors become
  U H, so reconstruction uses B H;
* section 2.3: a = q K^T / sqrt(d_h) (the scale is an argument here),
  p = softmax(a), o = p V; query head h reads KV head g(h) = h // (Hq/Hkv).
Nothing is reassociated, fused or computed online: keys and values are
reconstructed, then a two-pass (max-subtracted) softmax is applied.

The split-T merge follows the attention decomposition theorem stated on the
CaliDrop review page ("What carries the argument"): attention over a union of
disjoint token subsets is the combination of the per-subset attentions
weighted by each subset's share of the total sum of exponentiated scores.
"""

from __future__ import annotations

import numpy as np

from . import hadamard


def effective_factors(bk, bv, rotate, key_rank, value_rank):
    """Factors that reconstruct from the stored latents: B (no rotation) or
    B H (rotated cache, eq. 13), float64."""
    bk = np.asarray(bk, np.float64)
    bv = np.asarray(bv, np.float64)
    if not rotate:
        return bk, bv
    rk = hadamard.rotation_matrix(key_rank // 4, key_rank - key_rank // 4)
    rv = hadamard.rotation_matrix(value_rank // 4, value_rank - value_rank // 4)
    return bk @ rk, bv @ rv


def softmax(a):
    a = np.asarray(a, np.float64)
    m = np.max(a, axis=-1, keepdims=True)
    e = np.exp(a - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def reconstruct(cache, b, seq_len, bk_eff, bv_eff, g, head_dim):
    """K_g [T, d_h] and V_g [T, d_h] of KV head g, batch element b."""
    zk = cache.key_latents(b, seq_len)[:, g, :]
    zv = cache.value_latents(b, seq_len)
    k = zk @ bk_eff[g].T
    v = zv @ bv_eff[g * head_dim:(g + 1) * head_dim].T
    return k, v


def decode(cache, seq_len, q, bk, bv, sm_scale, n_q_heads, rotate,
           batches=None, heads=None):
    """out [len(batches), len(heads), d_h] float64: each query head attends
    to the first seq_len cached tokens of its batch element."""
    q = np.asarray(q, np.float64)
    n_kv = cache.H
    group = n_q_heads // n_kv
    d_h = q.shape[-1]
    bk_e, bv_e = effective_factors(bk, bv, rotate, cache.rk, cache.rv)
    batches = range(q.shape[0]) if batches is None else batches
    heads = range(n_q_heads) if heads is None else heads
    out = np.zeros((len(batches), len(heads), d_h))
    for bi, b in enumerate(batches):
        zk = cache.key_latents(b, seq_len)
        zv = cache.value_latents(b, seq_len)
        for hi, h in enumerate(heads):
            g = h // group
            k = zk[:, g, :] @ bk_e[g].T
            v = zv @ bv_e[g * d_h:(g + 1) * d_h].T
            p = softmax(sm_scale * (k @ q[b, h]))
            out[bi, hi] = p @ v
    return out


def decode_partial(cache, b, h, t0, t1, q, bk_e, bv_e, sm_scale, n_q_heads):
    """(m, l, o) of one query head over tokens [t0, t1): m = max score,
    l = sum exp(a - m), o = sum exp(a - m) v / l.  Empty ranges give
    (-inf, 0, 0)."""
    d_h = q.shape[-1]
    if t1 <= t0:
        return -np.inf, 0.0, np.zeros(d_h)
    g = h // (n_q_heads // cache.H)
    zk = cache.key_latents(b, t1)[t0:t1, g, :]
    zv = cache.value_latents(b, t1)[t0:t1]
    a = sm_scale * ((zk @ bk_e[g].T) @ np.asarray(q[b, h], np.float64))
    v = zv @ bv_e[g * d_h:(g + 1) * d_h].T
    m = np.max(a)
    e = np.exp(a - m)
    return m, float(e.sum()), (e @ v) / e.sum()


def merge_partials(parts):
    """Combine [(m, l, o)] of disjoint token subsets into full attention."""
    m = max(p[0] for p in parts)
    w = [0.0 if p[1] == 0 else np.exp(p[0] - m) * p[1] for p in parts]
    tot = sum(w)
    return sum(wi * p[2] for wi, p in zip(w, parts)) / tot


def project_latents(x, a_key, a_value, n_kv_heads, key_rank):
    """Z = X A (review Algorithm 2 step 1), float64 then float32."""
    x = np.asarray(x, np.float64)
    zk = (x @ np.asarray(a_key, np.float64)).astype(np.float32)
    zv = (x @ np.asarray(a_value, np.float64)).astype(np.float32)
    return zk.reshape(x.shape[0], n_kv_heads, key_rank), zv


def prefill(cache, ctx_len, x, a_key, a_value, q, bk, bv, sm_scale,
            n_q_heads, rotate, rows=None, heads=None):
    """Chunked causal prefill of a one-sequence cache.

    Projects the chunk X [C, D] into latents, appends them at [ctx_len,
    ctx_len + C) (rotation + quantization as in Cache.append), then query i
    (absolute position ctx_len + i) attends to positions 0 .. ctx_len + i of
    the stored cache.  Returns out [len(rows), len(heads), d_h] float64.
    """
    assert cache.B == 1
    c = x.shape[0]
    zk, zv = project_latents(x, a_key, a_value, cache.H, cache.rk)
    cache.append(zk[None], zv[None], ctx_len, c)
    return causal_attention(cache, ctx_len, q, bk, bv, sm_scale, n_q_heads,
                            rotate, rows, heads)


def causal_attention(cache, ctx_len, q, bk, bv, sm_scale, n_q_heads, rotate,
                     rows=None, heads=None, batch=0):
    """Causal attention of a chunk's queries q [C, Hq, d_h] (query i at
    absolute position ctx_len + i) over positions 0 .. ctx_len + i of the
    stored cache of one batch element.  out [len(rows), len(heads), d_h]."""
    c = q.shape[0]
    total = ctx_len + c
    q = np.asarray(q, np.float64)
    d_h = q.shape[-1]
    group = n_q_heads // cache.H
    bk_e, bv_e = effective_factors(bk, bv, rotate, cache.rk, cache.rv)
    rows = np.arange(c) if rows is None else np.asarray(rows)
    heads = range(n_q_heads) if heads is None else heads
    zkl = cache.key_latents(batch, total)
    zvl = cache.value_latents(batch, total)
    out = np.zeros((len(rows), len(heads), d_h))
    pos = np.arange(total)
    for hi, h in enumerate(heads):
        g = h // group
        k = zkl[:, g, :] @ bk_e[g].T
        v = zvl @ bv_e[g * d_h:(g + 1) * d_h].T
        a = sm_scale * (q[rows, h] @ k.T)                   # [rows, total]
        a = np.where(pos[None, :] <= (ctx_len + rows)[:, None], a, -np.inf)
        out[:, hi] = softmax(a) @ v
    return out
