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


def effective_factors(bk, bv, rotate, key_rank, value_rank, key_ranks=None):
    """Factors that reconstruct from the stored latents: B (no rotation) or
    B H (rotated cache, eq. 13), float64.  key_ranks: KV head g's key factor
    has key_ranks[g] columns (review section 4, learned per-head ranks); the
    columns past it do not exist and are taken as zero, so whatever a cache
    holds in those channels (a 4/3-bit tile's padding) never reaches a
    score."""
    bk = np.array(bk, np.float64)
    bv = np.asarray(bv, np.float64)
    if key_ranks is not None:
        for g, r in enumerate(key_ranks):
            bk[g, :, r:] = 0.0
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


def rope(x, pos, theta):
    """Rotary position embedding of the rows x [..., d_h] at positions pos
    [...] (review section 5.3: keys stay pre-RoPE latents and are rotated
    after reconstruction; Algorithm 2, step 4c).  The pages fix no variant;
    the one taken is the half-split pairing of LLaMA-family checkpoints:
    channel i < d_h/2 pairs with i + d_h/2, and the pair turns by the angle
    pos * theta^(-2i/d_h):
        (x_i, x_{i+d/2}) -> (x_i cos a - x_{i+d/2} sin a,
                             x_i sin a + x_{i+d/2} cos a).   float64."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half = d // 2
    inv = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(pos, np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def decode(cache, seq_len, q, bk, bv, sm_scale, n_q_heads, rotate,
           batches=None, heads=None, rope_theta=0.0, q_pos=None):
    """out [len(batches), len(heads), d_h] float64: each query head attends
    to the first seq_len cached tokens of its batch element.

    rope_theta > 0: the query (at position q_pos, by default seq_len - 1, the
    token just appended) and every reconstructed key (at its own position
    0 .. seq_len - 1) are rotated by `rope` before the scores; values are
    not rotated."""
    q = np.asarray(q, np.float64)
    n_kv = cache.H
    group = n_q_heads // n_kv
    d_h = q.shape[-1]
    bk_e, bv_e = effective_factors(bk, bv, rotate, cache.rk, cache.rv, cache.kr)
    batches = range(q.shape[0]) if batches is None else batches
    heads = range(n_q_heads) if heads is None else heads
    out = np.zeros((len(batches), len(heads), d_h))
    t = seq_len - 1 if q_pos is None else q_pos
    for bi, b in enumerate(batches):
        zk = cache.key_latents(b, seq_len)
        zv = cache.value_latents(b, seq_len)
        for hi, h in enumerate(heads):
            g = h // group
            k = zk[:, g, :] @ bk_e[g].T
            v = zv @ bv_e[g * d_h:(g + 1) * d_h].T
            qh = q[b, h]
            if rope_theta:
                k = rope(k, np.arange(seq_len), rope_theta)
                qh = rope(qh, t, rope_theta)
            p = softmax(sm_scale * (k @ qh))
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
            n_q_heads, rotate, rows=None, heads=None, rope_theta=0.0):
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
                            rotate, rows, heads, rope_theta=rope_theta)


def causal_attention(cache, ctx_len, q, bk, bv, sm_scale, n_q_heads, rotate,
                     rows=None, heads=None, batch=0, rope_theta=0.0):
    """Causal attention of a chunk's queries q [C, Hq, d_h] (query i at
    absolute position ctx_len + i) over positions 0 .. ctx_len + i of the
    stored cache of one batch element.  out [len(rows), len(heads), d_h].

    rope_theta > 0: as in `decode`, every reconstructed key is rotated by
    `rope` at its own position and query i at position ctx_len + i."""
    c = q.shape[0]
    total = ctx_len + c
    q = np.asarray(q, np.float64)
    d_h = q.shape[-1]
    group = n_q_heads // cache.H
    bk_e, bv_e = effective_factors(bk, bv, rotate, cache.rk, cache.rv, cache.kr)
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
        qh = q[rows, h]
        if rope_theta:
            k = rope(k, pos, rope_theta)
            qh = rope(qh, ctx_len + rows, rope_theta)
        a = sm_scale * (qh @ k.T)                           # [rows, total]
        a = np.where(pos[None, :] <= (ctx_len + rows)[:, None], a, -np.inf)
        out[:, hi] = softmax(a) @ v
    return out


def fuse_value_output(bv, w_o, n_q_heads, n_kv_heads, head_dim):
    """Per-query-head fused value/output factor F_h = B_value[g(h)]^T O_h
    (review section 5.3, eq. 12: the right-hand factor U_h^T O_h prepared
    offline; Algorithm 2, step 7).  bv [Hkv*d_h, R_v]; w_o [Hq*d_h, D] with
    O_h its rows h*d_h .. (h+1)*d_h - 1 (row-vector convention: y = o W_o).
    Returns F [Hq, R_v, D] float64."""
    bv = np.asarray(bv, np.float64)
    w_o = np.asarray(w_o, np.float64)
    group = n_q_heads // n_kv_heads
    out = []
    for h in range(n_q_heads):
        g = h // group
        bvg = bv[g * head_dim:(g + 1) * head_dim]           # [d_h, R_v]
        out.append(bvg.T @ w_o[h * head_dim:(h + 1) * head_dim])
    return np.stack(out)


def decode_hidden(cache, seq_len, q, bk, bv, w_o, sm_scale, n_q_heads, rotate,
                  batches=None):
    """Decode that ends in the hidden size (review Algorithm 2, steps 7-8):
    y[b] = sum_h o_h O_h, o_h the per-head attention output of `decode` and
    O_h the rows h*d_h .. (h+1)*d_h - 1 of w_o [Hq*d_h, D].  float64."""
    o = decode(cache, seq_len, q, bk, bv, sm_scale, n_q_heads, rotate, batches)
    w_o = np.asarray(w_o, np.float64)
    d_h = o.shape[-1]
    return sum(o[:, h] @ w_o[h * d_h:(h + 1) * d_h] for h in range(n_q_heads))


def decode_latent_rows(cache, seq_len, q, bk, sm_scale, n_q_heads, rotate,
                       batches=None, unrotated=False):
    """The per-head attention rows in the (stored) value latent,
    obar_h = softmax(a_h) Z_v [len(batches), Hq, R_v] float64 -- the left-hand
    factor p_h Z_V of eq. 12, before any value factor is applied.  With a
    rotated cache Z_v is the stored rotated latent (Z H); a fused factor for
    it is F_h with its R_v rows rotated the same way.  `unrotated` returns
    obar_h H instead (the rows in the unrotated latent: H H = I, eq. 13)."""
    q = np.asarray(q, np.float64)
    n_kv = cache.H
    group = n_q_heads // n_kv
    bk_e, _ = effective_factors(bk, np.zeros((1, cache.rv)), rotate, cache.rk,
                                cache.rv, cache.kr)
    batches = range(q.shape[0]) if batches is None else batches
    out = np.zeros((len(batches), n_q_heads, cache.rv))
    for bi, b in enumerate(batches):
        zk = cache.key_latents(b, seq_len)
        zv = cache.value_latents(b, seq_len)
        for h in range(n_q_heads):
            g = h // group
            p = softmax(sm_scale * ((zk[:, g, :] @ bk_e[g].T) @ q[b, h]))
            out[bi, h] = p @ zv
    if unrotated and rotate:
        rv = hadamard.rotation_matrix(cache.rv // 4, cache.rv - cache.rv // 4)
        out = out @ rv
    return out
