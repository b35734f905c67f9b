"""Shared plumbing for the GPU parity tests: build the same cache on the GPU
(through the C ABI) and in the oracle, from the same seeded inputs."""

from __future__ import annotations

import math

import numpy as np

import synth
from oracle import attention as oa
from oracle import cache as oc

TOL = 5e-3   # max|gpu - ref| / max|ref|, attention output


def sk():
    import decode_attention_starkv_amd as mod
    return mod


def qbits(w):
    """make_config keywords of the workload's precision split (quantized
    caches: the trailing block's width, 3 or 4 bits)."""
    return dict(lo_bits=w.lo_bits) if w.cache == "q43" else {}


def config_for(w, batch=None, max_tokens=None, num_splits=0, rotate=None, **kw):
    return sk().make_config(
        w.batch if batch is None else batch, w.n_q_heads, w.n_kv_heads,
        w.head_dim, w.key_rank, w.value_rank,
        w.max_tokens if max_tokens is None else max_tokens, w.cache,
        w.rotate if rotate is None else rotate, num_splits, **qbits(w), **kw)


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device="cuda", dtype=dtype or t.dtype)


def storage_dtype(w):
    import torch
    return torch.float32 if w.cache == "f32" else torch.bfloat16


def fill_random(gpu_cache, ocache, seed):
    """Give both caches the same random bytes (unused slots stay garbage)."""
    import torch
    rng = np.random.default_rng(seed)
    for i, key in enumerate(("key", "key_meta", "value", "value_meta")):
        n = ocache.buf[key].size
        if n == 0:
            continue
        data = rng.integers(0, 256, n, dtype=np.uint8)
        ocache.buf[key][:] = data
        gpu_cache.buffers[i][:n].copy_(torch.from_numpy(data))


def fill_byte(gpu_cache, ocache, value):
    for i, key in enumerate(("key", "key_meta", "value", "value_meta")):
        ocache.buf[key][:] = value
        gpu_cache.buffers[i].fill_(value)


def gpu_bytes(gpu_cache, ocache):
    out = {}
    for i, key in enumerate(("key", "key_meta", "value", "value_meta")):
        n = ocache.buf[key].size
        out[key] = gpu_cache.buffers[i][:n].cpu().numpy()
    return out


def append_both(w, cfg, gcache, ocache, pos, n, batch, chunk=4096, spike=None):
    """Append synthetic tokens [pos, pos+n) to both caches."""
    import torch
    for p0 in range(pos, pos + n, chunk):
        m = min(chunk, pos + n - p0)
        zs = [synth.latents(w, b, p0, m, spike=spike) for b in range(batch)]
        zk = np.stack([z[0] for z in zs])
        zv = np.stack([z[1] for z in zs])
        sk().starkv_append(cfg, gcache, dev(zk), dev(zv), p0, m)
        if ocache is not None:
            ocache.append(zk, zv, p0, m)
    torch.cuda.synchronize()


def gpu_decode(w, cfg, gcache, seq_len, q, batch):
    import torch
    bk, bv = synth.factors(w)
    dt = storage_dtype(w)
    out = torch.empty((batch, w.n_q_heads, w.head_dim), device="cuda",
                      dtype=torch.float32)
    ws = sk().workspace(cfg, sk().OP_DECODE, seq_len)
    sk().starkv_decode(cfg, gcache, seq_len, dev(q, dt), dev(bk, dt), dev(bv, dt),
                       1.0 / math.sqrt(w.head_dim), out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def oracle_decode(w, ocache, seq_len, q, batches=None):
    bk, bv = synth.factors(w)
    return oa.decode(ocache, seq_len, q, bk, bv, 1.0 / math.sqrt(w.head_dim),
                     w.n_q_heads, w.rotate, batches=batches)


def rel_err(got, ref):
    return float(np.abs(got - ref).max() / np.abs(ref).max())
