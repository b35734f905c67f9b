"""starkv_decode_step (append + decode in one call, the 4/3-bit append and
query projection in one launch) against starkv_append followed by
starkv_decode on a copy of the same cache: the cache bytes and the output
must be identical bit for bit, and the output within the decode bound of the
fp64 oracle reading those bytes."""

import math

import numpy as np
import pytest

import synth
from oracle import cache as oc

from helpers import (TOL, append_both, config_for, dev, fill_random, gpu_bytes,
                     oracle_decode, rel_err, sk, storage_dtype)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,batch,ctx,n", [
    ("l2_q43", 3, 700, 1), ("l2_q43", 2, 125, 5), ("l3_gqa_q43", 4, 1000, 1),
    ("l2_q43", 2, 640, 0), ("l2_bf16", 2, 300, 2), ("tiny", 1, 255, 1),
    ("l2_q4", 2, 700, 1)])
def test_decode_step_equals_append_then_decode(name, batch, ctx, n):
    import torch
    w = synth.WORKLOADS[name].replace(batch=batch)
    T = ((ctx + n + 63) // 64 + 1) * 64
    cfg = config_for(w, max_tokens=T)
    ga, gb = sk().LatentCache(cfg), sk().LatentCache(cfg)
    o = oc.Cache.for_workload(w, max_tokens=T)
    fill_random(ga, o, seed=ctx + n)
    print(f"decode_step {name} B={batch} ctx={ctx} n={n}", flush=True)
    append_both(w, cfg, ga, o, 0, ctx, batch)
    for x, y in zip(ga.buffers, gb.buffers):
        y.copy_(x)
    zs = [synth.latents(w, b, ctx, n) for b in range(batch)]
    zk = np.stack([z[0] for z in zs]).astype(np.float32)
    zv = np.stack([z[1] for z in zs]).astype(np.float32)
    if n:
        o.append(zk, zv, ctx, n)
    bk, bv = synth.factors(w)
    q = synth.round_to_bf16(synth.queries(w) * 4.0)
    dt = storage_dtype(w)
    qd, bkd, bvd = dev(q, dt), dev(bk, dt), dev(bv, dt)
    scale = 1.0 / math.sqrt(w.head_dim)
    ws = sk().workspace(cfg, sk().OP_DECODE, ctx + n)
    out_a = torch.empty((batch, w.n_q_heads, w.head_dim), device="cuda")
    out_b = torch.full_like(out_a, float("nan"))
    zkd, zvd = dev(zk), dev(zv)
    if n:
        sk().starkv_append(cfg, ga, zkd, zvd, ctx, n)
    sk().starkv_decode(cfg, ga, ctx + n, qd, bkd, bvd, scale, out_a, ws)
    sk().starkv_decode_step(cfg, gb, zkd, zvd, ctx, qd, bkd, bvd, scale, out_b, ws, n=n)
    torch.cuda.synchronize()
    for x, y in zip(ga.buffers, gb.buffers):
        assert torch.equal(x, y)
    got = gpu_bytes(gb, o)
    for key in got:
        assert np.array_equal(got[key], o.buf[key]), key
    a = out_a.cpu().numpy().astype(np.float64)
    b = out_b.cpu().numpy().astype(np.float64)
    assert np.array_equal(a, b)
    err = rel_err(b, oracle_decode(w, o, ctx + n, q))
    print(f"  rel err {err:.3e}", flush=True)
    assert err <= TOL
