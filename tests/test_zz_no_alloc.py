"""starkv_decode_noalloc (the library's fixed scratch array as workspace)
against starkv_decode (caller workspace), through the C ABI on the GPU.

Both run the same kernels on the same inputs, so the outputs must agree bit
for bit; each is also checked against the fp64 oracle to the decode bound.
Two calls in a row on one device, the second with a smaller input, show that
the shared array carries nothing over from the previous call.
"""

import math

import numpy as np
import pytest

import synth
from oracle import cache as oc

from helpers import (TOL, append_both, config_for, dev, fill_random, oracle_decode,
                     rel_err, sk, storage_dtype)

pytestmark = pytest.mark.gpu


def _both(name, batch, seq_len, q_scale=4.0, seed=0):
    import torch
    w = synth.WORKLOADS[name].replace(batch=batch)
    T = ((seq_len + 63) // 64 + 1) * 64
    cfg = config_for(w, max_tokens=T)
    assert sk().starkv_workspace_bytes(cfg, sk().OP_DECODE, seq_len) <= \
        sk().starkv_noalloc_scratch_bytes()
    g = sk().LatentCache(cfg)
    o = oc.Cache.for_workload(w, max_tokens=T)
    fill_random(g, o, seed=seq_len + seed)
    print(f"noalloc {name} B={batch} T={seq_len}", flush=True)
    append_both(w, cfg, g, o, 0, seq_len, batch)
    bk, bv = synth.factors(w)
    q = synth.round_to_bf16(synth.queries(w) * q_scale)
    dt = storage_dtype(w)
    qd, bkd, bvd = dev(q, dt), dev(bk, dt), dev(bv, dt)
    scale = 1.0 / math.sqrt(w.head_dim)
    out_ws = torch.empty((batch, w.n_q_heads, w.head_dim), device="cuda")
    out_na = torch.full_like(out_ws, float("nan"))
    ws = sk().workspace(cfg, sk().OP_DECODE, seq_len)
    sk().starkv_decode(cfg, g, seq_len, qd, bkd, bvd, scale, out_ws, ws)
    sk().starkv_decode_noalloc(cfg, g, seq_len, qd, bkd, bvd, scale, out_na)
    torch.cuda.synchronize()
    a = out_ws.cpu().numpy().astype(np.float64)
    b = out_na.cpu().numpy().astype(np.float64)
    ref = oracle_decode(w, o, seq_len, q)
    print(f"  noalloc vs workspace max diff {np.abs(a - b).max():.3e}, "
          f"vs oracle {rel_err(b, ref):.3e}", flush=True)
    return a, b, ref


@pytest.mark.parametrize("first,second", [
    (("l2_q43", 4, 5000), ("l2_q43", 2, 700)),
    (("l3_gqa_q43", 8, 3000), ("l3_gqa_q43", 1, 130)),
    (("l2_bf16", 6, 4096), ("l2_bf16", 2, 1000)),
])
def test_noalloc_matches_workspace_decode_twice(first, second):
    for i, (name, batch, seq_len) in enumerate((first, second)):
        a, b, ref = _both(name, batch, seq_len, seed=i)
        assert np.array_equal(a, b)
        assert rel_err(b, ref) <= TOL
