"""GPU decode vs the oracle when the latents or the query are far from unit
scale.

The decode path narrows three intermediates to fp16: the query record q~,
the value-contraction operand P * field weight * group scale (4/3-bit
cache), and the partial rows of each split (divided by their own l).  These
cases move the value latents by 1e-3 .. 1e2 (4/3-bit) and 1e-3 .. 1e5
(bf16), the key latents by 1e-2 .. 1e2, and sharpen the query by 32, and
require the same bound as every decode case: max|gpu - ref| / max|ref| <=
5e-3, the oracle (fp64) reading the same cache bytes.
"""

import math

import numpy as np
import pytest

import synth
from oracle import cache as oc

from helpers import TOL, config_for, dev, fill_random, gpu_decode, oracle_decode, rel_err, sk

pytestmark = pytest.mark.gpu


def run_scaled(name, seq_len, kscale=1.0, vscale=1.0, qscale=1.0, batch=2, **kw):
    import torch
    w = synth.WORKLOADS[name].replace(batch=batch, **kw)
    T = ((seq_len + 63) // 64 + 1) * 64
    cfg = config_for(w, max_tokens=T)
    g = sk().LatentCache(cfg)
    o = oc.Cache.for_workload(w, max_tokens=T)
    fill_random(g, o, seed=seq_len + 3)
    print(f"decode {name} T={seq_len} keys*{kscale} values*{vscale} q*{qscale} {kw}",
          flush=True)
    zs = [synth.latents(w, b, 0, seq_len) for b in range(batch)]
    zk = (np.stack([z[0] for z in zs]) * np.float32(kscale)).astype(np.float32)
    zv = (np.stack([z[1] for z in zs]) * np.float32(vscale)).astype(np.float32)
    sk().starkv_append(cfg, g, dev(zk), dev(zv), 0, seq_len)
    o.append(zk, zv, 0, seq_len)
    torch.cuda.synchronize()
    q = synth.round_to_bf16(synth.queries(w) * qscale)
    got = gpu_decode(w, cfg, g, seq_len, q, batch)
    ref = oracle_decode(w, o, seq_len, q)
    assert np.isfinite(got).all()
    err = rel_err(got, ref)
    print(f"  rel err {err:.3e}", flush=True)
    return err


@pytest.mark.parametrize("kscale,vscale,qscale", [
    (1.0, 1e-3, 1.0), (1.0, 1e2, 1.0), (1e2, 1.0, 1.0), (1e-2, 1.0, 32.0),
    (1.0, 1.0, 32.0)])
def test_q43_magnitudes(kscale, vscale, qscale):
    assert run_scaled("l2_q43", 1000, kscale, vscale, qscale) <= TOL


@pytest.mark.parametrize("kscale,vscale,qscale", [
    (1.0, 1e-3, 1.0), (1.0, 1e5, 1.0), (1e3, 1.0, 1.0), (1.0, 1.0, 32.0)])
def test_bf16_magnitudes(kscale, vscale, qscale):
    assert run_scaled("l2_bf16", 1000, kscale, vscale, qscale) <= TOL


def test_gqa_q43_sharp_query():
    assert run_scaled("l3_gqa_q43", 700, qscale=32.0, vscale=1e-2) <= TOL
