"""GPU decode over a uniform 4-bit cache (both precision blocks at 4 bits:
keys as four nibble planes, every value group in the 4-bit run layout)
against the fp64 oracle on the same seeded inputs.

Bar: max|gpu - ref| / max|ref| <= 5e-3.  The shapes cover every family of
the split kernel's instantiations: group sizes 1 / 2 / 4 / 8, one, two and
eight KV heads per score wave, value ranks 256 / 512 / 768 / 1024 (two to
eight value groups per value wave, the last with its three-slot ring), a
ragged tail, a single token, forced splits, a sharpened softmax with
outlier tokens, and 0xFF (NaN) bytes in unused slots.  The append side is
covered bit for bit by test_gpu_append.
"""

import numpy as np
import pytest

import synth
from oracle import cache as oc

from helpers import (TOL, append_both, config_for, fill_byte, fill_random, gpu_decode,
                     oracle_decode, rel_err, sk)

pytestmark = pytest.mark.gpu


def run_u4(seq_len, batch=2, q_scale=1.0, spike=None, num_splits=0, fill="random",
           **kw):
    w = synth.WORKLOADS["l2_q4"].replace(batch=batch, **kw)
    assert w.lo_bits == 4
    T = ((seq_len + 63) // 64 + 1) * 64
    cfg = config_for(w, max_tokens=T, num_splits=num_splits)
    g = sk().LatentCache(cfg)
    o = oc.Cache.for_workload(w, max_tokens=T)
    assert o.lob == 4
    if fill == "random":
        fill_random(g, o, seed=seq_len + 5)
    else:
        fill_byte(g, o, fill)
    print(f"u4 decode B={batch} T={seq_len} qx{q_scale} splits={num_splits} "
          f"fill={fill} {kw}", flush=True)
    append_both(w, cfg, g, o, 0, seq_len, batch, spike=spike)
    q = synth.queries(w, batch=batch, scale=q_scale)
    got = gpu_decode(w, cfg, g, seq_len, q, batch)
    ref = oracle_decode(w, o, seq_len, q)
    err = rel_err(got, ref)
    print(f"  rel err {err:.3e}", flush=True)
    return err


@pytest.mark.parametrize("hq,hkv,dh,rv", [
    (8, 8, 128, 256),      # G 1, two KV heads per score wave, two groups per value wave
    (16, 8, 128, 512),     # G 2
    (16, 4, 192, 768),     # G 4 (MFMA scores), six groups per value wave
    (16, 2, 256, 512),     # G 8
    (32, 32, 128, 1024),   # the measured shape: eight KV heads per wave, R_v 1024
])
def test_u4_shapes(hq, hkv, dh, rv):
    assert run_u4(777, n_q_heads=hq, n_kv_heads=hkv, head_dim=dh, value_rank=rv) <= TOL


@pytest.mark.parametrize("seq_len,splits", [(1, 0), (65, 0), (1000, 3), (2000, 64)])
def test_u4_lengths_and_splits(seq_len, splits):
    assert run_u4(seq_len, num_splits=splits, n_q_heads=8, n_kv_heads=8,
                  value_rank=1024) <= TOL


def test_u4_peaked_rotation_off():
    assert run_u4(700, q_scale=8.0, spike={5: 6.0, 650: -6.0, 300: 5.0}, rotate=False,
                  n_q_heads=8, n_kv_heads=2, value_rank=256) <= TOL


def test_u4_nan_unused_slots():
    assert run_u4(333, fill=0xFF, n_q_heads=4, n_kv_heads=4, value_rank=512) <= TOL

