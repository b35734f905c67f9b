"""GPU decode with rotary position embedding fused into latent-key scoring
(technical review of arXiv 2606.08382, section 5.3: pre-RoPE latent keys,
reconstruction + rotation + scoring fused at runtime; Algorithm 2, steps
4b-4d), against the fp64 oracle reading the same cache bytes with the same
bf16 factors and query: max|gpu - ref| / max|ref| <= 5e-3.

Cases: several tiles with a ragged tail, forced splits, peaked queries,
grouped heads, head dim 64 and 128, rotation on and off, NaN-filled unused
cache bytes, base 1e4 and 5e5, and the full l2_q43 shape (B = 16,
T = 32768) checked on sampled sequences.
"""

import math

import numpy as np
import pytest

import synth
from oracle import attention as oa
from oracle import cache as oc

from helpers import (TOL, append_both, config_for, dev, fill_byte, fill_random, qbits,
                     rel_err, sk)

pytestmark = pytest.mark.gpu


def run_rope(name, seq_len, theta, batch=2, q_scale=4.0, num_splits=0, fill="random",
             rotate=None, sample=None, max_tokens=None, **kw):
    import torch
    w = synth.WORKLOADS[name].replace(batch=batch, **kw)
    T = max_tokens or ((seq_len + 63) // 64 + 1) * 64
    rot = w.rotate if rotate is None else rotate
    cfg = sk().make_config(batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.key_rank,
                           w.value_rank, T, w.cache, rot, num_splits, rope_theta=theta,
                           **qbits(w))
    g = sk().LatentCache(cfg)
    o = oc.Cache(batch, w.n_kv_heads, w.key_rank, w.value_rank, T, w.cache, rot,
                 lo_bits=w.lo_bits)
    if fill == "random":
        fill_random(g, o, seed=seq_len + 11)
    else:
        fill_byte(g, o, fill)
    print(f"rope {name} B={batch} T={seq_len} theta={theta} q*{q_scale} "
          f"splits={sk().starkv_decode_splits(cfg, seq_len)} rot={rot} {kw}", flush=True)
    wr = w.replace(rotate=rot)
    append_both(wr, cfg, g, o if sample is None else None, 0, seq_len, batch)
    if sample is not None:
        for i, key in enumerate(("key", "key_meta", "value", "value_meta")):
            o.buf[key][:] = g.buffers[i][:o.buf[key].size].cpu().numpy()
    bk, bv = synth.factors(w)
    q = synth.round_to_bf16(synth.queries(w) * q_scale)
    bf = torch.bfloat16
    out = torch.empty((batch, w.n_q_heads, w.head_dim), device="cuda")
    ws = sk().workspace(cfg, sk().OP_DECODE, seq_len)
    scale = 1.0 / math.sqrt(w.head_dim)
    sk().starkv_decode(cfg, g, seq_len, dev(q, bf), dev(bk, bf), dev(bv, bf), scale, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    bs = list(range(batch)) if sample is None else sample
    ref = oa.decode(o, seq_len, q, bk, bv, scale, w.n_q_heads, rot, batches=bs,
                    rope_theta=theta)
    assert np.isfinite(got).all()
    err = rel_err(got[bs], ref)
    print(f"  rel err {err:.3e}", flush=True)
    return err


@pytest.mark.parametrize("seq_len,splits", [(700, 0), (1000, 3), (64, 0), (1, 0), (130, 2)])
def test_rope_mha(seq_len, splits):
    assert run_rope("l2_q43", seq_len, 10000.0, num_splits=splits,
                    n_q_heads=8, n_kv_heads=8, value_rank=256) <= TOL


def test_rope_odd_head_count():
    """Three query heads: the second score wave owns a single head, and the
    MFMAs of its second head slot are skipped."""
    assert run_rope("l2_q43", 500, 10000.0, n_q_heads=3, n_kv_heads=3,
                    value_rank=256, q_scale=4.0) <= TOL


def test_rope_gqa_base_5e5():
    assert run_rope("l3_gqa_q43", 1000, 500000.0, n_q_heads=8, n_kv_heads=2) <= TOL


def test_rope_head_dim_64_rotation_off_peaked():
    assert run_rope("l2_q43", 500, 10000.0, q_scale=8.0, rotate=False, head_dim=64,
                    n_q_heads=8, n_kv_heads=8, value_rank=256) <= TOL


def test_rope_nan_unused_slots():
    assert run_rope("l2_q43", 333, 10000.0, fill=0xFF, n_q_heads=4, n_kv_heads=4,
                    value_rank=512) <= TOL


@pytest.mark.parametrize("hq,hkv,dh,rv", [(8, 8, 128, 256), (8, 4, 64, 256)])
def test_rope_uniform_4bit(hq, hkv, dh, rv):
    """Uniform 4-bit keys (four nibble planes) under the rotary scoring."""
    assert run_rope("l2_q4", 700, 10000.0, n_q_heads=hq, n_kv_heads=hkv, head_dim=dh,
                    value_rank=rv) <= TOL


def test_rope_gqa_full_shape_groups():
    """The l3_gqa_q43 grouping (32 query heads on 8 KV heads, R_v 256)."""
    assert run_rope("l3_gqa_q43", 2000, 500000.0, batch=2) <= TOL


def test_rope_full_l2_q43_sampled():
    """B = 16, T = 32768, 32 heads, R_v 1024, rotated 4/3-bit cache: every
    sequence decoded on the GPU, two checked against the oracle."""
    w = synth.WORKLOADS["l2_q43"]
    assert run_rope("l2_q43", w.seq_len, 10000.0, batch=w.batch, q_scale=2.0,
                    sample=[0, 15], max_tokens=w.max_tokens) <= TOL
