"""GPU decode attention vs the fp64 oracle on the same seeded inputs.

Bar: max|gpu - ref| / max|ref| <= 5e-3.  Sizes span several 64-token tiles
and a ragged tail; stress variants sharpen the softmax (q x 8) or plant an
outlier token, so score errors cannot hide behind a near-uniform softmax;
unused cache slots hold random bytes or 0xFF (NaN patterns) that masking must
keep out.
"""

import numpy as np
import pytest

import synth
from oracle import cache as oc

from helpers import (TOL, append_both, config_for, fill_byte, fill_random,
                     gpu_decode, oracle_decode, rel_err, sk)

pytestmark = pytest.mark.gpu


def run_case(name, seq_len, batch=2, q_scale=1.0, spike=None, num_splits=0,
             fill="random", max_tokens=None, **kw):
    w = synth.WORKLOADS[name].replace(batch=batch, **kw)
    T = max_tokens or ((seq_len + 63) // 64 + 1) * 64
    cfg = config_for(w, max_tokens=T, num_splits=num_splits)
    g = sk().LatentCache(cfg)
    o = oc.Cache.for_workload(w, max_tokens=T)
    if fill == "random":
        fill_random(g, o, seed=seq_len)
    else:
        fill_byte(g, o, fill)
    print(f"decode {name} B={batch} T={seq_len} qx{q_scale} spike={spike} "
          f"splits={num_splits} fill={fill}", flush=True)
    append_both(w, cfg, g, o, 0, seq_len, batch, spike=spike)
    q = synth.queries(w, batch=batch, scale=q_scale)
    got = gpu_decode(w, cfg, g, seq_len, q, batch)
    ref = oracle_decode(w, o, seq_len, q)
    err = rel_err(got, ref)
    print(f"  rel err {err:.3e}", flush=True)
    return err, got


def test_tiny_workload_exact_shape():
    """The tiny workload as specified: B=1, 4 heads, d_h 64, T=256, fp32."""
    err, _ = run_case("tiny", 256, batch=1)
    assert err <= TOL


@pytest.mark.parametrize("name,seq_len", [
    ("tiny", 100), ("tiny", 1), ("l2_bf16", 1000), ("l2_bf16", 64),
    ("l2_q43", 1000), ("l2_q43", 777), ("l2_q43", 1), ("l2_q43", 65),
    ("l3_gqa_q43", 777), ("l3_gqa_q43", 130)])
def test_decode_parity(name, seq_len):
    err, _ = run_case(name, seq_len)
    assert err <= TOL


@pytest.mark.parametrize("name", ["tiny", "l2_bf16", "l2_q43", "l3_gqa_q43"])
def test_peaked_softmax(name):
    err, _ = run_case(name, 700, q_scale=8.0, spike={5: 6.0, 650: -6.0, 300: 5.0})
    assert err <= TOL


@pytest.mark.parametrize("name", ["l2_q43", "l3_gqa_q43"])
def test_rising_scores(name):
    """One token per tile with a latent row scaled up tile after tile: the
    running max of many heads moves again and again along the split, so the
    rescaling of the value accumulators runs on most tiles."""
    n = 1100
    spike = {64 * i + 9: 1.0 + 0.3 * i for i in range(n // 64)}
    err, _ = run_case(name, n, q_scale=8.0, spike=spike, num_splits=2)
    assert err <= TOL


@pytest.mark.parametrize("splits", [40, 64, 65])
def test_gqa_forced_splits(splits):
    """Value rank 256: up to 64 splits merge and up-project in one kernel
    (16 split rows requested up front, the rest in a loop); 65 splits take
    the separate merge and up-projection kernels."""
    # one tile per split (the last one ragged), so the split count is exact
    err, _ = run_case("l3_gqa_q43", 64 * splits - 7, num_splits=splits, q_scale=4.0)
    assert err <= TOL


@pytest.mark.parametrize("splits", [1, 3, 7])
def test_forced_splits(splits):
    err, _ = run_case("l2_q43", 900, num_splits=splits, q_scale=4.0)
    assert err <= TOL


@pytest.mark.parametrize("name", ["l2_bf16", "l2_q43", "tiny"])
def test_nan_poisoned_unused_slots(name):
    err, got = run_case(name, 333, fill=0xFF)
    assert np.isfinite(got).all()
    assert err <= TOL


def test_rotation_off_and_mha_subset():
    err, _ = run_case("l2_q43", 500, rotate=False)
    assert err <= TOL
    err, _ = run_case("l2_q43", 500, n_q_heads=8, n_kv_heads=8, value_rank=512)
    assert err <= TOL


def test_gqa_group_of_two_and_eight():
    err, _ = run_case("l3_gqa_q43", 300, n_q_heads=16, n_kv_heads=8)
    assert err <= TOL
    err, _ = run_case("l3_gqa_q43", 300, n_q_heads=32, n_kv_heads=4)
    assert err <= TOL


def test_deterministic_run_to_run():
    w = synth.WORKLOADS["l2_q43"].replace(batch=2)
    cfg = config_for(w, max_tokens=1024)
    g = sk().LatentCache(cfg)
    append_both(w, cfg, g, None, 0, 1000, 2)
    q = synth.queries(w, batch=2)
    a = gpu_decode(w, cfg, g, 1000, q, 2)
    b = gpu_decode(w, cfg, g, 1000, q, 2)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name,kw", [
    # one KV head per query head, 8-channel keys (whole rows, values early)
    ("l2_bf16", dict(n_q_heads=8, n_kv_heads=8, key_rank=8, value_rank=64)),
    # groups of 2, 24-channel keys in 32-channel registers, R_v 96
    ("l2_bf16", dict(n_q_heads=8, n_kv_heads=4, key_rank=24, value_rank=96)),
    # groups of 4, 64-channel keys (chunk loop), R_v 160 (idle value waves)
    ("l2_bf16", dict(n_q_heads=16, n_kv_heads=4, key_rank=64, value_rank=160)),
    # fp32, groups of 8, 40-channel keys
    ("tiny", dict(n_q_heads=16, n_kv_heads=2, head_dim=128, key_rank=40, value_rank=256)),
])
def test_plain_cache_shapes(name, kw):
    """Unquantized caches across the key-row and group-size variants of the
    plain split kernel, with a ragged tail."""
    err, _ = run_case(name, 333, q_scale=4.0, **kw)
    assert err <= TOL


@pytest.mark.parametrize("kw", [
    # one KV head (score waves 1-3 idle), groups of 8, d_h 256
    dict(n_q_heads=8, n_kv_heads=1, head_dim=256, value_rank=256),
    # two KV heads, groups of 2
    dict(n_q_heads=4, n_kv_heads=2, value_rank=256),
    # 16 KV heads in groups of 2, R_v 768 (six value groups per value wave)
    dict(n_q_heads=32, n_kv_heads=16, value_rank=768),
    # four KV heads in groups of 4 (MFMA scores, one KV head per score
    # wave), R_v 512
    dict(n_q_heads=16, n_kv_heads=4, value_rank=512),
])
def test_q43_shapes(kw):
    """4/3-bit caches across the score-wave head counts and value-wave group
    counts of the split kernel, with a ragged tail and a peaked softmax."""
    err, _ = run_case("l3_gqa_q43", 333, q_scale=4.0, **kw)
    assert err <= TOL


@pytest.mark.parametrize("name,batch,splits,kw", [
    # one sequence; weights of splits past the first 64 lanes
    ("l2_q43", 1, 70, dict()),
    # three sequences, value rank 512
    ("l2_q43", 3, 20, dict(value_rank=512)),
    # nine sequences, value rank 768
    ("l2_q43", 9, 5, dict(n_q_heads=8, n_kv_heads=8, value_rank=768)),
    # d_h 64
    ("l2_q43", 5, 12, dict(n_q_heads=8, n_kv_heads=8, head_dim=64, value_rank=512)),
    # 256 and 257 splits (splits dealt out among 4 waves per channel block)
    ("l2_q43", 2, 256, dict(n_q_heads=8, n_kv_heads=8, value_rank=512)),
    ("l2_q43", 2, 257, dict(n_q_heads=8, n_kv_heads=8, value_rank=512)),
    # bf16 cache (no rotation), value rank 1024, three sequences
    ("l2_bf16", 3, 33, dict()),
])
def test_wide_value_merge(name, batch, splits, kw):
    """Merge and up-projection for value ranks 512, 768 and 1024: batches
    that fill no multiple of 4 or 8 sequences, both head sizes, and split
    counts from 5 to 257 (one tile per split)."""
    # one tile per split (the last one ragged), so the split count is exact
    err, _ = run_case(name, 64 * splits - 7, batch=batch, num_splits=splits, q_scale=4.0, **kw)
    assert err <= TOL
