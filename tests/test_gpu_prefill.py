"""GPU chunked causal prefill vs the fp64 oracle on the same seeded inputs.

Per case:
* z_debug (the GPU's Z = X [A_key | A_value], bf16 inputs, fp32 result) is
  compared with the oracle's projection (X A in fp64, rounded to fp32):
  max|gpu - ref| / max|ref| <= 1e-4 (bf16 products are exact in fp32; the
  bound covers fp32 accumulation over D);
* the cache bytes after the call equal, bit for bit, the oracle packer
  applied to the GPU's z_debug on top of the same context bytes;
* the output equals oracle causal attention over those same bytes (query i
  at position ctx + i sees positions 0 .. ctx + i): max|gpu - ref| /
  max|ref| <= 5e-3.
Shapes span several tiles, ragged chunks and contexts, GQA group sizes
1/2/4/8, every supported value rank, rotation on and off, a batch of two,
a peaked softmax and NaN bytes in unused cache slots.  Rotary keys (review
section 5.3, Algorithm 2 steps 4b-4c): the same checks against the oracle
with RoPE on keys (at their positions) and queries (at ctx + i), d_h 64
and 128, GQA 1/2/4/8, both cache precisions, rotation on and off.
"""

import math

import numpy as np
import pytest

import synth
from oracle import attention as oa
from oracle import cache as oc

from helpers import TOL, append_both, config_for, dev, fill_byte, fill_random, rel_err, sk

pytestmark = pytest.mark.gpu

SMALL = dict(n_q_heads=8, n_kv_heads=8, head_dim=64, value_rank=256, hidden=128)


def chunk_inputs(w, chunk, batch, q_scale):
    """x [B, C, D], q [B, C, Hq, d_h] (per sequence seeds), shared A."""
    xs, qs = [], []
    ak = av = None
    for b in range(batch):
        x, a_k, a_v, q = synth.prefill_inputs(w.replace(seed=w.seed + 1000 * b), chunk)
        if b == 0:
            _, ak, av, _ = synth.prefill_inputs(w, chunk)
        xs.append(x)
        qs.append(synth.round_to_bf16(q * q_scale))
    return np.stack(xs), ak, av, np.stack(qs)


def run_prefill(ctx, chunk, batch=1, q_scale=1.0, rows=None, heads=None,
                fill="random", oracle_context=True, name="longchat_prefill",
                key_ranks=None, rope_theta=0.0, **kw):
    import torch
    w = synth.WORKLOADS[name].replace(batch=batch, **kw)
    T = ((ctx + chunk + 63) // 64 + 1) * 64
    cfg = config_for(w, max_tokens=T, key_ranks=key_ranks, rope_theta=rope_theta)
    g = sk().LatentCache(cfg)
    o = oc.Cache.for_workload(w, max_tokens=T, key_ranks=key_ranks)
    if fill == "random":
        fill_random(g, o, seed=ctx * 7 + chunk)
    else:
        fill_byte(g, o, fill)
    print(f"prefill B={batch} ctx={ctx} C={chunk} Hq={w.n_q_heads} Hkv={w.n_kv_heads} "
          f"dh={w.head_dim} rv={w.value_rank} D={w.hidden} rot={w.rotate} "
          f"qx{q_scale} fill={fill} theta={rope_theta}", flush=True)
    if ctx:
        append_both(w, cfg, g, o if oracle_context else None, 0, ctx, batch)
    if not oracle_context:
        # the context's packing is covered by the append tests: start the
        # oracle from the GPU's context bytes
        for i, key in enumerate(("key", "key_meta", "value", "value_meta")):
            o.buf[key][:] = g.buffers[i][:o.buf[key].size].cpu().numpy()
    x, ak, av, q = chunk_inputs(w, chunk, batch, q_scale)
    bk, bv = synth.factors(w)
    nk = w.n_kv_heads * w.key_rank
    out = torch.empty((batch, chunk, w.n_q_heads, w.head_dim), device="cuda")
    zdbg = torch.empty((batch, chunk, nk + w.value_rank), device="cuda")
    ws = sk().workspace(cfg, sk().OP_PREFILL, chunk)
    bf = torch.bfloat16
    scale = 1.0 / math.sqrt(w.head_dim)
    sk().starkv_prefill(cfg, g, ctx, chunk, dev(x, bf), w.hidden, dev(ak, bf),
                        dev(av, bf), dev(q, bf), dev(bk, bf), dev(bv, bf), scale,
                        out, ws, z_debug=zdbg)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    z = zdbg.cpu().numpy()

    # projection: the oracle's Z = X A (review Algorithm 2, step 1)
    zref = []
    for b in range(batch):
        zk_ref, zv_ref = oa.project_latents(x[b], ak, av, w.n_kv_heads, w.key_rank)
        zref.append(np.concatenate([zk_ref.reshape(chunk, nk), zv_ref], axis=1))
    zerr = rel_err(z.astype(np.float64), np.stack(zref).astype(np.float64))
    # packing of the GPU's latents
    o.append(z[:, :, :nk].reshape(batch, chunk, w.n_kv_heads, w.key_rank),
             z[:, :, nk:], ctx, chunk)
    for i, key in enumerate(("key", "key_meta", "value", "value_meta")):
        n = o.buf[key].size
        gb = g.buffers[i][:n].cpu().numpy()
        assert np.array_equal(gb, o.buf[key]), f"cache bytes differ in {key}"
    # attention over the stored bytes
    errs = []
    for b in range(batch):
        ref = oa.causal_attention(o, ctx, q[b], bk, bv, scale, w.n_q_heads,
                                  w.rotate, rows=rows, heads=heads, batch=b,
                                  rope_theta=rope_theta)
        gb = got[b]
        if rows is not None:
            gb = gb[np.asarray(rows)]
        if heads is not None:
            gb = gb[:, np.asarray(heads)]
        errs.append(rel_err(gb, ref))
    err = max(errs)
    print(f"  z rel err {zerr:.2e}, out rel err {err:.3e}", flush=True)
    return zerr, err, got


@pytest.mark.parametrize("ctx,chunk", [(100, 37), (0, 1), (0, 200), (64, 64),
                                       (131, 9), (5, 130)])
def test_prefill_parity(ctx, chunk):
    zerr, err, _ = run_prefill(ctx, chunk, **SMALL)
    assert zerr <= 1e-4
    assert err <= TOL


@pytest.mark.parametrize("hq,hkv,dh,rv", [(16, 4, 192, 768), (16, 2, 256, 512),
                                          (16, 8, 64, 256), (16, 16, 64, 1024)])
def test_prefill_gqa_and_ranks(hq, hkv, dh, rv):
    """Group sizes 4, 8, 2, 1 and value ranks 768, 512, 256, 1024 (the joint
    value latent needs R_v <= Hkv * d_h for orthonormal factors)."""
    kw = dict(SMALL, n_q_heads=hq, n_kv_heads=hkv, head_dim=dh, value_rank=rv)
    zerr, err, _ = run_prefill(77, 100, **kw)
    assert zerr <= 1e-4
    assert err <= TOL


def test_prefill_batch_rotation_off_and_peaked():
    zerr, err, _ = run_prefill(70, 45, batch=2, q_scale=8.0, rotate=False, **SMALL)
    assert zerr <= 1e-4
    assert err <= TOL


def test_prefill_per_head_key_ranks():
    """Per-head key ranks on the quantized cache (heads padded to the
    32-channel key tile): the appended chunk's padded channels are zero and
    the query side drops the factor columns past each head's rank."""
    ranks = [8, 32, 16, 24, 8, 16, 32, 24]
    zerr, err, _ = run_prefill(100, 70, key_ranks=ranks, **SMALL)
    assert zerr <= 1e-4
    assert err <= TOL


@pytest.mark.parametrize("rotate", [True, False])
def test_prefill_uniform_4bit(rotate):
    """A uniform 4-bit cache (both precision blocks at 4 bits): the key
    pre-pass reads four nibble planes, every value group takes the 4-bit
    operand path."""
    zerr, err, _ = run_prefill(100, 77, lo_bits=4, rotate=rotate, **SMALL)
    assert zerr <= 1e-4
    assert err <= TOL


def test_prefill_uniform_4bit_gqa_wide():
    """G 4, R_v 1024 (two column blocks of sixteen 4-bit groups each)."""
    kw = dict(SMALL, n_q_heads=16, n_kv_heads=4, head_dim=256, value_rank=1024)
    zerr, err, _ = run_prefill(64, 130, lo_bits=4, **kw)
    assert zerr <= 1e-4
    assert err <= TOL


def test_prefill_nan_unused_slots():
    """Unused cache bytes are 0xFF (NaN scales and zeros): masking keeps
    them out of every operand."""
    zerr, err, got = run_prefill(30, 50, fill=0xFF, **SMALL)
    assert np.isfinite(got).all()
    assert err <= TOL


def test_prefill_full_size_sampled():
    """The full chunked-prefill workload: 8192 queries against 24576 cached
    tokens (LongChat-7B shape, 4/3-bit rotated), checked on sampled rows and
    heads; bytes and projection checked in full."""
    w = synth.WORKLOADS["longchat_prefill"]
    rows = [0, 1, 63, 64, 4095, 8190, 8191]
    heads = [0, 13, 31]
    zerr, err, _ = run_prefill(w.seq_len, w.chunk, rows=rows, heads=heads,
                               oracle_context=False)
    assert zerr <= 1e-4
    assert err <= TOL


@pytest.mark.parametrize("ctx,chunk,hq,hkv,dh,rv,rotate", [
    (100, 70, 8, 8, 128, 256, True),       # 2 heads x 64 queries per workgroup
    (37, 130, 16, 8, 64, 512, True),       # 4 heads x 32 queries, G = 2
    (0, 90, 32, 8, 128, 1024, False),      # G = 4, two value column blocks
    (200, 67, 16, 2, 128, 256, True),      # G = 8
    (64, 1, 8, 8, 64, 256, True),          # a single query
])
def test_prefill_rotary_keys(ctx, chunk, hq, hkv, dh, rv, rotate):
    kw = dict(SMALL, n_q_heads=hq, n_kv_heads=hkv, head_dim=dh, value_rank=rv,
              rotate=rotate)
    zerr, err, _ = run_prefill(ctx, chunk, rope_theta=10000.0, **kw)
    assert zerr <= 1e-4
    assert err <= TOL


def test_prefill_rotary_keys_peaked_batch_uniform_4bit():
    """A batch of two with sharpened queries, far positions (theta 500 turns
    the pairs quickly) and the uniform 4-bit cache."""
    kw = dict(SMALL, head_dim=128, lo_bits=4)
    zerr, err, _ = run_prefill(300, 77, batch=2, q_scale=4.0, rope_theta=500.0, **kw)
    assert zerr <= 1e-4
    assert err <= TOL


def test_prefill_rotary_keys_per_head_ranks():
    kw = dict(SMALL, head_dim=128, n_q_heads=8, n_kv_heads=4)
    zerr, err, _ = run_prefill(90, 60, key_ranks=[8, 32, 16, 24], rope_theta=10000.0, **kw)
    assert zerr <= 1e-4
    assert err <= TOL


def test_prefill_rotary_keys_full_size_sampled():
    """The full chunked-prefill workload with rotary keys (theta 10000, the
    LLaMA base): 8192 queries at positions 24576 .. 32767, sampled rows and
    heads; bytes and projection checked in full."""
    w = synth.WORKLOADS["longchat_prefill"]
    rows = [0, 63, 64, 4095, 8191]
    heads = [0, 17, 31]
    zerr, err, _ = run_prefill(w.seq_len, w.chunk, rows=rows, heads=heads,
                               oracle_context=False, rope_theta=10000.0)
    assert zerr <= 1e-4
    assert err <= TOL


@pytest.mark.parametrize("case", [
    dict(ctx=30, chunk=150, fill=0xFF),                          # NaN unused slots
    dict(ctx=100, chunk=160, lo_bits=4),                         # uniform 4-bit
    dict(ctx=70, chunk=140, batch=2, q_scale=8.0, rotate=False),
    dict(ctx=100, chunk=150, key_ranks=[8, 32, 16, 24, 8, 16, 32, 24]),
    dict(ctx=40, chunk=150, n_q_heads=16, n_kv_heads=2, head_dim=128),   # G = 8
    dict(ctx=90, chunk=100, n_q_heads=16, n_kv_heads=4, head_dim=128, value_rank=512),
    # 16 KV heads (two per XCD in the workgroup order) and 3 query blocks
    # of a ragged chunk, padded to 8
    dict(ctx=77, chunk=600, n_q_heads=16, n_kv_heads=16, value_rank=512),
])
def test_prefill_reconstructed_values(case):
    """Chunks long enough that the values of every visible position are
    reconstructed once per call (C Hq (R_v - d_h) > Hkv d_h R_v: eq. 12 in
    its left-hand order) and the attention contracts over d_h: the same
    bar against the oracle, with unused slots NaN-filled, the uniform 4-bit
    cache, a peaked batch of two without rotation, per-head key ranks, G 8,
    d_h 128, and 16 KV heads over several query blocks."""
    kw = dict(SMALL)
    kw.update(case)
    ctx, chunk = kw.pop("ctx"), kw.pop("chunk")
    hq, hkv, dh, rv = kw["n_q_heads"], kw["n_kv_heads"], kw["head_dim"], kw["value_rank"]
    assert chunk * hq * (rv - dh) > hkv * dh * rv          # the reconstructing path
    assert rv <= hkv * dh                                  # orthonormal synthetic factors
    zerr, err, got = run_prefill(ctx, chunk, **kw)
    assert np.isfinite(got).all()
    assert zerr <= 1e-4
    assert err <= TOL
