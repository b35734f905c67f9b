"""GPU paged / ragged 4/3-bit caches against the oracle's paged forms.

The contiguous cache is filled on both sides, then both are permuted into a
page pool by the same random page table.  starkv_decode_paged with ragged
lengths (one of them 0) must match oracle.paged.decode_paged to the decode
bound (max|gpu - ref| / max|ref| <= 5e-3; the zero-length row exactly 0);
starkv_append_paged of one token per sequence at its own position must
leave the pool bit-identical to oracle.paged.append_paged; a decode after
the append checks the grown sequences.  Also with rotary keys (each query at
its own sequence's last position) and grouped heads.
"""

import math

import numpy as np
import pytest

import synth
from oracle import cache as oc
from oracle import paged

from helpers import TOL, append_both, config_for, dev, fill_random, qbits, rel_err, sk

pytestmark = pytest.mark.gpu

KEYS = ("key", "key_meta", "value", "value_meta")


def permute(gcache, ocache, table):
    """Pool page table[b][t] <- contiguous tile b*NT + t, on both sides."""
    import torch
    n = ocache.B * ocache.nt
    idx = torch.from_numpy(table.reshape(-1).astype(np.int64)).cuda()
    for i, k in enumerate(KEYS):
        g = gcache.buffers[i][:ocache.buf[k].size].view(n, -1)
        g.copy_(g.clone().index_copy_(0, idx, g.clone()))
        o = ocache.buf[k].reshape(n, -1)
        o[table.reshape(-1)] = o.copy()


def run_paged(name, batch, ctx, lens, rope=0.0, seed=0, **kw):
    import torch
    w = synth.WORKLOADS[name].replace(batch=batch, **kw)
    T = ((ctx + 1 + 63) // 64 + 1) * 64
    cfg = sk().make_config(batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.key_rank,
                           w.value_rank, T, w.cache, w.rotate, rope_theta=rope,
                           **qbits(w))
    g = sk().LatentCache(cfg)
    o = oc.Cache.for_workload(w, max_tokens=T)
    fill_random(g, o, seed=ctx + seed)
    print(f"paged {name} B={batch} ctx={ctx} lens={lens} rope={rope} {kw}", flush=True)
    append_both(w, cfg, g, o, 0, ctx, batch)
    rng = np.random.default_rng(seed + 99)
    table = rng.permutation(batch * o.nt).reshape(batch, o.nt).astype(np.int32)
    permute(g, o, table)
    table_d = torch.from_numpy(table).cuda()
    bk, bv = synth.factors(w)
    q = synth.round_to_bf16(synth.queries(w) * 4.0)
    bf = torch.bfloat16
    s = 1.0 / math.sqrt(w.head_dim)
    out = torch.empty((batch, w.n_q_heads, w.head_dim), device="cuda")

    def decode(lens_now):
        mx = max(max(lens_now), 1)
        ws = sk().workspace(cfg, sk().OP_DECODE, mx)
        sk().starkv_decode_paged(cfg, g, table_d, torch.tensor(lens_now, dtype=torch.int32,
                                                               device="cuda"),
                                 mx, dev(q, bf), dev(bk, bf), dev(bv, bf), s, out, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        ref = paged.decode_paged(o, table, lens_now, q, bk, bv, s, w.n_q_heads, w.rotate,
                                 rope_theta=rope)
        for b, n in enumerate(lens_now):
            if n == 0:
                assert np.array_equal(got[b], np.zeros_like(got[b]))
        live = [b for b, n in enumerate(lens_now) if n > 0]
        err = rel_err(got[live], ref[live])
        print(f"  lens {lens_now}: rel err {err:.3e}", flush=True)
        return err

    err1 = decode(lens)
    # one more token per sequence, each at its own end
    pos = [min(n, T - 1) for n in lens]
    zk = rng.standard_normal((batch, w.n_kv_heads, w.key_rank)).astype(np.float32) * 0.5
    zv = rng.standard_normal((batch, w.value_rank)).astype(np.float32) * 0.2
    sk().starkv_append_paged(cfg, g, table_d, torch.tensor(pos, dtype=torch.int32,
                                                          device="cuda"), dev(zk), dev(zv))
    torch.cuda.synchronize()
    paged.append_paged(o, table, pos, zk, zv)
    for i, k in enumerate(KEYS):
        assert np.array_equal(g.buffers[i][:o.buf[k].size].cpu().numpy(), o.buf[k]), k
    err2 = decode([p + 1 for p in pos])
    return max(err1, err2)


@pytest.mark.parametrize("lens", [[700, 1, 355, 640], [64, 0, 700, 129]])
def test_paged_ragged_mha(lens):
    assert run_paged("l2_q43", 4, 700, lens, n_q_heads=8, n_kv_heads=8,
                     value_rank=256) <= TOL


def test_paged_ragged_gqa():
    assert run_paged("l3_gqa_q43", 3, 1000, [1000, 513, 17], n_q_heads=8,
                     n_kv_heads=2, seed=1) <= TOL


def test_paged_ragged_rope():
    assert run_paged("l2_q43", 3, 500, [500, 200, 65], rope=10000.0, n_q_heads=8,
                     n_kv_heads=8, value_rank=256, seed=2) <= TOL


def test_paged_ragged_uniform_4bit():
    assert run_paged("l2_q4", 3, 700, [700, 1, 300], n_q_heads=8, n_kv_heads=8,
                     value_rank=256, seed=3) <= TOL


@pytest.mark.parametrize("name,ctx,chunk", [("longchat_prefill", 100, 70),
                                            ("longchat_prefill", 64, 129)])
def test_paged_prefill(name, ctx, chunk):
    """starkv_prefill_paged over a permuted pool of two sequences: the pool's
    bytes after the call equal oracle.paged.prefill_paged's (fed the GPU's
    own chunk latents, whose projection test_gpu_prefill checks), and so do
    the outputs, to the decode bound."""
    run_paged_prefill(name, ctx, chunk, lo_bits=3)


def test_paged_prefill_uniform_4bit():
    run_paged_prefill("longchat_prefill", 90, 60, lo_bits=4)


def test_paged_prefill_rotary_keys():
    """Rotary keys over the paged pool: the key reconstruction reads each
    position's latent through the page table."""
    run_paged_prefill("longchat_prefill", 70, 100, lo_bits=3, rope_theta=10000.0,
                      head_dim=128)


def run_paged_prefill(name, ctx, chunk, lo_bits, rope_theta=0.0, head_dim=64):
    import torch
    B = 2
    w = synth.WORKLOADS[name].replace(batch=B, n_q_heads=8, n_kv_heads=8, head_dim=head_dim,
                                      value_rank=256, hidden=128, lo_bits=lo_bits)
    T = ((ctx + chunk + 63) // 64 + 1) * 64
    cfg = config_for(w, max_tokens=T, rope_theta=rope_theta)
    g = sk().LatentCache(cfg)
    o = oc.Cache.for_workload(w, max_tokens=T)
    fill_random(g, o, seed=ctx + chunk)
    print(f"paged prefill B={B} ctx={ctx} C={chunk} lo_bits={lo_bits} theta={rope_theta} "
          f"dh={head_dim}", flush=True)
    append_both(w, cfg, g, o, 0, ctx, B)
    rng = np.random.default_rng(ctx)
    table = rng.permutation(B * o.nt).reshape(B, o.nt).astype(np.int32)
    permute(g, o, table)
    xs, qs = [], []
    ak = av = None
    for b in range(B):
        x, a_k, a_v, q = synth.prefill_inputs(w.replace(seed=w.seed + 1000 * b), chunk)
        if b == 0:
            _, ak, av, _ = synth.prefill_inputs(w, chunk)
        xs.append(x)
        qs.append(synth.round_to_bf16(q))
    x, q = np.stack(xs), np.stack(qs)
    bk, bv = synth.factors(w)
    nk = w.n_kv_heads * w.key_rank
    bf = torch.bfloat16
    out = torch.empty((B, chunk, w.n_q_heads, w.head_dim), device="cuda")
    zdbg = torch.empty((B, chunk, nk + w.value_rank), device="cuda")
    ws = sk().workspace(cfg, sk().OP_PREFILL, chunk)
    s = 1.0 / math.sqrt(w.head_dim)
    sk().starkv_prefill_paged(cfg, g, torch.from_numpy(table).cuda(), ctx, chunk, dev(x, bf),
                              w.hidden, dev(ak, bf), dev(av, bf), dev(q, bf), dev(bk, bf),
                              dev(bv, bf), s, out, ws, z_debug=zdbg)
    torch.cuda.synchronize()
    z = zdbg.cpu().numpy()
    ref = paged.prefill_paged(o, table, ctx, z[:, :, :nk].reshape(B, chunk, w.n_kv_heads,
                                                                   w.key_rank),
                              z[:, :, nk:], q, bk, bv, s, w.n_q_heads, w.rotate,
                              rope_theta=rope_theta)
    for i, k in enumerate(KEYS):
        assert np.array_equal(g.buffers[i][:o.buf[k].size].cpu().numpy(), o.buf[k]), k
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    err = rel_err(got, ref)
    print(f"  rel err {err:.3e}", flush=True)
    assert err <= TOL
