"""GPU decode with per-head key ranks (technical review of arXiv 2606.08382,
section 4 / Fig. 2: learned per-head ranks; eq. 15), fp32 and bf16 caches
(heads stored at their own ranks) and quantized caches (heads padded to the
32-channel key tile: section 6.2, rank rounding to a supported kernel tile):
append bytes bit-exact against the oracle packer, decode within 5e-3 of the
oracle over the same bytes and factors (B_key padded to the largest rank;
its columns past a head's rank, and the latent input past it, are set to
large values so that using them would show)."""

import math

import numpy as np
import pytest

import synth
from oracle import attention as oa
from oracle import cache as oc

from helpers import TOL, dev, fill_random, rel_err, sk

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,hq,ranks,T", [
    ("bf16", 8, [8, 64, 24, 40, 16, 8, 32, 56], 700),
    ("bf16", 16, [16, 8, 32, 24], 300),
    ("f32", 4, [8, 16, 24, 32], 200),
    ("bf16", 32, [64] * 8 + [8] * 8 + [32] * 16, 500),
])
def test_per_head_key_ranks(kind, hq, ranks, T):
    import torch
    rng = np.random.default_rng(T + hq)
    B, H, d, R = 2, len(ranks), 128 if kind == "bf16" else 64, 256
    rk = max(ranks)
    Tm = ((T + 63) // 64 + 1) * 64
    cfg = sk().make_config(B, hq, H, d, rk, R, Tm, kind, key_ranks=ranks)
    g = sk().LatentCache(cfg)
    o = oc.Cache(B, H, rk, R, Tm, kind, key_ranks=ranks)
    fill_random(g, o, seed=T)
    print(f"ranks {kind} Hq={hq} Hkv={H} ranks={ranks} T={T}", flush=True)
    zk = (rng.standard_normal((B, T, H, rk)) * 0.5).astype(np.float32)
    zv = (rng.standard_normal((B, T, R)) * 0.3).astype(np.float32)
    sk().starkv_append(cfg, g, dev(zk), dev(zv), 0, T)
    o.append(zk, zv, 0, T)
    torch.cuda.synchronize()
    for i, k in enumerate(("key", "key_meta", "value", "value_meta")):
        n = o.buf[k].size
        assert np.array_equal(g.buffers[i][:n].cpu().numpy(), o.buf[k]), k
    bk = np.linalg.qr(rng.standard_normal((H, d, rk)))[0][:, :, :rk]
    for h, r in enumerate(ranks):
        bk[h, :, r:] = 1e4
    bv = np.linalg.qr(rng.standard_normal((H * d, R)))[0]
    dt = torch.float32 if kind == "f32" else torch.bfloat16
    if kind == "bf16":
        bk, bv = synth.round_to_bf16(bk), synth.round_to_bf16(bv)
    q = rng.standard_normal((B, hq, d)) * 4 / math.sqrt(d)
    if kind == "bf16":
        q = synth.round_to_bf16(q)
    out = torch.empty((B, hq, d), device="cuda")
    ws = sk().workspace(cfg, sk().OP_DECODE, T)
    s = 1 / math.sqrt(d)
    sk().starkv_decode(cfg, g, T, dev(q, dt), dev(bk, dt), dev(bv, dt), s, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = oa.decode(o, T, q, bk, bv, s, hq, False)
    assert np.isfinite(got).all()
    err = rel_err(got, ref)
    print(f"  rel err {err:.3e}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("hq,ranks,rotate,lo_bits,theta,T", [
    (8, [8, 24, 16, 32], True, 3, 0.0, 700),
    (8, [32, 8, 8, 16, 24, 32, 16, 8], False, 3, 0.0, 333),
    (16, [16, 24, 8, 32], True, 4, 0.0, 500),
    (8, [8, 32, 16, 24, 8, 16, 32, 24], True, 3, 10000.0, 600),
])
def test_quantized_per_head_key_ranks(hq, ranks, rotate, lo_bits, theta, T):
    import torch
    rng = np.random.default_rng(T + hq + lo_bits)
    B, H, d, R = 2, len(ranks), 128, 256
    Tm = ((T + 63) // 64 + 1) * 64
    cfg = sk().make_config(B, hq, H, d, 32, R, Tm, "q43", rotate, key_ranks=ranks,
                           lo_bits=lo_bits, rope_theta=theta)
    g = sk().LatentCache(cfg)
    o = oc.Cache(B, H, 32, R, Tm, "q43", rotate, key_ranks=ranks, lo_bits=lo_bits)
    fill_random(g, o, seed=T)
    print(f"q43 ranks Hq={hq} Hkv={H} ranks={ranks} rot={rotate} lo_bits={lo_bits} "
          f"theta={theta} T={T}", flush=True)
    zk = (rng.standard_normal((B, T, H, 32)) * 0.5).astype(np.float32)
    for h, r in enumerate(ranks):
        zk[:, :, h, r:] = 50.0          # input past a head's rank is dropped
    zv = (rng.standard_normal((B, T, R)) * 0.3).astype(np.float32)
    sk().starkv_append(cfg, g, dev(zk), dev(zv), 0, T)
    o.append(zk, zv, 0, T)
    torch.cuda.synchronize()
    for i, k in enumerate(("key", "key_meta", "value", "value_meta")):
        n = o.buf[k].size
        assert np.array_equal(g.buffers[i][:n].cpu().numpy(), o.buf[k]), k
    bk = np.linalg.qr(rng.standard_normal((H, d, 32)))[0]
    for h, r in enumerate(ranks):
        bk[h, :, r:] = 1e4
    bv = np.linalg.qr(rng.standard_normal((H * d, R)))[0]
    bk, bv = synth.round_to_bf16(bk), synth.round_to_bf16(bv)
    q = synth.round_to_bf16(rng.standard_normal((B, hq, d)) * 8 / math.sqrt(d))
    out = torch.empty((B, hq, d), device="cuda")
    ws = sk().workspace(cfg, sk().OP_DECODE, T)
    s = 1 / math.sqrt(d)
    bf = torch.bfloat16
    sk().starkv_decode(cfg, g, T, dev(q, bf), dev(bk, bf), dev(bv, bf), s, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = oa.decode(o, T, q, bk, bv, s, hq, rotate, rope_theta=theta)
    assert np.isfinite(got).all()
    err = rel_err(got, ref)
    print(f"  rel err {err:.3e}", flush=True)
    assert err <= TOL
