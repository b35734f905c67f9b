"""GPU decode at the workloads' full sizes, in the launch configuration the
benchmark times (automatic splits), checked against the fp64 oracle on
sampled sequences (all heads).

The cache is filled on the GPU with seeded random latents of the workload's
channel statistics (starkv_append), then its bytes are copied into the
oracle's cache object: the packing is covered bit for bit by the append
tests, and here the oracle decodes exactly the bytes the GPU decoded.
Bar: max|gpu - ref| / max|ref| <= 5e-3 per sampled sequence.
"""

import math

import numpy as np
import pytest

import synth
from oracle import attention as oa
from oracle import cache as oc

from helpers import TOL, config_for, dev, rel_err, sk, storage_dtype

pytestmark = pytest.mark.gpu


def fill_gpu(w, cfg, g, seq_len):
    import torch
    kstd = torch.tensor(synth.key_channel_std(w), dtype=torch.float32, device="cuda")
    vstd = torch.tensor(synth.value_channel_std(w), dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    for p0 in range(0, seq_len, 4096):
        n = min(4096, seq_len - p0)
        zk = torch.randn((w.batch, n, w.n_kv_heads, w.key_rank), device="cuda",
                         generator=gen) * kstd
        zv = torch.randn((w.batch, n, w.value_rank), device="cuda", generator=gen) * vstd
        sk().starkv_append(cfg, g, zk.contiguous(), zv.contiguous(), p0, n)
    torch.cuda.synchronize()


def run_full(name, batch, seq_len, sample):
    import torch
    w = synth.WORKLOADS[name].replace(batch=batch)
    T = ((seq_len + 63) // 64) * 64
    cfg = config_for(w, max_tokens=T)
    print(f"full decode {name} B={batch} T={seq_len} splits="
          f"{sk().starkv_decode_splits(cfg, seq_len)} sample={sample}", flush=True)
    g = sk().LatentCache(cfg, fill=0xFF)
    fill_gpu(w, cfg, g, seq_len)
    bk, bv = synth.factors(w)
    q = synth.queries(w, batch=batch, scale=4.0)
    dt = storage_dtype(w)
    out = torch.empty((batch, w.n_q_heads, w.head_dim), device="cuda")
    ws = sk().workspace(cfg, sk().OP_DECODE, seq_len)
    scale = 1.0 / math.sqrt(w.head_dim)
    sk().starkv_decode(cfg, g, seq_len, dev(q, dt), dev(bk, dt), dev(bv, dt), scale,
                       out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    o = oc.Cache.for_workload(w, max_tokens=T)
    for i, key in enumerate(("key", "key_meta", "value", "value_meta")):
        o.buf[key][:] = g.buffers[i][:o.buf[key].size].cpu().numpy()
    del g
    errs = []
    for b in sample:
        ref = oa.decode(o, seq_len, q, bk, bv, scale, w.n_q_heads, w.rotate,
                        batches=[b])
        errs.append(rel_err(got[b:b + 1], ref))
    print(f"  rel errs {[f'{e:.2e}' for e in errs]}", flush=True)
    assert np.isfinite(got).all()
    return max(errs)


@pytest.mark.parametrize("batch,sample", [(1, [0]), (4, [0, 3]), (16, [0, 9, 15])])
def test_full_bf16_t4096(batch, sample):
    assert run_full("l2_bf16", batch, 4096, sample) <= TOL


def test_full_q43_b16_t32768():
    """The measured workload: B=16, T=32768, 4/3-bit rotated cache."""
    assert run_full("l2_q43", 16, 32768, [0, 15]) <= TOL


def test_full_u4_b16_t32768():
    """The measured workload's shape with a uniform 4-bit cache."""
    assert run_full("l2_q4", 16, 32768, [0, 15]) <= TOL


def test_full_gqa_q43_b32_t16384():
    assert run_full("l3_gqa_q43", 32, 16384, [0, 31]) <= TOL


def test_full_tiny():
    assert run_full("tiny", 1, 256, [0]) <= TOL


def test_full_q43_b1_t131072():
    """One sequence of 128K tokens (the longest context of the pages' speed
    figures), 4/3-bit rotated: 256 automatic splits, so the merge deals the
    splits out among four waves per channel block over four batches of
    row loads, and the kernels index tiles up to 2047."""
    assert run_full("l2_q43", 1, 131072, [0]) <= TOL
