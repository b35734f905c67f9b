"""GPU value/output factor fusion and decode through it, vs the fp64 oracle
(review section 5.3, eq. 12; Algorithm 2, steps 7-8).

* starkv_fuse_value_output: every entry of the GPU's fused factor F (bf16,
  read back through its documented layout) is within one bf16 rounding of
  the oracle's fp64 F_h = B_value[g(h)]^T O_h (same bf16 inputs): relative
  2^-8 of the entry plus 2^-20 of max|F| for fp32 accumulation of d_h terms.
* starkv_decode_hidden: y = sum_h obar_h F_h against the oracle's latent
  attention rows (same cache bytes, factors, query) times the GPU's own F
  in fp64: max|gpu - ref| / max|ref| <= 5e-3.
"""

import math

import numpy as np
import pytest

import synth
from oracle import attention as oa
from oracle import cache as oc

from helpers import TOL, append_both, config_for, dev, fill_random, rel_err, sk

pytestmark = pytest.mark.gpu


def unblock_F(raw, hq, rv, D):
    """[D/16][Hq*R_v/8][16][8] bf16 bits -> F [Hq, R_v, D] float64."""
    K = hq * rv
    a = raw.reshape(D // 16, K // 8, 16, 8).transpose(1, 3, 0, 2).reshape(K, D)
    f = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return f.reshape(hq, rv, D)


def make_wo(w, D, seed):
    rng = np.random.default_rng(seed)
    return synth.round_to_bf16(rng.standard_normal((w.n_q_heads * w.head_dim, D))
                               / math.sqrt(w.n_q_heads * w.head_dim))


@pytest.mark.parametrize("name,batch,seq_len,D,kw", [
    ("l2_q43", 3, 700, 512, dict(n_q_heads=8, n_kv_heads=8, value_rank=256)),
    ("l3_gqa_q43", 2, 1000, 384, {}),
    ("l2_bf16", 2, 300, 256, dict(n_q_heads=8, n_kv_heads=4, value_rank=512)),
    ("l2_q43", 17, 333, 128, dict(n_q_heads=4, n_kv_heads=4, value_rank=256)),
    ("l2_q43", 70, 100, 256, dict(n_q_heads=4, n_kv_heads=4, value_rank=256)),
    ("l2_q4", 2, 500, 256, dict(n_q_heads=8, n_kv_heads=8, value_rank=512)),
])
def test_fused_factor_and_hidden_decode(name, batch, seq_len, D, kw):
    import torch
    w = synth.WORKLOADS[name].replace(batch=batch, **kw)
    T = ((seq_len + 63) // 64 + 1) * 64
    cfg = config_for(w, max_tokens=T)
    g = sk().LatentCache(cfg)
    o = oc.Cache.for_workload(w, max_tokens=T)
    fill_random(g, o, seed=seq_len)
    print(f"hidden {name} B={batch} T={seq_len} D={D} {kw}", flush=True)
    append_both(w, cfg, g, o, 0, seq_len, batch)
    bk, bv = synth.factors(w)
    bk, bv = synth.round_to_bf16(bk), synth.round_to_bf16(bv)
    w_o = make_wo(w, D, seed=D)
    bf = torch.bfloat16
    F = torch.empty(sk().starkv_fused_factor_bytes(cfg, D), dtype=torch.uint8, device="cuda")
    sk().starkv_fuse_value_output(cfg, dev(bv, bf), dev(w_o, bf), D, F)
    q = synth.round_to_bf16(synth.queries(w) * 4.0)
    y = torch.empty((batch, D), device="cuda")
    ws = torch.empty(sk().starkv_decode_hidden_workspace_bytes(cfg, seq_len, D),
                     dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(w.head_dim)
    sk().starkv_decode_hidden(cfg, g, seq_len, dev(q, bf), dev(bk, bf), F, D, scale, y, ws)
    torch.cuda.synchronize()
    Fg = unblock_F(F.cpu().numpy().view(np.uint16), w.n_q_heads, w.value_rank, D)
    Fr = oa.fuse_value_output(bv, w_o, w.n_q_heads, w.n_kv_heads, w.head_dim)
    bound = 2.0 ** -8 * np.abs(Fr) + 2.0 ** -20 * np.abs(Fr).max()
    assert np.all(np.abs(Fg - Fr) <= bound)
    rows = oa.decode_latent_rows(o, seq_len, q, bk, scale, w.n_q_heads, w.rotate,
                                 unrotated=True)
    ref = np.einsum("bhr,hrn->bn", rows, Fg)
    got = y.cpu().numpy().astype(np.float64)
    err = rel_err(got, ref)
    print(f"  F max rel {np.abs(Fg - Fr).max() / np.abs(Fr).max():.2e}, y rel err {err:.3e}",
          flush=True)
    assert err <= TOL
