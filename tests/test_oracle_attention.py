"""Pins for the oracle's attention (CPU only).

Checked against what the pages and mathematics fix:
* with full rank, identity factors and an fp32 cache, the method is textbook
  softmax attention (technical review of arXiv 2606.08382, section 2.3):
  compare with a scalar-loop implementation and torch's float64 SDPA;
* brute force with scalar loops on tiny shapes (reconstruction of eq. 2);
* eq. 2 / eq. 12 reassociation: q (Z U^T)^T = (q U) Z^T and
  (P Z) U^T = P (Z U^T) -- the identity the latent-space GPU path relies on;
* the attention decomposition theorem (CaliDrop review) for split merges,
  including empty and single-token subsets;
* GQA -> MHA with duplicated heads, token-permutation invariance, prefill row
  i == decode at seq_len T0+i+1, causality;
* a quantized + rotated cache stays within its quantization error of the
  exact-latent attention (catches a wrong rotation or scale).
"""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import attention as oa
from oracle import cache as oc


def _f32_cache(b, hkv, rk, rv, t, rng):
    c = oc.Cache(b, hkv, rk, rv, ((t + 63) // 64) * 64, "f32")
    zk = rng.standard_normal((b, t, hkv, rk)).astype(np.float32)
    zv = rng.standard_normal((b, t, rv)).astype(np.float32)
    c.append(zk, zv, 0, t)
    return c, zk, zv


def test_full_rank_identity_factors_is_textbook_attention():
    rng = np.random.default_rng(0)
    b, hq, d, t = 2, 4, 16, 77
    c, zk, zv = _f32_cache(b, hq, d, hq * d, t, rng)
    bk = np.stack([np.eye(d)] * hq)
    bv = np.eye(hq * d)
    q = rng.standard_normal((b, hq, d))
    scale = 1 / math.sqrt(d)
    out = oa.decode(c, t, q, bk, bv, scale, hq, rotate=False)
    # scalar loops
    for bb in range(b):
        for h in range(hq):
            s = [scale * sum(float(q[bb, h, i]) * float(zk[bb, j, h, i])
                             for i in range(d)) for j in range(t)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            tot = sum(e)
            for i in range(d):
                o = sum(e[j] * float(zv[bb, j, h * d + i]) for j in range(t)) / tot
                assert abs(o - out[bb, h, i]) <= 1e-12
    # torch SDPA in float64 on the CPU
    qt = torch.tensor(q, dtype=torch.float64)[:, :, None, :]
    kt = torch.tensor(np.transpose(zk, (0, 2, 1, 3)), dtype=torch.float64)
    vt = torch.tensor(zv.reshape(b, t, hq, d).transpose(0, 2, 1, 3).copy(),
                      dtype=torch.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    assert np.allclose(out, ref[:, :, 0].numpy(), atol=1e-12, rtol=0)


@pytest.mark.parametrize("b,hq,hkv,d,rk,rv,t", [
    (1, 1, 1, 4, 2, 3, 1), (2, 2, 1, 8, 4, 4, 2), (1, 4, 2, 6, 3, 5, 3),
    (2, 4, 4, 8, 4, 4, 5), (1, 2, 2, 5, 4, 2, 33)])
def test_brute_force_tiny(b, hq, hkv, d, rk, rv, t):
    rng = np.random.default_rng(t * 10 + hq)
    c, zk, zv = _f32_cache(b, hkv, rk, rv, t, rng)
    bk = rng.standard_normal((hkv, d, rk))
    bv = rng.standard_normal((hkv * d, rv))
    q = rng.standard_normal((b, hq, d))
    out = oa.decode(c, t, q, bk, bv, 0.37, hq, rotate=False)
    g = hq // hkv
    for bb in range(b):
        for h in range(hq):
            kv = h // g
            keys = [[sum(float(zk[bb, j, kv, r]) * bk[kv, i, r] for r in range(rk))
                     for i in range(d)] for j in range(t)]
            vals = [[sum(float(zv[bb, j, r]) * bv[kv * d + i, r] for r in range(rv))
                     for i in range(d)] for j in range(t)]
            s = [0.37 * sum(q[bb, h, i] * keys[j][i] for i in range(d))
                 for j in range(t)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            for i in range(d):
                o = sum(e[j] * vals[j][i] for j in range(t)) / sum(e)
                assert abs(o - out[bb, h, i]) <= 1e-12 * max(1, abs(o))


def test_latent_space_reassociation_eq2_eq12():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((50, 32))
    u = rng.standard_normal((128, 32))
    q = rng.standard_normal(128)
    assert np.allclose(q @ (z @ u.T).T, (q @ u) @ z.T, atol=1e-12)
    p = rng.random((32, 50))
    zv = rng.standard_normal((50, 1024))
    uv = rng.standard_normal((128, 1024))
    assert np.allclose((p @ zv) @ uv.T, p @ (zv @ uv.T), atol=1e-10)


def test_split_merge_decomposition_theorem():
    rng = np.random.default_rng(5)
    b, hq, hkv, d, rk, rv, t = 1, 4, 2, 8, 4, 6, 101
    c, _, _ = _f32_cache(b, hkv, rk, rv, t, rng)
    bk = rng.standard_normal((hkv, d, rk))
    bv = rng.standard_normal((hkv * d, rv))
    q = rng.standard_normal((b, hq, d)) * 3
    full = oa.decode(c, t, q, bk, bv, 0.5, hq, rotate=False)
    for cuts in ([0, 101], [0, 0, 101], [0, 1, 2, 101], [0, 50, 50, 100, 101],
                 sorted([0, 101] + list(rng.integers(0, 101, 6)))):
        for h in range(hq):
            parts = [oa.decode_partial(c, 0, h, cuts[i], cuts[i + 1], q, bk, bv,
                                       0.5, hq) for i in range(len(cuts) - 1)]
            assert np.allclose(oa.merge_partials(parts), full[0, h], atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(6)
    b, hq, hkv, d, rk, rv, t = 2, 8, 2, 8, 4, 12, 40
    c, zk, zv = _f32_cache(b, hkv, rk, rv, t, rng)
    bk = rng.standard_normal((hkv, d, rk))
    bv = rng.standard_normal((hkv * d, rv))
    q = rng.standard_normal((b, hq, d))
    gqa = oa.decode(c, t, q, bk, bv, 0.3, hq, rotate=False)
    g = hq // hkv
    c2 = oc.Cache(b, hq, rk, rv, 64, "f32")
    c2.append(np.repeat(zk, g, axis=2), zv, 0, t)
    bk2 = np.repeat(bk, g, axis=0)
    bv2 = np.concatenate([bv[(h // g) * d:(h // g + 1) * d] for h in range(hq)])
    mha = oa.decode(c2, t, q, bk2, bv2, 0.3, hq, rotate=False)
    assert np.allclose(gqa, mha, atol=1e-12)
    # duplicated query heads give identical rows
    q[:, 1] = q[:, 0]
    out = oa.decode(c, t, q, bk, bv, 0.3, hq, rotate=False)
    assert np.array_equal(out[:, 0], out[:, 1])


def test_token_permutation_invariance():
    rng = np.random.default_rng(7)
    b, h, d, rk, rv, t = 1, 2, 8, 4, 6, 70
    c, zk, zv = _f32_cache(b, h, rk, rv, t, rng)
    perm = rng.permutation(t)
    c2 = oc.Cache(b, h, rk, rv, 128, "f32")
    c2.append(zk[:, perm], zv[:, perm], 0, t)
    bk = rng.standard_normal((h, d, rk))
    bv = rng.standard_normal((h * d, rv))
    q = rng.standard_normal((b, h, d))
    assert np.allclose(oa.decode(c, t, q, bk, bv, 1.0, h, False),
                       oa.decode(c2, t, q, bk, bv, 1.0, h, False), atol=1e-12)


def test_prefill_rows_equal_decode_and_are_causal():
    w = synth.WORKLOADS["longchat_prefill"].replace(
        n_q_heads=4, n_kv_heads=4, value_rank=256, hidden=64, seq_len=70,
        chunk=40)
    x, ak, av, q = synth.prefill_inputs(w)
    bk, bv = synth.factors(w)
    scale = 1 / math.sqrt(w.head_dim)

    def fresh():
        c = oc.Cache.for_workload(w)
        zk, zv = synth.batch_latents(w, 0, w.seq_len)
        c.append(zk, zv, 0, w.seq_len)
        return c

    c = fresh()
    rows = [0, 1, 17, 39]
    out = oa.prefill(c, w.seq_len, x, ak, av, q, bk, bv, scale, 4, True, rows=rows)
    for ri, i in enumerate(rows):
        dec = oa.decode(c, w.seq_len + i + 1, q[i][None], bk, bv, scale, 4, True)
        assert np.allclose(out[ri], dec[0], atol=1e-12)
    # causality: changing the chunk's later tokens leaves row 17 unchanged
    x2 = x.copy()
    x2[30:] = synth.round_to_bf16(x2[30:] * 3 + 1)
    c2 = fresh()
    out2 = oa.prefill(c2, w.seq_len, x2, ak, av, q, bk, bv, scale, 4, True,
                      rows=[17])
    assert np.allclose(out2[0], out[2], atol=1e-14, rtol=1e-12)


def test_quantized_rotated_cache_is_close_to_exact_latents():
    w = synth.WORKLOADS["l2_q43"].replace(batch=1, seq_len=256, n_q_heads=8,
                                          n_kv_heads=8, value_rank=256)
    zk, zv = synth.batch_latents(w, 0, 256)
    bk, bv = synth.factors(w)
    q = synth.queries(w) * 8
    scale = 1 / math.sqrt(w.head_dim)
    cq = oc.Cache.for_workload(w)
    cq.append(zk, zv, 0, 256)
    exact = oc.Cache(1, 8, 32, 256, 256, "f32")
    exact.append(zk, zv, 0, 256)
    oq_ = oa.decode(cq, 256, q, bk, bv, scale, 8, rotate=True)
    oe = oa.decode(exact, 256, q, bk, bv, scale, 8, rotate=False)
    rel = np.abs(oq_ - oe).max() / np.abs(oe).max()
    # 3-bit noise does not average away relative to an output that is itself
    # an average of near-independent value vectors: about 13 % here
    assert rel < 0.25
    # a wrong rotation (reconstructing without H) is far off
    bad = oa.decode(cq, 256, q, bk, bv, scale, 8, rotate=False)
    assert np.abs(bad - oe).max() / np.abs(oe).max() > 0.8
