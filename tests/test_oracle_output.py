"""Pins for the oracle's value/output factor fusion and head sum (CPU).

Technical review of arXiv 2606.08382, section 5.3, eq. 12:
p_h (Z_V U_h^T) O_h = (p_h Z_V)(U_h^T O_h), the right-hand factor prepared
offline; Algorithm 2, steps 7-8 (apply the head-specific value/output
factors, sum the heads).  Pinned by scalar loops, one hand-placed element
(catches a transposed factor or a wrong query-to-KV-head map), the eq. 12
identity between the two association orders (through independent oracle
paths: per-head outputs times O_h vs latent rows times the fused factor,
also for a rotated 4/3-bit cache, eq. 13), and the head sum with an
identity output projection.
"""

import math

import numpy as np
import pytest

import synth
from oracle import attention as oa
from oracle import cache as oc


def test_fuse_value_output_scalar_loops():
    rng = np.random.default_rng(1)
    hq, hkv, d, rv, D = 4, 2, 3, 5, 6
    bv = rng.standard_normal((hkv * d, rv))
    w_o = rng.standard_normal((hq * d, D))
    F = oa.fuse_value_output(bv, w_o, hq, hkv, d)
    assert F.shape == (hq, rv, D)
    for h in range(hq):
        g = h // (hq // hkv)
        for r in range(rv):
            for n in range(D):
                want = sum(bv[g * d + i, r] * w_o[h * d + i, n] for i in range(d))
                assert abs(F[h, r, n] - want) <= 1e-12


def test_fuse_value_output_hand_placed_element():
    hq, hkv, d, rv, D = 4, 2, 3, 5, 6
    bv = np.zeros((hkv * d, rv))
    bv[1 * d + 2, 3] = 1.0            # KV head 1, value dim 2, latent channel 3
    w_o = np.zeros((hq * d, D))
    w_o[2 * d + 2, 4] = 5.0           # query head 2 (KV head 1), dim 2 -> hidden 4
    F = oa.fuse_value_output(bv, w_o, hq, hkv, d)
    want = np.zeros((hq, rv, D))
    want[2, 3, 4] = 5.0
    assert np.array_equal(F, want)


def _f32_cache(rng, b, hkv, rk, rv, t):
    c = oc.Cache(b, hkv, rk, rv, ((t + 63) // 64) * 64, "f32")
    c.append(rng.standard_normal((b, t, hkv, rk)).astype(np.float32),
             rng.standard_normal((b, t, rv)).astype(np.float32), 0, t)
    return c


def test_eq12_association_orders_agree_unquantized():
    rng = np.random.default_rng(2)
    b, hq, hkv, d, rk, rv, t, D = 2, 4, 2, 8, 4, 12, 50, 10
    c = _f32_cache(rng, b, hkv, rk, rv, t)
    bk = rng.standard_normal((hkv, d, rk))
    bv = rng.standard_normal((hkv * d, rv))
    w_o = rng.standard_normal((hq * d, D))
    q = rng.standard_normal((b, hq, d))
    y = oa.decode_hidden(c, t, q, bk, bv, w_o, 0.4, hq, rotate=False)
    rows = oa.decode_latent_rows(c, t, q, bk, 0.4, hq, rotate=False)
    F = oa.fuse_value_output(bv, w_o, hq, hkv, d)
    y2 = np.einsum("bhr,hrn->bn", rows, F)
    assert np.allclose(y, y2, atol=1e-12)


def test_eq12_association_orders_agree_rotated_q43():
    w = synth.WORKLOADS["l2_q43"].replace(batch=1, n_q_heads=8, n_kv_heads=4,
                                          value_rank=256, head_dim=64)
    zk, zv = synth.batch_latents(w, 0, 130)
    c = oc.Cache.for_workload(w, max_tokens=192)
    c.append(zk, zv, 0, 130)
    bk, bv = synth.factors(w)
    rng = np.random.default_rng(3)
    w_o = rng.standard_normal((w.n_q_heads * w.head_dim, 256))
    q = synth.queries(w) * 4
    s = 1 / math.sqrt(w.head_dim)
    y = oa.decode_hidden(c, 130, q, bk, bv, w_o, s, w.n_q_heads, rotate=True)
    # rows in the stored (rotated) latent need the fused factor of the
    # rotated value factor B_value H (eq. 13) ...
    rows = oa.decode_latent_rows(c, 130, q, bk, s, w.n_q_heads, rotate=True)
    _, bv_e = oa.effective_factors(bk, bv, True, w.key_rank, w.value_rank)
    F_rot = oa.fuse_value_output(bv_e, w_o, w.n_q_heads, w.n_kv_heads, w.head_dim)
    assert np.allclose(y, np.einsum("bhr,hrn->bn", rows, F_rot), atol=1e-12)
    # ... and unrotated rows the plain fused factor
    rows_u = oa.decode_latent_rows(c, 130, q, bk, s, w.n_q_heads, rotate=True,
                                   unrotated=True)
    F = oa.fuse_value_output(bv, w_o, w.n_q_heads, w.n_kv_heads, w.head_dim)
    assert np.allclose(y, np.einsum("bhr,hrn->bn", rows_u, F), atol=1e-12)
    # a fused factor built without the rotation is far off
    bad = np.einsum("bhr,hrn->bn", rows, F)
    assert np.abs(bad - y).max() > 0.3 * np.abs(y).max()


def test_head_sum_with_identity_output_projection():
    rng = np.random.default_rng(4)
    b, hq, hkv, d, rk, rv, t = 2, 4, 4, 5, 3, 7, 20
    c = _f32_cache(rng, b, hkv, rk, rv, t)
    bk = rng.standard_normal((hkv, d, rk))
    bv = rng.standard_normal((hkv * d, rv))
    q = rng.standard_normal((b, hq, d))
    o = oa.decode(c, t, q, bk, bv, 0.3, hq, rotate=False)
    y = oa.decode_hidden(c, t, q, bk, bv, np.eye(hq * d), 0.3, hq, rotate=False)
    assert np.allclose(y, o.reshape(b, hq * d), atol=1e-14)
