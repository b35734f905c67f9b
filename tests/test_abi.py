"""The C ABI on the CPU: the library loads, exports every entry point the
header declares, reports sizes that match the oracle's format, and rejects bad
arguments on the host before any HIP call (no compute call needs a GPU here).
"""

import ctypes
import os
import re

import numpy as np
import pytest

import synth
from oracle import cache as oc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "starkv.h")

sk = pytest.importorskip("decode_attention_starkv_amd")
if not os.path.exists(sk.LIB_PATH):
    pytest.skip("libstarkv.so not built", allow_module_level=True)


def _cfg(w, **kw):
    base = dict(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                head_dim=w.head_dim, key_rank=w.key_rank,
                value_rank=w.value_rank, max_tokens=w.max_tokens,
                cache_dtype=w.cache, rotate=w.rotate)
    base.update(kw)
    if base["cache_dtype"] == "q43" and "lo_bits" not in kw:
        base["lo_bits"] = w.lo_bits
    return sk.make_config(**base)


def test_every_declared_entry_point_is_exported():
    declared = re.findall(r"STARKV_API\s+[\w\s\*]+?\b(starkv_\w+)\s*\(",
                          open(HEADER).read())
    assert set(declared) == set(sk.ENTRY_POINTS)
    lib = sk.load_library()
    for name in declared:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_cache_bytes_match_oracle_layout(name):
    w = synth.WORKLOADS[name]
    cfg = _cfg(w)
    lay = oc.layout(w.batch, w.n_kv_heads, w.key_rank, w.value_rank,
                    w.max_tokens, w.cache, lo_bits=w.lo_bits)
    got = [sk.starkv_cache_bytes(cfg, i) for i in range(4)]
    assert got == [lay["key"], lay["key_meta"], lay["value"], lay["value_meta"]]


def test_metric_cache_is_1216_bytes_per_token():
    w = synth.WORKLOADS["l2_q43"]
    cfg = _cfg(w)
    total = sum(sk.starkv_cache_bytes(cfg, i) for i in range(4))
    assert total == w.batch * w.max_tokens * 1216


def test_workspace_and_splits():
    w = synth.WORKLOADS["l2_q43"]
    cfg = _cfg(w)
    s = sk.starkv_decode_splits(cfg, w.seq_len)
    assert s == 16                      # 16 sequences x 16 splits = 256 groups
    ws = sk.starkv_workspace_bytes(cfg, sk.OP_DECODE, w.seq_len)
    assert ws >= w.batch * s * w.n_q_heads * w.value_rank * 2   # fp16 rows
    assert sk.starkv_decode_splits(_cfg(w, num_splits=5), w.seq_len) == 5
    assert sk.starkv_decode_splits(cfg, 1) == 1
    assert sk.starkv_decode_splits(cfg, 65) == 2
    # a split never ends up empty
    for t in (64, 100, 1000, 4097):
        s = sk.starkv_decode_splits(cfg, t)
        tiles = (t + 63) // 64
        tps = -(-tiles // s)
        assert (s - 1) * tps < tiles


def test_strerror():
    assert sk.starkv_strerror(0) == "success"
    assert "capacity" in sk.starkv_strerror(sk.STARKV_ECAPACITY)
    assert sk.starkv_strerror(-99) == "unknown status"


def _fake_cache():
    return sk.StarkvCache(0x10000, 0x20000, 0x30000, 0x40000)


def test_config_validation_codes():
    w = synth.WORKLOADS["l2_q43"]
    lib = sk.load_library()
    assert lib.starkv_cache_bytes(None, 0) == 0
    bad = [
        (dict(batch=0), sk.STARKV_EINVAL),
        (dict(n_kv_heads=3), sk.STARKV_EINVAL),          # 32 % 3 != 0
        (dict(max_tokens=100), sk.STARKV_EINVAL),        # not a multiple of 64
        (dict(cache_dtype=7), sk.STARKV_EINVAL),
        (dict(n_q_heads=64, n_kv_heads=64), sk.STARKV_EUNSUPPORTED),
        (dict(n_kv_heads=2), sk.STARKV_EUNSUPPORTED),    # group of 16
        (dict(key_rank=16), sk.STARKV_EUNSUPPORTED),     # q43 needs 32
        (dict(value_rank=1056), sk.STARKV_EUNSUPPORTED),
        (dict(head_dim=100), sk.STARKV_EUNSUPPORTED),
        (dict(cache_dtype="bf16", rotate=True), sk.STARKV_EUNSUPPORTED),
        # the precision split of the quantized cache (review section 6.1,
        # eq. 14): fields out of range are invalid, other splits unsupported
        (dict(hi_bits=0), sk.STARKV_EINVAL),
        (dict(lo_bits=9), sk.STARKV_EINVAL),
        (dict(group_size=0), sk.STARKV_EINVAL),
        (dict(key_hi_channels=33), sk.STARKV_EINVAL),
        (dict(value_hi_channels=-1), sk.STARKV_EINVAL),
        (dict(hi_bits=8), sk.STARKV_EUNSUPPORTED),
        (dict(lo_bits=2), sk.STARKV_EUNSUPPORTED),
        (dict(group_size=16), sk.STARKV_EUNSUPPORTED),
        (dict(key_hi_channels=6), sk.STARKV_EUNSUPPORTED),     # a 20:80 split
        (dict(value_hi_channels=204), sk.STARKV_EUNSUPPORTED),
        # unquantized caches have no precision split
        (dict(cache_dtype="bf16", rotate=False, hi_bits=4), sk.STARKV_EINVAL),
        (dict(cache_dtype="bf16", rotate=False, group_size=32), sk.STARKV_EINVAL),
        (dict(rope_theta=-1.0), sk.STARKV_EINVAL),
        (dict(rope_theta=float("nan")), sk.STARKV_EINVAL),
        (dict(rope_theta=float("inf")), sk.STARKV_EINVAL),
        (dict(cache_dtype="bf16", rotate=False, key_ranks=[7] * 32), sk.STARKV_EINVAL),
        (dict(cache_dtype="bf16", rotate=False, key_ranks=[40] * 32), sk.STARKV_EINVAL),
    ]
    cache = _fake_cache()
    for kw, code in bad:
        cfg = _cfg(w, **kw)
        assert sk.starkv_cache_bytes(cfg, 0) == 0, kw
        st = lib.starkv_append(ctypes.byref(cfg), ctypes.byref(cache),
                               0x1000, 0x2000, 0, 1, None)
        assert st == code, (kw, st)


def test_default_layout_fields_are_the_quarter_split():
    w = synth.WORKLOADS["l2_q43"]
    cfg = _cfg(w)
    assert (cfg.hi_bits, cfg.lo_bits, cfg.group_size, cfg.key_hi_channels,
            cfg.value_hi_channels) == (4, 3, 32, 8, 256)
    plain = _cfg(synth.WORKLOADS["l2_bf16"])
    assert (plain.hi_bits, plain.lo_bits, plain.group_size,
            plain.key_hi_channels, plain.value_hi_channels) == (0, 0, 0, 0, 0)
    assert ctypes.sizeof(sk.StarkvConfig) == 72


def test_uniform_4bit_support():
    """Both precision blocks at 4 bits (the 4-bit cache of the review's speed
    figures, section 6.1): accepted for decode (latent and rotary scores) and
    prefill, 1024 key bytes per tile-head and 32 value bytes per channel and
    tile."""
    lib = sk.load_library()
    w = synth.WORKLOADS["l2_q4"]
    cfg = _cfg(w)
    assert cfg.lo_bits == 4
    nt = w.max_tokens // 64
    assert sk.starkv_cache_bytes(cfg, 0) == w.batch * w.n_kv_heads * nt * 1024
    assert sk.starkv_cache_bytes(cfg, 2) == w.batch * nt * 32 * w.value_rank
    # per token: 32 heads x (16 B codes + 8 B meta) keys, 512 B codes +
    # 128 B meta values
    total = sum(sk.starkv_cache_bytes(cfg, i) for i in range(4))
    assert total == w.batch * w.max_tokens * 1408
    assert sk.starkv_decode_splits(cfg, w.seq_len) > 0
    assert sk.starkv_workspace_bytes(cfg, sk.OP_DECODE, w.seq_len) > 0
    rope = _cfg(w, rope_theta=10000.0)
    assert sk.starkv_workspace_bytes(rope, sk.OP_DECODE, w.seq_len) > 0
    for hq, hkv, rv in ((32, 8, 256), (16, 2, 512), (16, 4, 768), (8, 8, 1024)):
        c = _cfg(w, n_q_heads=hq, n_kv_heads=hkv, value_rank=rv)
        assert sk.starkv_decode_splits(c, 1000) > 0, (hq, hkv, rv)
    # the prefill reads both layouts, with or without rotary keys; rotary
    # keys of d_h 256 are refused before any HIP call
    small = _cfg(w, max_tokens=256)
    assert sk.starkv_workspace_bytes(small, sk.OP_PREFILL, 64) > 0
    assert sk.starkv_workspace_bytes(_cfg(w, max_tokens=256, rope_theta=1e4),
                                     sk.OP_PREFILL, 64) > 0
    wide = _cfg(w, max_tokens=256, head_dim=256, rope_theta=1e4)
    assert sk.starkv_workspace_bytes(wide, sk.OP_PREFILL, 64) == 0
    cache = _fake_cache()
    st = lib.starkv_prefill(ctypes.byref(wide),
                            ctypes.byref(cache), 0, 64, 0x1000, 4096, 0x2000, 0x3000,
                            0x4000, 0x5000, 0x6000, ctypes.c_float(0.1), 0x7000, None,
                            0x8000, 1 << 30, None)
    assert st == sk.STARKV_EUNSUPPORTED
    # other trailing widths stay unsupported
    assert sk.starkv_cache_bytes(_cfg(w, lo_bits=2), 0) == 0
    assert sk.starkv_cache_bytes(_cfg(w, lo_bits=5), 0) == 0


def test_q43_shape_without_decode_kernel_is_rejected_before_launch():
    """Twelve KV heads (three per score wave) have no decode kernel: the
    cache and its append are fine, decode says so before any HIP call."""
    lib = sk.load_library()
    w = synth.WORKLOADS["l2_q43"]
    for hq, hkv in ((12, 12), (24, 12), (20, 20), (28, 28)):
        cfg = _cfg(w, n_q_heads=hq, n_kv_heads=hkv)
        assert sk.starkv_cache_bytes(cfg, 0) > 0
        assert sk.starkv_decode_splits(cfg, 1000) == 0
        assert sk.starkv_workspace_bytes(cfg, sk.OP_DECODE, 1000) == 0
        cache = _fake_cache()
        st = lib.starkv_decode(ctypes.byref(cfg), ctypes.byref(cache), 100, 0x1000,
                               0x2000, 0x3000, ctypes.c_float(0.1), 0x4000,
                               0x5000, 1 << 30, None)
        assert st == sk.STARKV_EUNSUPPORTED, (hq, hkv, st)


def test_noalloc_rejects_shapes_beyond_its_scratch_before_any_hip_call():
    lib = sk.load_library()
    assert sk.starkv_noalloc_scratch_bytes() == 64 << 20
    w = synth.WORKLOADS["l2_q43"]
    big = _cfg(w, batch=512, max_tokens=4096)
    assert sk.starkv_workspace_bytes(big, sk.OP_DECODE, 4096) > 64 << 20
    cache = _fake_cache()
    args = (0x1000, 0x2000, 0x3000, ctypes.c_float(0.1), 0x4000, None)
    assert lib.starkv_decode_noalloc(ctypes.byref(big), ctypes.byref(cache), 4096,
                                     *args) == sk.STARKV_EWORKSPACE
    cfg = _cfg(w)
    assert lib.starkv_decode_noalloc(ctypes.byref(cfg), ctypes.byref(cache), 0,
                                     *args) == sk.STARKV_EINVAL
    assert lib.starkv_decode_noalloc(ctypes.byref(cfg), ctypes.byref(cache),
                                     w.max_tokens + 1, *args) == sk.STARKV_ECAPACITY
    assert lib.starkv_decode_noalloc(ctypes.byref(cfg), ctypes.byref(cache), 100,
                                     None, 0x2000, 0x3000, ctypes.c_float(0.1), 0x4000,
                                     None) == sk.STARKV_EINVAL
    # the metric shape fits
    assert sk.starkv_workspace_bytes(cfg, sk.OP_DECODE, w.seq_len) <= 64 << 20


def test_decode_step_validation_before_any_hip_call():
    lib = sk.load_library()
    w = synth.WORKLOADS["l2_q43"]
    cfg = _cfg(w)
    cp, cc = ctypes.byref(cfg), ctypes.byref(_fake_cache())
    tail = (0x3000, 0x4000, 0x5000, ctypes.c_float(0.1), 0x6000, 0x7000, 1 << 30, None)
    step = lambda zk, zv, pos, n, *t: lib.starkv_decode_step(cp, cc, zk, zv, pos, n, *t)
    assert step(0x1000, 0x2000, -1, 1, *tail) == sk.STARKV_EINVAL
    assert step(0x1000, 0x2000, 5, -1, *tail) == sk.STARKV_EINVAL
    assert step(0x1000, 0x2000, w.max_tokens, 1, *tail) == sk.STARKV_ECAPACITY
    assert step(0x1000, 0x2000, 0, 0, *tail) == sk.STARKV_EINVAL          # seq_len 0
    assert step(None, 0x2000, 5, 1, *tail) == sk.STARKV_EINVAL
    assert step(0x1004, 0x2000, 5, 1, *tail) == sk.STARKV_EINVAL
    small = tail[:6] + (16, None)
    assert step(0x1000, 0x2000, 5, 1, *small) == sk.STARKV_EWORKSPACE
    assert lib.starkv_decode_step_profiled(cp, cc, 0x1000, 0x2000, 5, 1, *tail,
                                           None) == sk.STARKV_EINVAL


def test_hidden_decode_validation():
    lib = sk.load_library()
    w = synth.WORKLOADS["l2_q43"]
    cfg = _cfg(w)
    assert sk.starkv_fused_factor_bytes(cfg, 4096) == 32 * 1024 * 4096 * 2
    assert sk.starkv_fused_factor_bytes(cfg, 100) == 0            # not a multiple of 128
    assert sk.starkv_fused_factor_bytes(_cfg(synth.WORKLOADS["tiny"]), 256) == 0   # fp32
    assert sk.starkv_decode_hidden_workspace_bytes(cfg, 1000, 4096) > \
        sk.starkv_workspace_bytes(cfg, sk.OP_DECODE, 1000)
    cp, cc = ctypes.byref(cfg), ctypes.byref(_fake_cache())
    assert lib.starkv_fuse_value_output(cp, 0x1000, 0x2000, 0, 0x3000, None) == sk.STARKV_EINVAL
    assert lib.starkv_fuse_value_output(cp, 0x1000, 0x2000, 100, 0x3000, None) == \
        sk.STARKV_EUNSUPPORTED
    assert lib.starkv_fuse_value_output(cp, None, 0x2000, 256, 0x3000, None) == sk.STARKV_EINVAL
    args = (0x1000, 0x2000, 0x3000, 256, ctypes.c_float(0.1), 0x4000)
    assert lib.starkv_decode_hidden(cp, cc, 100, *args, 0x5000, 16, None) == sk.STARKV_EWORKSPACE
    assert lib.starkv_decode_hidden(cp, cc, 0, *args, 0x5000, 1 << 30, None) == sk.STARKV_EINVAL
    bad = (0x1000, 0x2000, 0x3000, 200, ctypes.c_float(0.1), 0x4000)
    assert lib.starkv_decode_hidden(cp, cc, 100, *bad, 0x5000, 1 << 30, None) == \
        sk.STARKV_EUNSUPPORTED


def test_rope_support_and_workspace():
    lib = sk.load_library()
    w = synth.WORKLOADS["l2_q43"]
    plain = _cfg(w)
    rope = _cfg(w, rope_theta=10000.0)
    assert sk.starkv_cache_bytes(rope, 0) == sk.starkv_cache_bytes(plain, 0)
    # the rotary scores need their own workspace on top of decode's
    assert sk.starkv_workspace_bytes(rope, sk.OP_DECODE, 4096) > \
        sk.starkv_workspace_bytes(plain, sk.OP_DECODE, 4096)
    assert sk.starkv_decode_splits(rope, 4096) > 0
    cache = _fake_cache()
    args = (0x1000, 0x2000, 0x3000, ctypes.c_float(0.1), 0x4000, 0x5000, 1 << 30, None)
    for cfg in (_cfg(synth.WORKLOADS["l2_bf16"], rope_theta=10000.0),   # plain caches
                _cfg(w, head_dim=256, rope_theta=10000.0)):             # head dim 256
        assert lib.starkv_decode(ctypes.byref(cfg), ctypes.byref(cache), 100,
                                 *args) == sk.STARKV_EUNSUPPORTED
    # prefill with rotary keys: the keys are reconstructed at d_h channels
    # (workspace grows by the wider keys and queries); d_h 64 and 128 only
    lc = synth.WORKLOADS["longchat_prefill"]
    pre = _cfg(lc, rope_theta=10000.0)
    assert sk.starkv_workspace_bytes(pre, sk.OP_PREFILL, 4096) > \
        sk.starkv_workspace_bytes(_cfg(lc), sk.OP_PREFILL, 4096)
    assert sk.starkv_workspace_bytes(_cfg(lc, head_dim=64, rope_theta=10000.0),
                                     sk.OP_PREFILL, 4096) > 0
    wide = _cfg(lc, head_dim=256, rope_theta=10000.0)
    assert sk.starkv_workspace_bytes(wide, sk.OP_PREFILL, 4096) == 0
    pargs = (0x1000, 4096, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000,
             ctypes.c_float(0.1), 0x7000, None)
    assert lib.starkv_prefill(ctypes.byref(wide), ctypes.byref(cache), 0, 64, *pargs,
                              0x8000, 1 << 34, None) == sk.STARKV_EUNSUPPORTED


def test_paged_validation():
    lib = sk.load_library()
    w = synth.WORKLOADS["l2_q43"]
    cfg = _cfg(w)
    cp, cc = ctypes.byref(cfg), ctypes.byref(_fake_cache())
    # append: table / positions / latents required, one page at least
    assert lib.starkv_append_paged(cp, cc, None, 4, 0x100, 0x1000, 0x2000, None) == sk.STARKV_EINVAL
    assert lib.starkv_append_paged(cp, cc, 0x100, 0, 0x200, 0x1000, 0x2000, None) == sk.STARKV_EINVAL
    assert lib.starkv_append_paged(cp, cc, 0x102, 4, 0x200, 0x1000, 0x2000, None) == sk.STARKV_EINVAL
    bf = _cfg(synth.WORKLOADS["l2_bf16"])
    assert lib.starkv_append_paged(ctypes.byref(bf), cc, 0x100, 4, 0x200, 0x1000, 0x2000,
                                   None) == sk.STARKV_EUNSUPPORTED
    tail = (0x1000, 0x2000, 0x3000, ctypes.c_float(0.1), 0x4000, 0x5000, 1 << 30, None)
    # decode: the pages must cover max_seq_len; max_seq_len within capacity
    assert lib.starkv_decode_paged(cp, cc, 0x100, 4, 0x200, 257, *tail) == sk.STARKV_EINVAL
    assert lib.starkv_decode_paged(cp, cc, 0x100, 4096, 0x200, w.max_tokens + 1,
                                   *tail) == sk.STARKV_ECAPACITY
    assert lib.starkv_decode_paged(cp, cc, None, 4, 0x200, 100, *tail) == sk.STARKV_EINVAL
    assert lib.starkv_decode_paged(cp, cc, 0x100, 4, None, 100, *tail) == sk.STARKV_EINVAL
    short = tail[:6] + (16, None)
    assert lib.starkv_decode_paged(cp, cc, 0x100, 4, 0x200, 100, *short) == sk.STARKV_EWORKSPACE
    # prefill: a table is required, its pages must cover ctx_len + chunk,
    # rotary keys of d_h 256 are refused; all before any HIP call
    pre = (0x1000, 4096, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, ctypes.c_float(0.1),
           0x7000, None, 0x8000, 1 << 40, None)
    assert lib.starkv_prefill_paged(cp, cc, None, 8, 0, 64, *pre) == sk.STARKV_EINVAL
    assert lib.starkv_prefill_paged(cp, cc, 0x100, 2, 100, 64, *pre) == sk.STARKV_EINVAL
    assert lib.starkv_prefill_paged(cp, cc, 0x102, 8, 100, 64, *pre) == sk.STARKV_EINVAL
    rope = _cfg(w, head_dim=256, rope_theta=1e4)
    assert lib.starkv_prefill_paged(ctypes.byref(rope), cc, 0x100, 8, 100, 64,
                                    *pre) == sk.STARKV_EUNSUPPORTED
    assert lib.starkv_prefill_paged(cp, cc, 0x100, 8, 100, 64,
                                    *(pre[:11] + (16, None))) == sk.STARKV_EWORKSPACE


def test_per_head_key_ranks_cache_bytes():
    w = synth.WORKLOADS["l2_bf16"]
    ranks = [8, 64, 24, 40] * 8
    cfg = _cfg(w, key_rank=64, key_ranks=ranks)
    lay = oc.layout(w.batch, w.n_kv_heads, 64, w.value_rank, w.max_tokens, "bf16",
                    key_ranks=ranks)
    assert sk.starkv_cache_bytes(cfg, sk.BUF_KEY) == lay["key"] == \
        w.batch * w.max_tokens * sum(ranks) * 2
    assert sk.starkv_decode_splits(cfg, 1000) > 0
    # quantized caches keep every head's 32-channel key tile (section 6.2:
    # rank rounding to a supported kernel tile, eq. 15's padding term)
    qw = synth.WORKLOADS["l2_q43"]
    plain = _cfg(qw)
    for lob in (3, 4):
        q = _cfg(qw, key_ranks=[8, 16, 24, 32] * 8, lo_bits=lob)
        for i in range(4):
            assert sk.starkv_cache_bytes(q, i) == sk.starkv_cache_bytes(
                _cfg(qw, lo_bits=lob), i) > 0
        assert sk.starkv_decode_splits(q, 1000) == sk.starkv_decode_splits(plain, 1000)
    # ranks past the tile, or not a multiple of 8, are invalid
    assert sk.starkv_cache_bytes(_cfg(qw, key_ranks=[40] * 32), 0) == 0
    assert sk.starkv_cache_bytes(_cfg(qw, key_ranks=[12] * 32), 0) == 0


def test_call_validation_before_any_hip_call():
    w = synth.WORKLOADS["l2_q43"]
    lib = sk.load_library()
    cfg = _cfg(w)
    cache = _fake_cache()
    cp, cc = ctypes.byref(cfg), ctypes.byref(cache)
    # append: capacity, negative sizes, null / misaligned pointers
    assert lib.starkv_append(cp, cc, 0x1000, 0x2000, w.max_tokens, 1, None) == sk.STARKV_ECAPACITY
    assert lib.starkv_append(cp, cc, 0x1000, 0x2000, -1, 1, None) == sk.STARKV_EINVAL
    assert lib.starkv_append(cp, cc, None, 0x2000, 0, 1, None) == sk.STARKV_EINVAL
    assert lib.starkv_append(cp, cc, 0x1004, 0x2000, 0, 1, None) == sk.STARKV_EINVAL
    assert lib.starkv_append(cp, cc, None, None, 5, 0, None) == sk.STARKV_OK
    nometa = sk.StarkvCache(0x10000, None, 0x30000, None)
    assert lib.starkv_append(cp, ctypes.byref(nometa), 0x1000, 0x2000, 0, 1, None) == sk.STARKV_EINVAL
    # decode: seq_len range, workspace
    args = (0x1000, 0x2000, 0x3000, ctypes.c_float(0.1), 0x4000)
    assert lib.starkv_decode(cp, cc, 0, *args, 0x5000, 1 << 30, None) == sk.STARKV_EINVAL
    assert lib.starkv_decode(cp, cc, w.max_tokens + 1, *args, 0x5000, 1 << 30, None) == sk.STARKV_ECAPACITY
    assert lib.starkv_decode(cp, cc, 100, *args, 0x5000, 16, None) == sk.STARKV_EWORKSPACE
    assert lib.starkv_decode(cp, cc, 100, *args, None, 1 << 30, None) == sk.STARKV_EWORKSPACE
    assert lib.starkv_decode(cp, cc, 100, None, 0x2000, 0x3000, ctypes.c_float(0.1),
                             0x4000, 0x5000, 1 << 30, None) == sk.STARKV_EINVAL
    # prefill: capacity and workspace
    pre = synth.WORKLOADS["longchat_prefill"]
    pcfg = _cfg(pre)
    pp = ctypes.byref(pcfg)
    pargs = (0x1000, 4096, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000,
             ctypes.c_float(0.1), 0x7000, None)
    assert lib.starkv_prefill(pp, cc, pre.max_tokens, 1, *pargs, 0x8000, 1 << 34, None) == sk.STARKV_ECAPACITY
    assert lib.starkv_prefill(pp, cc, 0, 64, *pargs, 0x8000, 0, None) == sk.STARKV_EWORKSPACE
    f32 = _cfg(synth.WORKLOADS["tiny"])
    assert lib.starkv_prefill(ctypes.byref(f32), cc, 0, 64, *pargs, 0x8000, 1 << 34,
                              None) == sk.STARKV_EUNSUPPORTED
    # stream-read measurement helper: alignment, size and sink checked first
    assert lib.starkv_stream_read(0x1004, 1 << 20, 0x2000, None) == sk.STARKV_EINVAL
    assert lib.starkv_stream_read(0x1000, 0, 0x2000, None) == sk.STARKV_EINVAL
    assert lib.starkv_stream_read(0x1000, 100, 0x2000, None) == sk.STARKV_EINVAL
    assert lib.starkv_stream_read(0x1000, 1 << 20, None, None) == sk.STARKV_EINVAL
    assert lib.starkv_stream_read(0x1000, 1 << 20, 0x2002, None) == sk.STARKV_EINVAL
    # head dims that decode takes but the prefill's up-projection tiles do not
    for dh in (96, 160):
        c = _cfg(pre, head_dim=dh)
        assert sk.starkv_cache_bytes(c, 0) > 0
        assert lib.starkv_prefill(ctypes.byref(c), cc, 0, 64, *pargs, 0x8000, 1 << 34,
                                  None) == sk.STARKV_EUNSUPPORTED, dh


def test_prefill_workspace_follows_the_value_order():
    """The prefill's workspace per chunk length follows the value order it
    takes: fp32 partial rows (C Hq R_v 4 bytes) below the reconstruction
    threshold, position-sized value buffers above it (host only)."""
    w = synth.WORKLOADS["longchat_prefill"]
    cfg = _cfg(w)
    thr = w.n_kv_heads * w.head_dim * w.value_rank // (w.n_q_heads * (w.value_rank - w.head_dim))
    below = sk.starkv_workspace_bytes(cfg, sk.OP_PREFILL, thr)        # joint latent
    above = sk.starkv_workspace_bytes(cfg, sk.OP_PREFILL, thr + 1)    # reconstructed
    assert below > 0 and above > 0
    part_rows = w.batch * thr * w.n_q_heads * w.value_rank * 4
    values = w.batch * w.max_tokens * w.n_kv_heads * w.head_dim * 2
    assert below >= part_rows
    assert above >= values
    # the full chunk reconstructs: no C-sized fp32 partial rows
    full = sk.starkv_workspace_bytes(cfg, sk.OP_PREFILL, w.chunk)
    assert full < w.batch * w.chunk * w.n_q_heads * w.value_rank * 4
