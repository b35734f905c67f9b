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
                    w.max_tokens, w.cache)
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
    assert ws >= w.batch * s * w.n_q_heads * w.value_rank * 4
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
    ]
    cache = _fake_cache()
    for kw, code in bad:
        cfg = _cfg(w, **kw)
        assert sk.starkv_cache_bytes(cfg, 0) == 0, kw
        st = lib.starkv_append(ctypes.byref(cfg), ctypes.byref(cache),
                               0x1000, 0x2000, 0, 1, None)
        assert st == code, (kw, st)


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
