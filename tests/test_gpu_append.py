"""GPU append (quantize + pack) is bit-exact with the oracle packer.

Both caches start from the same random bytes, so every bit that an append must
leave alone is checked too.  Step sizes cover a first fill, single-token
decode appends, a range that crosses a tile boundary, and a range that ends at
capacity.
"""

import numpy as np
import pytest

import synth
from oracle import cache as oc

from helpers import append_both, config_for, fill_random, gpu_bytes, sk

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny", dict(batch=2)),
    ("l2_bf16", dict(batch=2, n_q_heads=8, n_kv_heads=8)),
    ("l2_q43", dict(batch=2)),
    ("l2_q43", dict(batch=2, rotate=False)),
    ("l3_gqa_q43", dict(batch=3)),
    ("l2_q4", dict(batch=2)),
    ("l2_q4", dict(batch=2, rotate=False, value_rank=256)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(CASES)])
def test_append_bit_exact(name, kw):
    w = synth.WORKLOADS[name].replace(**kw)
    T = 256
    cfg = config_for(w, max_tokens=T)
    g = sk().LatentCache(cfg)
    o = oc.Cache.for_workload(w, max_tokens=T)
    fill_random(g, o, seed=11)
    for pos, n in [(0, 150), (150, 1), (151, 1), (152, 37), (189, 67)]:
        print(f"append {name} {kw} pos={pos} n={n}", flush=True)
        append_both(w, cfg, g, o, pos, n, w.batch)
        got = gpu_bytes(g, o)
        for key, ref in o.buf.items():
            if ref.size:
                bad = np.nonzero(got[key] != ref)[0]
                assert bad.size == 0, (key, pos, n, bad[:10])


def test_append_large_chunk_bit_exact():
    """A prefill-sized append (many whole tiles) of the metric layout."""
    w = synth.WORKLOADS["l2_q43"].replace(batch=1)
    T = 4096
    cfg = config_for(w, max_tokens=T)
    g = sk().LatentCache(cfg)
    o = oc.Cache.for_workload(w, max_tokens=T)
    fill_random(g, o, seed=12)
    append_both(w, cfg, g, o, 33, T - 33, 1)
    got = gpu_bytes(g, o)
    for key, ref in o.buf.items():
        assert np.array_equal(got[key], ref), key
