"""Seeded synthetic inputs for the latent-KV attention path.

This module is shared by the tests, the bench and the oracle's callers.  It
draws random numbers and rounds them to their storage dtype; it holds none of
the method's arithmetic (no quantization, packing, rotation or attention).

Workload shapes follow the five decode/prefill workloads the STAR-KV pages
measure or describe (technical review of arXiv 2606.08382, section 8.1 and
Appendix Figure 12: LLaMA-2-7B at batch 16; model card of the LongChat-7B
STAR-KV checkpoint: LongChat-7B at 4K/32K context), with the distribution
recipe below:

* factors: random matrices with orthonormal columns (QR of a Gaussian) --
  the U_r of eq. 2 of the review; for the tiny workload they are additionally
  scaled by singular values sigma_i = i^-0.5, while its latents are N(0, 1);
* latents for the LLaMA-shaped workloads: N(0, 1) times a per-channel std that
  decays as i^-0.5 (i is 1-based inside each key head and inside the joint
  value latent), with round(2 %) of the channels (chosen by the seed) scaled
  by 8 -- the ordering by singular value that the review's section 6.1 says
  the latent cache inherits;
* queries: N(0, 1) / sqrt(d_h); prefill hidden states X: N(0, 1);
* everything is rounded to the storage dtype (bf16, or fp32 for the tiny
  workload) before either side sees it.

Every array is a deterministic function of (workload seed, stream id, batch
index, token chunk), so a caller can regenerate one batch element or one token
range without drawing the rest.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

TOKEN_CHUNK = 1024  # latents are drawn in independent chunks of this many tokens


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    key_rank: int
    value_rank: int
    seq_len: int          # cached tokens for decode; context length T0 for prefill
    cache: str            # "f32" | "bf16" | "q43"
    rotate: bool
    seed: int
    factor_sigma: bool = False   # tiny workload: sigma_i = i^-0.5 on the factors
    decaying_latents: bool = True
    hidden: int = 0       # prefill only: D
    chunk: int = 0        # prefill only: C
    lo_bits: int = 3      # q43 caches: bits of the trailing block (4 = uniform 4-bit)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_tokens(self) -> int:
        t = self.seq_len + self.chunk
        return ((t + 63) // 64) * 64

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # Tiny single-layer decode, fp32 latents, no quantization or rotation.
    "tiny": Workload("tiny", batch=1, n_q_heads=4, n_kv_heads=4, head_dim=64,
                     key_rank=16, value_rank=64, seq_len=256, cache="f32",
                     rotate=False, seed=20260100, factor_sigma=True,
                     decaying_latents=False),
    # LLaMA-2-7B-shaped decode with bf16 latents (batch 1, 4 or 16).
    "l2_bf16": Workload("l2_bf16", batch=16, n_q_heads=32, n_kv_heads=32,
                        head_dim=128, key_rank=32, value_rank=1024,
                        seq_len=4096, cache="bf16", rotate=False, seed=20260200),
    # Same shape, Hadamard-rotated 4/3-bit latents, batch 16 at 32K context.
    "l2_q43": Workload("l2_q43", batch=16, n_q_heads=32, n_kv_heads=32,
                       head_dim=128, key_rank=32, value_rank=1024,
                       seq_len=32768, cache="q43", rotate=True, seed=20260300),
    # Same shape with the uniform 4-bit cache of the pages' speed figures.
    "l2_q4": Workload("l2_q4", batch=16, n_q_heads=32, n_kv_heads=32,
                      head_dim=128, key_rank=32, value_rank=1024,
                      seq_len=32768, cache="q43", rotate=True, seed=20260600,
                      lo_bits=4),
    # LLaMA-3-8B-shaped GQA decode: 32 query heads over 8 KV heads.
    "l3_gqa_q43": Workload("l3_gqa_q43", batch=32, n_q_heads=32, n_kv_heads=8,
                           head_dim=128, key_rank=32, value_rank=256,
                           seq_len=16384, cache="q43", rotate=True,
                           seed=20260400),
    # LongChat-7B-shaped chunked causal prefill: 8192-token chunk on 24576
    # cached tokens, hidden size 4096.
    "longchat_prefill": Workload("longchat_prefill", batch=1, n_q_heads=32,
                                 n_kv_heads=32, head_dim=128, key_rank=32,
                                 value_rank=1024, seq_len=24576, cache="q43",
                                 rotate=True, seed=20260500, hidden=4096,
                                 chunk=8192),
}


# ---------------------------------------------------------------- rounding --

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 (ties to even); returns float32 values."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16 << 16
    return bits.astype(np.uint32).view(np.float32).reshape(f.shape)


def storage_round(x: np.ndarray, cache: str) -> np.ndarray:
    """Round factors / queries / hidden states to their storage dtype."""
    if cache == "f32":
        return np.asarray(x, dtype=np.float32)
    return round_to_bf16(x)


def _rng(w: Workload, *stream) -> np.random.Generator:
    return np.random.default_rng([w.seed, *stream])


# ---------------------------------------------------------------- channels --

def key_channel_std(w: Workload) -> np.ndarray:
    """Per-channel std of the key latent, shape [n_kv_heads, key_rank]."""
    if not w.decaying_latents:
        return np.ones((w.n_kv_heads, w.key_rank))
    i = np.arange(1, w.key_rank + 1, dtype=np.float64)
    std = np.tile(i ** -0.5, (w.n_kv_heads, 1)).reshape(-1)
    n_out = int(round(0.02 * std.size))
    idx = _rng(w, 10).choice(std.size, size=n_out, replace=False)
    std[idx] *= 8.0
    return std.reshape(w.n_kv_heads, w.key_rank)


def value_channel_std(w: Workload) -> np.ndarray:
    """Per-channel std of the joint value latent, shape [value_rank]."""
    if not w.decaying_latents:
        return np.ones(w.value_rank)
    i = np.arange(1, w.value_rank + 1, dtype=np.float64)
    std = i ** -0.5
    n_out = int(round(0.02 * std.size))
    idx = _rng(w, 11).choice(std.size, size=n_out, replace=False)
    std[idx] *= 8.0
    return std


# ----------------------------------------------------------------- factors --

def _orthonormal(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    q, r = np.linalg.qr(rng.standard_normal((rows, cols)))
    return q * np.sign(np.diag(r))[None, :]


def factors(w: Workload):
    """Up-projection factors in the row-vector convention.

    B_key   [n_kv_heads, head_dim, key_rank]:  K_g = Z_k,g @ B_key[g].T
    B_value [n_kv_heads*head_dim, value_rank]: V   = Z_v @ B_value.T
    Returned as float32 arrays holding storage-dtype values.
    """
    rng = _rng(w, 1)
    bk = np.stack([_orthonormal(rng, w.head_dim, w.key_rank)
                   for _ in range(w.n_kv_heads)])
    bv = _orthonormal(rng, w.n_kv_heads * w.head_dim, w.value_rank)
    if w.factor_sigma:
        bk = bk * (np.arange(1, w.key_rank + 1) ** -0.5)[None, None, :]
        bv = bv * (np.arange(1, w.value_rank + 1) ** -0.5)[None, :]
    return storage_round(bk, w.cache), storage_round(bv, w.cache)


def queries(w: Workload, batch: int | None = None, scale: float = 1.0):
    """Decode queries q [batch, n_q_heads, head_dim] ~ N(0, 1)/sqrt(d_h)."""
    b = w.batch if batch is None else batch
    q = _rng(w, 2).standard_normal((b, w.n_q_heads, w.head_dim))
    return storage_round(q * (scale / math.sqrt(w.head_dim)), w.cache)


# ----------------------------------------------------------------- latents --

def latents(w: Workload, b: int, t0: int, n: int, spike: dict | None = None):
    """Latents of batch element b for tokens [t0, t0+n) (the append inputs).

    Returns (z_key [n, n_kv_heads, key_rank], z_value [n, value_rank]) float32.
    Tokens are drawn in independent chunks so any range can be regenerated.
    `spike` = {token: factor} multiplies the whole latent row of those tokens,
    a needle-like outlier for stress tests.
    """
    kstd = key_channel_std(w).reshape(-1).astype(np.float32)
    vstd = value_channel_std(w).astype(np.float32)
    width = kstd.size + vstd.size
    out = np.empty((n, width), dtype=np.float32)
    c0, c1 = t0 // TOKEN_CHUNK, (t0 + n - 1) // TOKEN_CHUNK if n else -1
    for c in range(c0, c1 + 1):
        draw = _rng(w, 3, b, c).standard_normal((TOKEN_CHUNK, width),
                                                dtype=np.float32)
        lo = max(t0, c * TOKEN_CHUNK)
        hi = min(t0 + n, (c + 1) * TOKEN_CHUNK)
        out[lo - t0:hi - t0] = draw[lo - c * TOKEN_CHUNK:hi - c * TOKEN_CHUNK]
    out[:, :kstd.size] *= kstd
    out[:, kstd.size:] *= vstd
    if spike:
        for t, f in spike.items():
            if t0 <= t < t0 + n:
                out[t - t0] *= np.float32(f)
    zk = out[:, :kstd.size].reshape(n, w.n_kv_heads, w.key_rank)
    zv = out[:, kstd.size:]
    return np.ascontiguousarray(zk), np.ascontiguousarray(zv)


def batch_latents(w: Workload, t0: int, n: int, batch: int | None = None):
    """Stacked latents for all batch elements: [B, n, Hkv, r_k], [B, n, R_v]."""
    bs = range(w.batch if batch is None else batch)
    pairs = [latents(w, b, t0, n) for b in bs]
    return (np.stack([p[0] for p in pairs]), np.stack([p[1] for p in pairs]))


# ----------------------------------------------------------------- prefill --

def prefill_inputs(w: Workload, chunk: int | None = None):
    """Prefill chunk inputs for batch element 0.

    X [C, D] ~ N(0, 1); A_key [D, n_kv_heads*key_rank] and A_value
    [D, value_rank] have N(0, 1)/sqrt(D) entries times the latent channel std,
    so X @ A has the same channel statistics as the decode latents;
    Q [C, n_q_heads, head_dim] ~ N(0, 1)/sqrt(d_h).  All rounded to bf16.
    """
    c = w.chunk if chunk is None else chunk
    d = w.hidden
    x = _rng(w, 4).standard_normal((c, d), dtype=np.float32)
    ak = _rng(w, 5).standard_normal((d, w.n_kv_heads * w.key_rank))
    ak *= key_channel_std(w).reshape(1, -1) / math.sqrt(d)
    av = _rng(w, 6).standard_normal((d, w.value_rank))
    av *= value_channel_std(w).reshape(1, -1) / math.sqrt(d)
    q = _rng(w, 7).standard_normal((c, w.n_q_heads, w.head_dim),
                                   dtype=np.float32) / math.sqrt(w.head_dim)
    return (round_to_bf16(x), round_to_bf16(ak), round_to_bf16(av),
            round_to_bf16(q))
