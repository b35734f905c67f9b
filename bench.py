#!/usr/bin/env python3
"""Benchmark of latent-KV decode attention on one MI355X.

One step = one decode step of the whole hot path for a batch of sequences:
one starkv_decode_step call -- the append of the step's new token (quantize +
pack, n = 1 per sequence) and the decode over seq_len cached tokens (query
projection, split scores + online softmax + MFMA P.Z_v, split merge, value
up-projection); the append and the query projection share one launch (every cache kind but rotary keys).

Default workload: B = 16 sequences, T = 32768 cached tokens, LLaMA-2-7B-shaped
(32 heads, d_h 128, key rank 32 per head, joint value rank 1024), 4/3-bit
Hadamard-rotated latent cache -- 1216 bytes per token, 637.5 MB per step.
Inputs are seeded synthetic tensors already resident in HBM; before each
timed step a 1 GiB buffer is written so the 256 MB Infinity Cache and the L2s
hold none of the cache (as when the other layers of a model run in between).

Prints one JSON line (metric, value = tokens attended per second = B*T / step
time, roofline of the split kernel measured with HIP events on its launch
stream, CPU oracle baseline on a bounded sample).  The step rate is timed
over plain calls; per-kernel times come from a second pass of the same
number of steps in which the library records events between its kernels.

--workload longchat_prefill times the chunked causal prefill instead (one
starkv_prefill of an 8192-token chunk on 24576 cached tokens per step) and
reports the attention kernel against the MFMA peak; with --rope-theta the
keys are reconstructed and rotated at their positions, and the scores run
over d_h channels instead of r_k.

--t-sweep runs the default decode workload at T = 8K, 16K, 32K, 64K and 128K
(one child process each) and prints one JSON line per T plus a line with the
marginal bandwidth of the split kernel (bytes added / time added between
successive T) and its fixed cost per launch.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("latent-KV decode attention: tokens attended/s and % HBM roofline "
          "at B=16, T=32K")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA, published peak
COUNTERS = os.path.join(ROOT, "profiles", "split_kernel_l2_q43_counters.json")
# sources of the split kernel the counters describe: a change to any of them
# invalidates the committed traffic figure
SPLIT_SRCS = [os.path.join(ROOT, "decode_attention_starkv_amd", "csrc", f)
              for f in ("decode.hip", "split_q43.h", "device.h", "internal.h")]


PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "prefill_attn_longchat_counters.json")
PREFILL_SRCS = [os.path.join(ROOT, "decode_attention_starkv_amd", "csrc", f)
                for f in ("prefill.hip", "device.h", "internal.h")]


def sources_sha256(paths):
    h = hashlib.sha256()
    for f in paths:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def split_sources_sha256():
    return sources_sha256(SPLIT_SRCS)


def prefill_traffic_from_counters(w, ctx, chunk):
    """HBM bytes per prefill attention launch from committed rocprofv3
    counters, or None if its sources changed since they were taken or the run
    is not the configuration they were taken on (longchat_prefill defaults)."""
    if (w.name, w.batch, ctx, chunk) != ("longchat_prefill", 1, 24576, 8192):
        return None
    if not os.path.exists(PREFILL_COUNTERS):
        return None
    rec = json.load(open(PREFILL_COUNTERS))
    if rec.get("prefill_sources_sha256") != sources_sha256(PREFILL_SRCS):
        return None
    return rec.get("hbm_bytes_per_launch")



def prefill_reconstructs(w, chunk):
    """The library's choice for a prefill chunk: reconstruct the values of
    every visible position once (eq. 12 in its left-hand order) when the
    chunk's queries outweigh it, C Hq (R_v - d_h) > Hkv d_h R_v, for d_h 64
    or 128; else contract with the joint latent."""
    return (w.cache == "q43" and w.head_dim in (64, 128) and w.value_rank > w.head_dim
            and chunk * w.n_q_heads * (w.value_rank - w.head_dim)
            > w.n_kv_heads * w.head_dim * w.value_rank)


def cache_label(w):
    kind = "u4" if w.cache == "q43" and w.lo_bits == 4 else w.cache
    return kind + (" rotated" if w.rotate else "")


def qbits(w):
    """make_config keywords of a quantized workload's precision split (the
    trailing block's width: 3 bits, or 4 for a uniform 4-bit cache)."""
    return dict(lo_bits=w.lo_bits) if w.cache == "q43" else {}

def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="l2_q43")
    p.add_argument("--batch", type=int, default=0)
    p.add_argument("--seq-len", type=int, default=0)
    p.add_argument("--splits", type=int, default=0)
    p.add_argument("--no-flush", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=32768)
    p.add_argument("--rope-theta", type=float, default=0.0,
                   help="rotary position embedding of the keys (base theta): "
                        "fused into the latent-key scoring (decode) or applied "
                        "to the reconstructed keys (prefill)")
    p.add_argument("--hidden", type=int, default=0,
                   help="decode through the fused value/output factor into a "
                        "hidden size of this width (starkv_decode_hidden)")
    p.add_argument("--t-sweep", action="store_true",
                   help="decode at T = 8K .. 128K, one JSON line per T")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run one plain 1 GiB device-to-device copy, the "
                        "reference for scaling HBM byte counters")
    return p.parse_args()


def percentiles(v):
    """p10 / p50 / p90 of a list of times (nearest rank)."""
    s = sorted(v)
    pick = lambda q: s[min(len(s) - 1, max(0, int(math.ceil(q * len(s))) - 1))]
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


def host_info():
    """What the CPU baseline ran on: CPU model, usable cores, BLAS."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = []
    try:
        import numpy  # noqa: F401  (loads the BLAS it reports)
        from threadpoolctl import threadpool_info
        blas = sorted({f"{i.get('internal_api')}:{i.get('num_threads')}"
                       for i in threadpool_info()})
    except Exception:  # noqa: BLE001
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)),
            "blas": blas}


def t_sweep():
    """Decode at several T (one child process each, this process never
    touches the GPU) and the split kernel's marginal bandwidth between them."""
    import subprocess
    rows = []
    for T in (8192, 16384, 32768, 65536, 131072):
        cmd = [sys.executable, os.path.abspath(__file__), "--seq-len", str(T),
               "--steps", "20", "--warmup", "10", "--no-cpu-baseline"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stderr[-2000:])
            sys.exit(res.returncode)
        r = json.loads(res.stdout.strip().splitlines()[-1])
        split_us = r["kernels_ms"]["split"] * 1e3
        row = {"t_sweep": True, "seq_len": T, "batch": r["config"]["batch"],
               "splits": r["config"]["splits"], "ms_per_step": r["ms_per_step"],
               "tokens_per_s": r["value"], "split_us": split_us,
               "split_hbm_frac": r["roofline"]["frac"],
               "cache_bytes": r["algorithmic_bytes"]["cache"]}
        rows.append(row)
        print(json.dumps(row), flush=True)
    marg = []
    for a, b in zip(rows, rows[1:]):
        db = b["cache_bytes"] - a["cache_bytes"]
        dt = (b["split_us"] - a["split_us"]) * 1e-6
        marg.append({"from_T": a["seq_len"], "to_T": b["seq_len"],
                     "marginal_GBps": db / dt / 1e9})
    last = marg[-1]["marginal_GBps"] if marg else None
    fixed = (rows[-1]["split_us"] - rows[-1]["cache_bytes"] / (last * 1e9) * 1e6) if last else None
    print(json.dumps({"t_sweep_summary": True, "marginal": marg,
                      "fixed_us_per_launch_at_last_rate": fixed}), flush=True)


def algorithmic_bytes(w, cfg, seq_len, sk):
    """Cache bytes one decode call must read (codes + fp16 scale/zero) for
    seq_len tokens of every sequence, and the factor bytes."""
    per_token = sum(sk.starkv_cache_bytes(cfg, i) for i in range(4)) / (
        cfg.batch * cfg.max_tokens)
    cache = per_token * cfg.batch * seq_len
    es = 4 if w.cache == "f32" else 2
    factors = (w.n_kv_heads * w.head_dim * w.key_rank
               + w.n_kv_heads * w.head_dim * w.value_rank) * es
    return cache, factors


def fill_cache(w, cfg, cache, seq_len, sk, torch):
    """Append seq_len synthetic tokens to every sequence, on the GPU."""
    import synth
    kstd = torch.tensor(synth.key_channel_std(w), dtype=torch.float32, device="cuda")
    vstd = torch.tensor(synth.value_channel_std(w), dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    chunk = 4096
    for p0 in range(0, seq_len, chunk):
        n = min(chunk, seq_len - p0)
        zk = torch.randn((cfg.batch, n, w.n_kv_heads, w.key_rank), device="cuda",
                         generator=gen) * kstd
        zv = torch.randn((cfg.batch, n, w.value_rank), device="cuda",
                         generator=gen) * vstd
        sk.starkv_append(cfg, cache, zk.contiguous(), zv.contiguous(), p0, n)
    torch.cuda.synchronize()


def cpu_baseline(w, seq_len, min_s=10.0, max_reps=30):
    """The oracle, as it stands, on a bounded sample of the workload: decode
    of all heads of one sequence over seq_len tokens, repeated until at least
    min_s seconds of CPU work (its cache build is setup, not timed)."""
    import numpy as np
    import synth
    from oracle import attention as oa
    from oracle import cache as oc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    w1 = w.replace(batch=1)
    c = oc.Cache.for_workload(w1, max_tokens=((seq_len + 63) // 64) * 64)
    for p0 in range(0, seq_len, 8192):
        n = min(8192, seq_len - p0)
        zk, zv = synth.batch_latents(w1, p0, n)
        c.append(zk, zv, p0, n)
    bk, bv = synth.factors(w1)
    q = synth.queries(w1)
    reps, dt = 0, 0.0
    while dt < min_s and reps < max_reps:
        t0 = time.perf_counter()
        out = oa.decode(c, seq_len, q, bk, bv, 1 / math.sqrt(w.head_dim),
                        w.n_q_heads, w.rotate)
        dt += time.perf_counter() - t0
        reps += 1
        assert np.isfinite(out).all()
    return {"value": reps * seq_len / dt, "unit": "tokens attended/s",
            "cores": threads, "kind": "oracle", "host": host_info(),
            "sample": f"{reps} x decode of 1 sequence x {seq_len} tokens x "
                      f"{w.n_q_heads} heads of the same workload (fp64 numpy, "
                      f"{dt:.1f} s total)"}


def prefill_pairs(ctx, chunk, n_q_heads):
    """(query, head, key) pairs of a causal chunk: query i sees ctx + i + 1."""
    return n_q_heads * (chunk * ctx + chunk * (chunk + 1) // 2)


def cpu_baseline_prefill(w, n_rows=64, min_s=10.0, max_reps=30, rope_theta=0.0):
    """The oracle, as it stands, on a bounded sample of the prefill workload:
    causal attention of n_rows evenly spaced queries of the chunk (all heads)
    over the cache, repeated until at least min_s seconds of CPU work;
    building the cache is setup, not timed."""
    import numpy as np
    import synth
    from oracle import attention as oa
    from oracle import cache as oc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    ctx, chunk = w.seq_len, w.chunk
    total = ctx + chunk
    c = oc.Cache.for_workload(w, max_tokens=((total + 63) // 64) * 64)
    for p0 in range(0, total, 8192):
        n = min(8192, total - p0)
        zk, zv = synth.batch_latents(w, p0, n)
        c.append(zk, zv, p0, n)
    bk, bv = synth.factors(w)
    _, _, _, q = synth.prefill_inputs(w)
    rows = np.linspace(0, chunk - 1, n_rows).astype(np.int64)
    reps, dt = 0, 0.0
    while dt < min_s and reps < max_reps:
        t0 = time.perf_counter()
        out = oa.causal_attention(c, ctx, q, bk, bv, 1 / math.sqrt(w.head_dim),
                                  w.n_q_heads, w.rotate, rows=rows, rope_theta=rope_theta)
        dt += time.perf_counter() - t0
        reps += 1
        assert np.isfinite(out).all()
    return {"value": reps * n_rows / dt, "unit": "chunk tokens/s", "cores": threads,
            "host": host_info(),
            "kind": "oracle",
            "sample": f"{reps} x causal attention of {n_rows} evenly spaced queries "
                      f"x {w.n_q_heads} heads of the {chunk}-token chunk over "
                      f"{ctx}+ cached tokens"
                      + (f", rotary keys theta {rope_theta:g}" if rope_theta else "")
                      + f" (fp64 numpy, {dt:.1f} s total)"}


def run_prefill(args, w, torch, sk, synth):
    ctx, chunk = (args.seq_len or w.seq_len), w.chunk
    T = ((ctx + chunk + 63) // 64) * 64
    rope = args.rope_theta
    cfg = sk.make_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim,
                         w.key_rank, w.value_rank, T, w.cache, w.rotate, rope_theta=rope,
                         **qbits(w))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"# workload {w.name} B={w.batch} ctx={ctx} chunk={chunk} rope_theta={rope}",
          file=sys.stderr, flush=True)
    cache = sk.LatentCache(cfg)
    if ctx:
        fill_cache(w, cfg, cache, ctx, sk, torch)
    x, ak, av, q = synth.prefill_inputs(w, chunk)
    bk, bv = synth.factors(w)
    bf = torch.bfloat16
    x_t = torch.from_numpy(x).to(dev, bf).reshape(w.batch, chunk, w.hidden).contiguous()
    ak_t = torch.from_numpy(ak).to(dev, bf)
    av_t = torch.from_numpy(av).to(dev, bf)
    q_t = torch.from_numpy(q).to(dev, bf).reshape(w.batch, chunk, w.n_q_heads,
                                                   w.head_dim).contiguous()
    bk_t = torch.from_numpy(bk).to(dev, bf)
    bv_t = torch.from_numpy(bv).to(dev, bf)
    out = torch.empty((w.batch, chunk, w.n_q_heads, w.head_dim), device=dev)
    ws = sk.workspace(cfg, sk.OP_PREFILL, chunk)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(w.head_dim)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()

    def step(i):
        if not args.no_flush:
            flush.fill_(i & 0xFF)
        sk.starkv_prefill_profiled(cfg, cache, ctx, chunk, x_t, w.hidden, ak_t, av_t,
                                   q_t, bk_t, bv_t, scale, out, ws, ev)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    step_ms, kern = [], [[] for _ in range(5)]
    for i in range(args.steps):
        step(i)
        torch.cuda.synchronize()
        step_ms.append(ev[0].elapsed_time(ev[5]))
        for k in range(5):
            kern[k].append(ev[k].elapsed_time(ev[k + 1]))
        print(f"# step {i} {step_ms[-1]:.3f} ms (attention {kern[3][-1]:.3f} ms)",
              file=sys.stderr, flush=True)
    assert torch.isfinite(out).all()
    mean = lambda v: sum(v) / len(v)
    ms = mean(step_ms)
    attn_ms = mean(kern[3])
    pairs = prefill_pairs(ctx, chunk, w.n_q_heads) * w.batch
    rec = prefill_reconstructs(w, chunk)
    # scores over the r_k latent channels, or over the d_h channels of the
    # reconstructed rotary keys; then the value contraction over d_h
    # (reconstructed values) or over R_v (the joint latent)
    attn_flops = pairs * 2 * ((w.head_dim if rope else w.key_rank)
                              + (w.head_dim if rec else w.value_rank))
    # the reconstruction itself (a pre-pass): 2 Hkv d_h R_v per position
    recon_flops = (2 * w.batch * (ctx + chunk) * w.n_kv_heads * w.head_dim * w.value_rank
                   if rec else 0)
    gemm_flops = 2 * w.batch * chunk * w.hidden * (w.n_kv_heads * w.key_rank + w.value_rank)
    achieved = attn_flops / (attn_ms * 1e-3) / 1e12
    res = {
        "metric": "chunked causal prefill over the latent cache: chunk tokens/s",
        "value": w.batch * chunk / (ms * 1e-3),
        "unit": "chunk tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{w.name} prefill" + (" rope" if rope else ""),
                   "batch": w.batch, "rope_theta": rope,
                   "ctx_len": ctx, "chunk": chunk, "hidden": w.hidden,
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "key_rank": w.key_rank,
                   "value_rank": w.value_rank,
                   "cache": cache_label(w)},
        "roofline": {"bound": "mfma",
                     "kernel": "prefill_attn_rec_kernel" if rec else "prefill_attn_kernel",
                     "achieved": achieved, "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_PEAK_TFLOPS,
                     "traffic": None if rope else prefill_traffic_from_counters(w, ctx, chunk)},
        # prepasses: the keys and queries of the scores (and, when the values
        # are reconstructed, their dequantization and reconstruction GEMM);
        # up_projection: empty when the attention writes d_h-wide rows
        "values": "reconstructed" if rec else "joint latent",
        "kernels_ms": {"gemm": mean(kern[0]), "append": mean(kern[1]),
                       "prepasses": mean(kern[2]), "attention": attn_ms,
                       "up_projection": mean(kern[4])},
        # the latent projection Z = X A (Algorithm 2, step 1) on MFMA
        "projection_gemm_mfma": {
            "flop": gemm_flops,
            "tflops": gemm_flops / (mean(kern[0]) * 1e-3) / 1e12,
            "frac": gemm_flops / (mean(kern[0]) * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS},
        "algorithmic_flops": {"attention": attn_flops, "projection": gemm_flops,
                              "value_reconstruction": recon_flops},
    }
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline_prefill(w, rope_theta=rope)
    print(json.dumps(res))


def run_hidden(args, w, torch, sk, synth):
    """Decode that ends in the hidden size through the fused factor
    F_h = B_value[g(h)]^T O_h (review section 5.3, eq. 12; Algorithm 2, steps
    7-8).  One step = one starkv_decode_hidden call; the roofline is the
    hidden GEMM's (it streams F once)."""
    seq_len = args.seq_len or w.seq_len
    D = args.hidden
    cfg = sk.make_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim,
                         w.key_rank, w.value_rank, ((seq_len + 63) // 64) * 64,
                         w.cache, w.rotate, args.splits, **qbits(w))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"# workload {w.name} B={w.batch} T={seq_len} hidden={D}", file=sys.stderr,
          flush=True)
    cache = sk.LatentCache(cfg)
    fill_cache(w, cfg, cache, seq_len, sk, torch)
    bk, bv = synth.factors(w)
    bf = torch.bfloat16
    bk_t = torch.from_numpy(bk).to(dev, bf)
    bv_t = torch.from_numpy(bv).to(dev, bf)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 7)
    w_o = (torch.randn((w.n_q_heads * w.head_dim, D), device=dev, generator=gen)
           / math.sqrt(w.n_q_heads * w.head_dim)).to(bf)
    F = torch.empty(sk.starkv_fused_factor_bytes(cfg, D), dtype=torch.uint8, device=dev)
    sk.starkv_fuse_value_output(cfg, bv_t, w_o, D, F)
    q_t = torch.from_numpy(synth.queries(w)).to(dev, bf)
    y = torch.empty((w.batch, D), device=dev)
    ws = torch.empty(sk.starkv_decode_hidden_workspace_bytes(cfg, seq_len, D),
                     dtype=torch.uint8, device=dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(w.head_dim)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()

    def step(i, profiled):
        if not args.no_flush:
            flush.fill_(i & 0xFF)
        ev[6].record()
        sk.starkv_decode_hidden(cfg, cache, seq_len, q_t, bk_t, F, D, scale, y, ws,
                                events=ev[:6] if profiled else None)
        ev[7].record()

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    step_ms, kern = [], [[] for _ in range(5)]
    for i in range(args.steps):
        step(i, False)
        torch.cuda.synchronize()
        step_ms.append(ev[6].elapsed_time(ev[7]))
    for i in range(args.steps):
        step(i, True)
        torch.cuda.synchronize()
        for k in range(5):
            kern[k].append(ev[k].elapsed_time(ev[k + 1]))
        print(f"# profiled step {i}: hidden gemm {kern[3][-1]:.4f} ms", file=sys.stderr,
              flush=True)
    assert torch.isfinite(y).all()
    mean = lambda v: sum(v) / len(v)
    ms = mean(step_ms)
    gemm_ms = mean(kern[3])
    f_bytes = F.numel()
    gemm_bytes = f_bytes + w.batch * w.n_q_heads * w.value_rank * 4 + w.batch * D * 4
    cache_bytes, _ = algorithmic_bytes(w, cfg, seq_len, sk)
    achieved = gemm_bytes / (gemm_ms * 1e-3) / 1e9
    res = {
        "metric": "latent-KV decode into the hidden size through the fused "
                  "value/output factor: tokens attended/s",
        "value": w.batch * seq_len / (ms * 1e-3), "unit": "tokens attended/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{w.name} decode_hidden", "batch": w.batch,
                   "seq_len": seq_len, "hidden": D, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "key_rank": w.key_rank, "value_rank": w.value_rank,
                   "cache": cache_label(w),
                   "fused_factor_bytes": f_bytes,
                   "cache_flushed_before_step": not args.no_flush},
        "roofline": {"bound": "hbm", "kernel": "hidden_gemm_kernel",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None},
        "step_hbm_frac": (cache_bytes + gemm_bytes) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kernels_ms": {"qproj": mean(kern[0]), "split": mean(kern[1]),
                       "merge": mean(kern[2]), "hidden_gemm": gemm_ms,
                       "k_slice_reduce": mean(kern[4])},
        "algorithmic_bytes": {"cache": cache_bytes, "hidden_gemm": gemm_bytes},
    }
    print(json.dumps(res))


def stream_read_ceiling(torch, sk, dev, gib=2, reps=10):
    """Measured streaming-read bandwidth (GB/s): starkv_stream_read over a
    buffer 8x the Infinity Cache, read once per pass with the split kernel's
    non-temporal 16-byte loads; the median of `reps` passes."""
    buf = torch.full((gib << 30,), 7, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sk.starkv_stream_read(buf, sink)
    ts = []
    for _ in range(reps):
        e0.record()
        sk.starkv_stream_read(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del buf
    torch.cuda.empty_cache()
    ts.sort()
    return (gib << 30) / (ts[len(ts) // 2] * 1e-3) / 1e9


def traffic_from_counters(w, batch, seq_len, splits):
    """HBM bytes per split-kernel launch from committed rocprofv3 counters,
    or None if the kernel source changed since they were taken or the run is
    not the configuration they were taken on (l2_q43, B 16, T 32768)."""
    if (w.name, batch, seq_len, splits) != ("l2_q43", 16, 32768, 16):
        return None
    if not os.path.exists(COUNTERS):
        return None
    rec = json.load(open(COUNTERS))
    if rec.get("split_sources_sha256") != split_sources_sha256():
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the decode path runs on one GPU only; "
                          "--gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    if args.t_sweep:
        return t_sweep()
    import torch

    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "read_bytes": 1 << 30,
                          "write_bytes": 1 << 30}))
        return

    import decode_attention_starkv_amd as sk
    import synth

    w = synth.WORKLOADS[args.workload]
    if args.batch:
        w = w.replace(batch=args.batch)
    if w.chunk:
        return run_prefill(args, w, torch, sk, synth)
    if args.hidden:
        return run_hidden(args, w, torch, sk, synth)
    seq_len = args.seq_len or w.seq_len
    cfg = sk.make_config(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim,
                         w.key_rank, w.value_rank, ((seq_len + 63) // 64) * 64,
                         w.cache, w.rotate, args.splits, rope_theta=args.rope_theta,
                         **qbits(w))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"# workload {w.name} B={w.batch} T={seq_len} rope_theta={args.rope_theta} splits="
          f"{sk.starkv_decode_splits(cfg, seq_len)}", file=sys.stderr, flush=True)

    cache = sk.LatentCache(cfg)
    fill_cache(w, cfg, cache, seq_len, sk, torch)
    bk, bv = synth.factors(w)
    dt = torch.float32 if w.cache == "f32" else torch.bfloat16
    bk_t = torch.from_numpy(bk).to(dev, dt)
    bv_t = torch.from_numpy(bv).to(dev, dt)
    q_t = torch.from_numpy(synth.queries(w)).to(dev, dt)
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), device=dev)
    ws = sk.workspace(cfg, sk.OP_DECODE, seq_len)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 1)
    new_k = (torch.randn((w.batch, 1, w.n_kv_heads, w.key_rank), device=dev,
                         generator=gen)
             * torch.tensor(synth.key_channel_std(w), dtype=torch.float32, device=dev))
    new_v = (torch.randn((w.batch, 1, w.value_rank), device=dev, generator=gen)
             * torch.tensor(synth.value_channel_std(w), dtype=torch.float32, device=dev))
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(w.head_dim)

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
    for e in ev:
        e.record()          # create the events before handing them out
    torch.cuda.synchronize()


    def step(i, profiled):
        if not args.no_flush:
            flush.fill_(i & 0xFF)
        ev[5].record()
        # append the step's new token at seq_len - 1, then decode over seq_len
        sk.starkv_decode_step(cfg, cache, new_k, new_v, seq_len - 1, q_t, bk_t, bv_t,
                              scale, out, ws, events=ev[:5] if profiled else None)
        ev[6].record()

    def attention_call(i):
        if not args.no_flush:
            flush.fill_(i & 0xFF)
        ev[5].record()
        sk.starkv_decode(cfg, cache, seq_len, q_t, bk_t, bv_t, scale, out, ws)
        ev[6].record()

    # Pass 1 (the step rate): plain calls, one event pair around each step.
    # Pass 2 (per-kernel times, the roofline): the library records events
    # between its kernels, which costs ~16 us of step time, so it is timed
    # separately over the same number of steps.
    # Pass 3: the decode attention call alone (no append), one event pair.
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    step_ms, kern_ms, app_ms = [], [[], [], [], []], []
    wall0 = time.perf_counter()
    for i in range(args.steps):
        step(i, False)
        torch.cuda.synchronize()
        step_ms.append(ev[5].elapsed_time(ev[6]))
        print(f"# step {i} {step_ms[-1]:.4f} ms", file=sys.stderr, flush=True)
    wall = time.perf_counter() - wall0
    for i in range(args.steps):
        step(i, True)
        torch.cuda.synchronize()
        for j in range(4):
            kern_ms[j].append(ev[j].elapsed_time(ev[j + 1]))
        print(f"# profiled step {i}: split {kern_ms[1][-1]:.4f} ms", file=sys.stderr,
              flush=True)
    call_ms = []
    for i in range(args.steps):
        attention_call(i)
        torch.cuda.synchronize()
        call_ms.append(ev[5].elapsed_time(ev[6]))
    print(f"# decode call alone {sum(call_ms) / len(call_ms):.4f} ms", file=sys.stderr,
          flush=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    stream_gbs = stream_read_ceiling(torch, sk, dev)

    mean = lambda v: sum(v) / len(v)
    ms = mean(step_ms)
    split_ms = mean(kern_ms[1])
    cache_bytes, factor_bytes = algorithmic_bytes(w, cfg, seq_len, sk)
    achieved = cache_bytes / (split_ms * 1e-3) / 1e9
    tokens = w.batch * seq_len
    roofline = {"bound": "hbm", "kernel": "split_kernel",
                "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "traffic": traffic_from_counters(w, w.batch, seq_len,
                                                 sk.starkv_decode_splits(cfg, seq_len))}
    if args.rope_theta:
        # rotary keys: the dominant kernel is the rotary score kernel, timed
        # alone by events[0..1]; its work is 2 d_h r_k flop per (token, query
        # head) for q~ = Trig M plus 2 r_k for the dot with the latent
        rope_ms = mean(kern_ms[0])
        flops = tokens * w.n_q_heads * (2 * w.head_dim * w.key_rank + 2 * w.key_rank)
        tf = flops / (rope_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": "rope_score_kernel", "achieved": tf,
                    "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": tf / MFMA_PEAK_TFLOPS, "traffic": None,
                    "key_bytes_GBps": tokens * w.n_kv_heads * 21 / (rope_ms * 1e-3) / 1e9}
        achieved = None
    res = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens attended/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{w.name} decode" + (" rope" if args.rope_theta else ""),
                   "batch": w.batch, "rope_theta": args.rope_theta,
                   "seq_len": seq_len, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "key_rank": w.key_rank, "value_rank": w.value_rank,
                   "cache": cache_label(w),
                   "splits": sk.starkv_decode_splits(cfg, seq_len),
                   "cache_flushed_before_step": not args.no_flush},
        "roofline": roofline,
        "split_vs_stream_read": ({"stream_read_GBps": stream_gbs,
                                  "frac": achieved / stream_gbs} if achieved else
                                 {"stream_read_GBps": stream_gbs}),
        # whole step (append + the decode attention call) and the decode
        # attention call alone (query projection, split, merge, up-projection)
        # against the HBM peak; roofline.frac above is the split kernel alone
        "step_hbm_frac": (cache_bytes + factor_bytes) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "decode_call_ms": mean(call_ms),
        "decode_call_hbm_frac": (cache_bytes + factor_bytes) / (mean(call_ms) * 1e-3) / 1e9
                                / HBM_PEAK_GBS,
        # the joint-value contraction P Z_v on MFMA inside the split kernel:
        # 2 B T Hq R_v flop against the dense fp16 MFMA peak (the kernel is
        # bound by HBM, so this is low by design; it is the step the pages
        # move onto matrix units)
        "pzv_mfma": {"flop": 2.0 * tokens * w.n_q_heads * w.value_rank,
                     "tflops": 2.0 * tokens * w.n_q_heads * w.value_rank
                               / (split_ms * 1e-3) / 1e12,
                     "frac": 2.0 * tokens * w.n_q_heads * w.value_rank
                             / (split_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS},
        "ms_per_step_percentiles": percentiles(step_ms),
        "split_ms_percentiles": percentiles(kern_ms[1]),
        # with rotary keys the first interval is the rotary score kernel
        "kernels_ms": {("rope_scores" if args.rope_theta
                        else "append_and_qproj"): mean(kern_ms[0]),
                       "split": split_ms, "merge": mean(kern_ms[2]),
                       "vproj": mean(kern_ms[3])},
        "algorithmic_bytes": {"cache": cache_bytes, "factors": factor_bytes},
        "wall_s_timed_loop": wall,
    }
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, min(seq_len, args.cpu_sample_tokens))
    print(json.dumps(res))


if __name__ == "__main__":
    main()
