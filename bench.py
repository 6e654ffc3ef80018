"""Benchmark of the INT2 KV-cache hot path on one MI355X.

Workload (LLM-style decode): batch 16, 32 query heads / 8 KV heads (GQA
4:1), head_dim 128, 32768 cached tokens; keys INT2 per channel over
64-token windows, values INT2 per token in groups of 32; synthetic inputs
(RoPE'd keys with log-uniform per-channel scales, N(0,1) values, one query
token per sequence).

One step = kv_quantize_append of the whole 32768-token context of every
sequence into the packed cache, then attn_int2_decode of the new query
against it.  Inputs are resident in HBM before timing starts.  `value` is
the whole job's effective bandwidth: algorithmic bytes of all timed steps
(bf16 K/V read + packed cache written by the append; packed cache + query
read and output written by the decode) over the wall time of the timed
region.  Per-call times come from HIP events on the stream the library
launches on.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "INT2 decode-attn effective GB/s & %HBM peak; quantize-append Mtok/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
B, HQ, HKV, D, T = 16, 32, 8, 128, 32768
CPU_SAMPLE_SEQS = 4            # oracle timed on 4 of the 16 sequences

# Algorithmic bytes per step (what the method must move, not what a kernel
# happens to move): the append reads bf16 K and V and writes codes and
# parameter words; the decode reads the packed cache and the query and
# writes the fp32 output.
APPEND_READ = 2 * B * T * HKV * D * 2
CACHE_BYTES = (B * HKV * T * D // 4          # key codes
               + B * HKV * (T // 64) * D * 4  # key window parameters
               + B * HKV * T * D // 4         # value codes
               + B * HKV * T * (D // 32) * 4)  # value parameters
APPEND_BYTES = APPEND_READ + CACHE_BYTES
DECODE_BYTES = CACHE_BYTES + B * HQ * D * 2 + B * HQ * D * 4

COUNTERS = os.path.join(ROOT, "profiles", "window_append_llm_decode_counters.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "bit_kv_cache_int2_amd", "csrc", f)
                  for f in ("quantize.hip", "device.h")]


def _source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counter_traffic():
    """HBM bytes per append launch from the committed rocprofv3 counter
    summary, or None when it is missing or was taken on other kernel code."""
    if not os.path.exists(COUNTERS):
        return None
    kv = {}
    with open(COUNTERS) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    try:
        if kv.get("source_sha256") != _source_hash(KERNEL_SOURCES):
            return None
        return float(kv["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(d) -> dict:
    """The oracle as it stands, on a bounded sample: the first
    CPU_SAMPLE_SEQS sequences (all 8 KV heads, all 32768 tokens): append,
    then fp64 attention for their 32 query heads."""
    import numpy as np

    import oracle
    import synth

    S = CPU_SAMPLE_SEQS
    K = np.ascontiguousarray(d["K"][:S])
    V = np.ascontiguousarray(d["V"][:S])
    q = synth.bf16_bits_to_f32(d["q"][:S]).astype(np.float64).reshape(S, 1, HQ, D)
    t0 = time.perf_counter()
    c = oracle.Cache(S, HKV, D, T)
    c.append(K, V, 0)
    c.attention(q, T, 1.0 / math.sqrt(D))
    dt = time.perf_counter() - t0
    frac = S / B
    return {"value": round((APPEND_BYTES + DECODE_BYTES) * frac / dt / 1e9, 4), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{S} of {B} sequences (all {HKV} kv heads, {T} tokens): append + fp64 "
                      f"attention, {dt:.2f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the path has no multi-GPU leg "
              "(sharding is described in DESIGN.md); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import bit_kv_cache_int2_amd as kv
    import synth

    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    d = synth.llm_decode(B=B, Hkv=HKV, Hq=HQ, D=D, T=T)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    Kd, Vd, qd = to_dev(d["K"]), to_dev(d["V"]), to_dev(d["q"])
    cache = kv.KVCache(B, HKV, D, T)
    ws = kv.decode_workspace(cache, HQ, T)
    out = torch.empty((B, HQ, D), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    torch.cuda.synchronize()
    print(f"inputs ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    def step(ev=None):
        if ev:
            ev[0].record()
        kv.kv_quantize_append(cache, Kd, Vd, 0)
        if ev:
            ev[1].record()
        kv.attn_int2_decode(cache, T, qd, scale, out=out, workspace=ws)
        if ev:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_app = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps * 1e-3
    t_dec = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps * 1e-3
    print(f"timed {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    value = (APPEND_BYTES + DECODE_BYTES) * args.steps / wall / 1e9
    app_gbs = APPEND_BYTES / t_app / 1e9
    dec_gbs = DECODE_BYTES / t_dec / 1e9
    traffic = _counter_traffic()
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": "llm_decode_gqa", "batch": B, "q_heads": HQ, "kv_heads": HKV,
                   "head_dim": D, "context": T, "keys": "int2 per channel, 64-token windows",
                   "values": "int2 per token, groups of 32"},
        "decode": {"us": round(t_dec * 1e6, 2), "effective_gbs": round(dec_gbs, 1),
                   "pct_hbm_peak": round(100 * dec_gbs / HBM_PEAK_GBS, 2),
                   "bytes": DECODE_BYTES},
        "quantize_append": {"us": round(t_app * 1e6, 2),
                            "mtok_s": round(B * T / t_app / 1e6, 1),
                            "effective_gbs": round(app_gbs, 1),
                            "pct_hbm_peak": round(100 * app_gbs / HBM_PEAK_GBS, 2),
                            "bytes": APPEND_BYTES},
        "roofline": {"kernel": "window_append_kernel", "bound": "hbm",
                     "achieved": round(app_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(app_gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
        "roofline_decode": {"kernel": "decode_partial_kernel + decode_reduce_kernel",
                            "bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4)},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
