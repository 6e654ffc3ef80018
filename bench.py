"""Benchmark of the INT2 KV-cache hot path on one MI355X.

Default line (LLM-style decode): batch 16, 32 query heads / 8 KV heads (GQA
4:1), head_dim 128, 32768 cached tokens; keys INT2 per channel over
64-token windows, values INT2 per token in groups of 32; synthetic inputs
(RoPE'd keys with log-uniform per-channel scales, N(0,1) values, one query
token per sequence), resident in HBM before timing starts.

One step = kv_quantize_append of the whole 32768-token context of every
sequence, a 512 MiB read that evicts the 256 MB Infinity Cache, then
attn_int2_decode of the new query against the packed cache.  `value` is the
decode's effective bandwidth: its algorithmic bytes (packed cache + query
read, output written) over the median of its per-call HIP-event times
(events on the stream the library launches on; p10/p90 beside it); the
append's Mtok/s is reported beside it.

The same line carries the other workloads, each with its own roofline and
the oracle timed on the host cores on a bounded sample:
  toy          -- head_dim 64, 512 tokens, one head: decode and append latency;
  video_chunk  -- 40 heads, 4680 query rows against 31200 cached tokens of
                  256-centroid keys (4 GPU k-means rounds from the seeded
                  picks) and rotated values, plus the append of the chunk and
                  the quantisation of the whole 31200-token history;
  long_history -- 40 heads, 1560 query rows against 93600 window-key tokens,
                  plus the append of the new 1560-token frame, and the
                  quantisation of the whole 93600-token history;
  sensitivity  -- 40 heads, 1560 query rows against 65536 tokens of QSAC
                  top-4 centroid keys with rank-8 PSAC (centroids from 4
                  k-means rounds; weights and principal directions from the
                  1024 calibration queries), and the quantisation of the whole
                  65536-token history (the QSAC choice and PSAC terms).
Chunk rooflines are bf16/fp16 MFMA: 4 * q_len * n_tokens * head_dim * heads
flops per call.  Every roofline also carries the fraction of the peak
re-measured on the GPU in the same run (`peaks_measured`: an elementwise
1 GiB kernel for HBM, an MFMA loop for the matrix cores) beside the vendor
figure.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
    python bench.py --workload llm_decode|toy|video_chunk|long_history|sensitivity
                    (one leg alone, for profiling), kmeans, variants, copy

--workload copy runs a plain 1 GiB elementwise copy, the reference for scaling
rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes.
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
MFMA_PEAK_TFS = 2500.0         # MI355X dense fp16/bf16 MFMA, vendor figure
B, HQ, HKV, D, T = 16, 32, 8, 128, 32768
FLUSH_BYTES = 512 << 20        # > the 256 MB Infinity Cache
CPU_SAMPLE_SEQS = 8            # oracle leg of the decode line: this many of the 16 sequences
CPU_CHUNK_ROWS = 512           # oracle leg of a chunk workload: head 0, this many query rows

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

COPY_BYTES = 1 << 30
CSRC = os.path.join(ROOT, "bit_kv_cache_int2_amd", "csrc")
# committed rocprofv3 counter summaries: (file, sources the counters were taken on)
APPEND_COUNTERS = (os.path.join(ROOT, "profiles", "tile_append_llm_decode_counters.txt"),
                   [os.path.join(CSRC, f) for f in ("quantize.hip", "device.h")])
DECODE_COUNTERS = (os.path.join(ROOT, "profiles", "decode_mfma_llm_decode_counters.txt"),
                   [os.path.join(CSRC, f) for f in ("decode.hip", "code_operand.h", "device.h")])
CHUNK_COUNTERS = {w: (os.path.join(ROOT, "profiles", f"chunk_kernel_{w}_counters.txt"),
                      [os.path.join(CSRC, f) for f in ("chunk.hip", "code_operand.h", "device.h")])
                  for w in ("video_chunk", "long_history", "sensitivity")}


def _source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counter_traffic(spec):
    """HBM bytes per launch from a committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by a plain copy's counters), or None
    when it is missing or was taken on other kernel code."""
    path, sources = spec
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    try:
        if kv.get("source_sha256") != _source_hash(sources):
            return None
        return float(kv["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def _stats(ts) -> dict:
    """Median, p10, p90 and mean of per-call times (seconds) in us."""
    import numpy as np
    a = np.asarray(ts, np.float64) * 1e6
    return {"median_us": round(float(np.median(a)), 2), "p10_us": round(float(np.percentile(a, 10)), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2), "mean_us": round(float(a.mean()), 2),
            "calls": int(a.size)}


def _to_dev(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def copy_calibration(steps: int) -> int:
    """A plain elementwise kernel over COPY_BYTES (dst = ~src: each byte
    read once and written once per launch), for scaling rocprofv3's
    FETCH_SIZE and WRITE_SIZE counters to bytes.  (A same-dtype copy_ would
    go to the copy engine, which the counters do not see.)"""
    import torch

    torch.cuda.set_device(0)
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(max(steps, 1)):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"workload": "copy", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                      "launches": max(steps, 1)}), flush=True)
    return 0


def measured_peaks() -> dict:
    """The two roofline denominators re-measured on this GPU beside the
    vendor figures: HBM by the plain elementwise kernel above over 1 GiB
    (dst = ~src, 2 GiB moved per launch), dense fp16 MFMA by the library's
    matrix-core probe (an MFMA loop on register operands, two blocks of
    four waves per CU) and, for context, by a library GEMM (8192 x 8192 x
    8192, torch.mm); medians of 20 per-call HIP-event times after 5 warm-up
    calls."""
    import numpy as np
    import torch

    import bit_kv_cache_int2_amd as kv

    def timed(fn):
        for _ in range(5):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for e0, e1 in evs:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e-3

    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: torch.bitwise_not(src, out=dst))
    del src, dst
    n = 8192
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(n, n, device="cuda", dtype=torch.float16, generator=g)
    b = torch.randn(n, n, device="cuda", dtype=torch.float16, generator=g)
    c = torch.empty(n, n, device="cuda", dtype=torch.float16)
    t_mm = timed(lambda: torch.mm(a, b, out=c))
    del a, b, c
    blocks = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    probe_out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    flops = kv.mfma_peak_probe(blocks, 20000, probe_out)
    t_loop = timed(lambda: kv.mfma_peak_probe(blocks, 20000, probe_out))
    del probe_out
    torch.cuda.empty_cache()
    return {"hbm_gbs": round(2 * COPY_BYTES / t_copy / 1e9, 1),
            "mfma_fp16_tflops": round(flops / t_loop / 1e12, 1),
            "gemm_fp16_tflops": round(2.0 * n ** 3 / t_mm / 1e12, 1),
            "method": "HBM: elementwise dst = ~src over 1 GiB (2 GiB moved); MFMA: an MFMA loop "
                      "(v_mfma_f32_16x16x32_f16 on registers, 2 blocks of 4 waves per CU); GEMM: "
                      "fp16 8192^3 torch.mm; medians of 20 HIP-event-timed calls"}


def _generator_constants() -> dict:
    import synth
    return {"rng": "counter-based SplitMix64 per (seed, stream, index), fp64 Box-Muller normals, bf16 RNE",
            "seed": f"{synth.SEED_BASE:#x} + workload number",
            "streams": {"K": synth.S_K, "V": synth.S_V, "queries": synth.S_Q, "calibration queries": synth.S_QCAL,
                        "k-means picks": synth.S_KMEANS, "per-channel key scales": synth.S_SIGMA,
                        "query subspace": synth.S_SUBSPACE}}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------- decode line
def decode_leg(steps: int, warmup: int) -> tuple[dict, dict]:
    """The default line's GPU part; returns (record, host inputs)."""
    import torch

    import bit_kv_cache_int2_amd as kv
    import synth

    t_gen = time.perf_counter()
    d = synth.llm_decode(B=B, Hkv=HKV, Hq=HQ, D=D, T=T)
    Kd, Vd, qd = _to_dev(d["K"]), _to_dev(d["V"]), _to_dev(d["q"])
    cache = kv.KVCache(B, HKV, D, T)
    ws = kv.decode_workspace(cache, HQ, T)
    out = torch.empty((B, HQ, D), dtype=torch.float32, device="cuda")
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
    flush_sink = torch.zeros((), dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    torch.cuda.synchronize()
    print(f"llm_decode: inputs ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    def step(i, ev=None):
        if ev:
            ev[0].record()
        kv.kv_quantize_append(cache, Kd, Vd, 0)
        if ev:
            ev[1].record()
        # evicts the Infinity Cache between append and decode; a read leaves
        # no dirty lines for the timed kernels to write back (a 512 MiB fill
        # cost the append ~6% and the decode ~9%)
        flush_sink.copy_(flush.sum(dtype=torch.int32))
        if ev:
            ev[2].record()
        kv.attn_int2_decode(cache, T, qd, scale, out=out, workspace=ws)
        if ev:
            ev[3].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_app = [e[0].elapsed_time(e[1]) * 1e-3 for e in evs]
    t_dec = [e[2].elapsed_time(e[3]) * 1e-3 for e in evs]
    print(f"llm_decode: timed {steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)
    sd, sa = _stats(t_dec), _stats(t_app)
    dec_gbs = DECODE_BYTES / (sd["median_us"] * 1e-6) / 1e9
    dec_gbs_mean = DECODE_BYTES / (sd["mean_us"] * 1e-6) / 1e9
    app_gbs = APPEND_BYTES / (sa["median_us"] * 1e-6) / 1e9
    app_gbs_mean = APPEND_BYTES / (sa["mean_us"] * 1e-6) / 1e9
    rec = {
        "metric": METRIC, "value": round(dec_gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16-mfma/fp32-acc", "data": "synthetic",
        "config": {"workload": "llm_decode_gqa", "batch": B, "q_heads": HQ, "kv_heads": HKV,
                   "head_dim": D, "context": T, "keys": "int2 per channel, 64-token windows",
                   "values": "int2 per token, groups of 32"},
        "arithmetic": "decode: fp16 MFMA operands (exact 2-bit code operands; query folded into "
                      "the window scales as fp16 hi + lo; fp16 p*s), fp32 accumulation and softmax; "
                      "append: fp32 min/max and thresholds, fp16 scale/zero",
        "decode": dict(sd, effective_gbs=round(dec_gbs, 1),
                       pct_hbm_peak=round(100 * dec_gbs / HBM_PEAK_GBS, 2), bytes=DECODE_BYTES,
                       infinity_cache="512 MiB read between the append and each decode"),
        "quantize_append": dict(sa, mtok_s=round(B * T / (sa["median_us"] * 1e-6) / 1e6, 1),
                                effective_gbs=round(app_gbs, 1),
                                pct_hbm_peak=round(100 * app_gbs / HBM_PEAK_GBS, 2),
                                bytes=APPEND_BYTES),
        "roofline": {"kernel": "decode_mfma_kernel + decode_reduce_kernel", "bound": "hbm",
                     "achieved": round(dec_gbs_mean, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs_mean / HBM_PEAK_GBS, 4),
                     "traffic": _counter_traffic(DECODE_COUNTERS), "time": "mean per call"},
        "roofline_append": {"kernel": "tile_append_kernel", "bound": "hbm",
                            "achieved": round(app_gbs_mean, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(app_gbs_mean / HBM_PEAK_GBS, 4),
                            "traffic": _counter_traffic(APPEND_COUNTERS), "time": "mean per call"},
    }
    return rec, d


def cpu_decode_baseline(d) -> dict:
    """The oracle as it stands on the first CPU_SAMPLE_SEQS sequences (all
    8 KV heads, all 32768 tokens): append, then fp64 attention for their 32
    query heads, timed separately; value = the attention's effective GB/s
    (the decode's algorithmic bytes, scaled to the sample)."""
    import numpy as np

    import oracle
    import synth

    S = CPU_SAMPLE_SEQS
    K = np.ascontiguousarray(d["K"][:S])
    V = np.ascontiguousarray(d["V"][:S])
    q = synth.bf16_bits_to_f32(d["q"][:S]).astype(np.float64).reshape(S, 1, HQ, D)
    c = oracle.Cache(S, HKV, D, T)
    t0 = time.perf_counter()
    c.append(K, V, 0)
    t_app = time.perf_counter() - t0
    t0 = time.perf_counter()
    c.attention(q, T, 1.0 / math.sqrt(D))
    t_att = time.perf_counter() - t0
    frac = S / B
    return {"value": round(DECODE_BYTES * frac / t_att / 1e9, 4), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "append_mtok_s": round(S * T / t_app / 1e6, 4),
            "sample": f"{S} of {B} sequences (all {HKV} kv heads, {T} tokens): fp64 attention "
                      f"{t_att:.2f} s, append {t_app:.2f} s"}


# ---------------------------------------------------------------- toy (config 1)
def toy_leg(steps: int, warmup: int, with_cpu: bool) -> dict:
    """head_dim 64, 512 tokens, one head, 16 centroids (4 GPU k-means rounds
    from the seeded picks), plain values, one fp32 query: per-call latency of
    the append and the decode (the cache fits in L2: no roofline claim)."""
    import numpy as np
    import torch

    import bit_kv_cache_int2_amd as kv
    import synth

    d = synth.toy_single_head()
    c = kv.KVCache(1, 1, 64, 512, key_mode=kv.KEY_CENTROID, n_centroids=16)
    Kd, Vd = _to_dev(d["K"]), _to_dev(d["V"])
    Kf = synth.bf16_bits_to_f32(d["K"])[0, :, 0]
    c.centroids.copy_(torch.from_numpy(np.ascontiguousarray(Kf[d["kmeans_init"][0, 0]]))[None, None])
    kv.kv_kmeans(Kd, c.centroids, 4)
    q = torch.from_numpy(d["q"]).cuda()
    out = torch.empty((1, 1, 64), dtype=torch.float32, device="cuda")
    ws = kv.decode_workspace(c, 1, 512)

    def step(ev=None):
        if ev:
            ev[0].record()
        kv.kv_quantize_append(c, Kd, Vd, 0)
        if ev:
            ev[1].record()
        kv.attn_int2_decode(c, 512, q, 0.125, out=out, workspace=ws)
        if ev:
            ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    rec = {"config": {"workload": "toy_single_head", "heads": 1, "head_dim": 64, "context": 512,
                      "keys": "16 centroids + int2 residual", "values": "int2 per token, groups of 32"},
           "decode": _stats([e[1].elapsed_time(e[2]) * 1e-3 for e in evs]),
           "quantize_append": _stats([e[0].elapsed_time(e[1]) * 1e-3 for e in evs]),
           "roofline": None}
    if with_cpu:
        rec["cpu_baseline"] = cpu_toy_baseline(d)
    return rec


def cpu_toy_baseline(d) -> dict:
    """The oracle on the whole toy workload: its own 4 k-means rounds from
    the seeded picks (untimed), then the append and the fp64 decode."""
    import numpy as np

    import oracle
    import synth

    Kf = np.ascontiguousarray(synth.bf16_bits_to_f32(d["K"])[0, :, 0])
    o = oracle.Cache(1, 1, 64, 512, oracle.KEY_CENTROID, oracle.VAL_GROUP, C=16)
    o.centroids[0, 0] = oracle.kmeans(Kf, 16, d["kmeans_init"][0, 0], 4)[0]
    t0 = time.perf_counter()
    o.append(d["K"], d["V"], 0)
    t1 = time.perf_counter()
    o.attention(d["q"].astype(np.float64).reshape(1, 1, 1, 64), 512, 0.125)
    t2 = time.perf_counter()
    return {"value": round((t2 - t1) * 1e6, 1), "unit": "us (decode latency)",
            "cores": oracle.num_threads(), "kind": "oracle", "append_us": round((t1 - t0) * 1e6, 1),
            "sample": "the whole workload"}


# ---------------------------------------------------------------- chunk workloads
def _psac_sign(U):
    """The principal-direction sign rule: the largest-magnitude component
    of each column positive (the first one on ties)."""
    import numpy as np
    U = U.copy()
    for m in range(U.shape[1]):
        i = int(np.argmax(np.abs(U[:, m])))
        if U[i, m] < 0:
            U[:, m] = -U[:, m]
    return U


def chunk_leg(name: str, steps: int, warmup: int, history_quantize: bool = True) -> tuple[dict, dict]:
    """Chunk attention of 40 heads (head_dim 128) against a packed history;
    returns (record, host inputs + calibration for the oracle leg)."""
    import numpy as np
    import torch

    import bit_kv_cache_int2_amd as kv
    import synth

    t_gen = time.perf_counter()
    kmeans_rounds = 0
    if name == "long_history":
        d = synth.long_history()
        H, Tn, Lq = d["Hkv"], d["T"], d["Lq"]
        cache = kv.KVCache(1, H, D, ((Tn + Lq + 63) // 64) * 64)
        desc = {"workload": "long_history", "heads": H, "head_dim": D, "context": Tn, "q_len": Lq,
                "keys": "int2 per channel, 64-token windows + bf16 tail",
                "values": "int2 per token, groups of 32", "append_per_step": Lq}
    elif name == "video_chunk":
        d = synth.video_chunk()
        H, Tn, Lq = d["Hkv"], d["T"], d["Lq"]
        cache = kv.KVCache(1, H, D, ((Tn + Lq + 63) // 64) * 64, key_mode=kv.KEY_CENTROID,
                           n_centroids=256, value_mode=kv.VAL_HADAMARD)
        kmeans_rounds = 4
        desc = {"workload": "video_chunk", "heads": H, "head_dim": D, "context": Tn, "q_len": Lq,
                "keys": "256 centroids (4 k-means rounds) + int2 residual, groups of 32",
                "values": "Walsh-Hadamard rotated, int2 per token, groups of 32",
                "append_per_step": Lq}
    elif name == "sensitivity":
        d = synth.sensitivity_aware()
        H, Tn, Lq = d["Hkv"], d["T"], d["Lq"]
        cache = kv.KVCache(1, H, D, ((Tn + 63) // 64) * 64, key_mode=kv.KEY_CENTROID_QSAC,
                           n_centroids=256, qsac_topk=4, psac_rank=8, value_mode=kv.VAL_HADAMARD)
        kmeans_rounds = 4
        # query sensitivity and principal directions of the 1024 calibration
        # queries: w = mean q^2, U = top-8 eigenvectors of the uncentred second
        # moment (fp64), largest component of each made positive
        qc = synth.bf16_bits_to_f32(d["q_cal"]).astype(np.float64)
        w = (qc ** 2).mean(0).astype(np.float32)                       # [H][D]
        U = np.stack([_psac_sign(np.linalg.eigh(qc[:, h].T @ qc[:, h] / qc.shape[0])[1][:, ::-1][:, :8])
                      for h in range(H)]).astype(np.float32)
        cache.sens_w.copy_(torch.from_numpy(w[None]))
        cache.psac_basis.copy_(torch.from_numpy(np.ascontiguousarray(U[None])))
        desc = {"workload": "sensitivity", "heads": H, "head_dim": D, "context": Tn, "q_len": Lq,
                "keys": "256 centroids (4 k-means rounds), QSAC top-4, int2 residual, PSAC rank 8 fp16",
                "values": "Walsh-Hadamard rotated, int2 per token, groups of 32",
                "calibration": "w and U from 1024 calibration queries", "append_per_step": 0}
    else:
        raise SystemExit(f"unknown workload {name}")
    Kd, Vd, qd = _to_dev(d["K"]), _to_dev(d["V"]), _to_dev(d["q"])
    if kmeans_rounds:
        K = synth.bf16_bits_to_f32(d["K"])[0]
        cent = np.stack([K[d["kmeans_init"][0, h], h] for h in range(H)])[None]
        del K
        cache.centroids.copy_(torch.from_numpy(np.ascontiguousarray(cent)))
        kv.kv_kmeans(Kd, cache.centroids, kmeans_rounds)
    kv.kv_quantize_append(cache, Kd, Vd, 0)
    Kn = _to_dev(d["K_new"]) if "K_new" in d else None
    Vn = _to_dev(d["V_new"]) if "V_new" in d else None
    out = torch.empty((1, Lq, H, D), dtype=torch.float32, device="cuda")
    ws = kv.chunk_workspace(cache, Lq, H, Tn)
    scale = 1.0 / math.sqrt(D)
    # window keys: the chunk reads the history's unfinished window from the
    # tail, which the step's own append overwrites; each step restores it
    tail0 = cache.k_tail.clone() if cache.k_tail is not None else None
    torch.cuda.synchronize()
    print(f"{name}: inputs and cache ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr,
          flush=True)

    rec = {"config": desc}
    if history_quantize:
        # quantisation of the whole history (Tn tokens x 40 heads): the same
        # call that built the cache, so the state is unchanged
        hist = lambda: kv.kv_quantize_append(cache, Kd, Vd, 0)
        for _ in range(warmup):
            hist()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for i in range(steps):
            evs[i][0].record()
            hist()
            evs[i][1].record()
        torch.cuda.synchronize()
        sh = _stats([e[0].elapsed_time(e[1]) * 1e-3 for e in evs])
        rec["quantize_history"] = dict(sh, tokens=Tn, mtok_s=round(Tn / (sh["median_us"] * 1e-6) / 1e6, 1))
        if name == "long_history":   # window keys: bound by HBM
            hbytes = Tn * H * (2 * D * 2 + D // 4 + D // 4 + (D // 32) * 4) + (Tn // 64) * H * D * 4
            rec["quantize_history"].update(
                effective_gbs=round(hbytes / (sh["median_us"] * 1e-6) / 1e9, 1),
                pct_hbm_peak=round(100 * hbytes / (sh["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
                bytes=hbytes)
        else:                        # centroid keys: the assignment's arithmetic
            rec["quantize_history"]["keys"] = desc["keys"]

    def step(ev=None):
        if tail0 is not None:
            cache.k_tail.copy_(tail0)
        if ev:
            ev[0].record()
        kv.attn_int2_chunk(cache, Tn, qd, scale, out=out, workspace=ws)
        if ev:
            ev[1].record()
        if Kn is not None:
            kv.kv_quantize_append(cache, Kn, Vn, Tn)
        if ev:
            ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sc = _stats([e[0].elapsed_time(e[1]) * 1e-3 for e in evs])
    flops = 4.0 * Lq * Tn * D * H
    tfs = flops / (sc["median_us"] * 1e-6) / 1e12
    tfs_mean = flops / (sc["mean_us"] * 1e-6) / 1e12
    rec.update({
        "ms_per_step": round(wall / steps * 1e3, 4), "steps": steps, "warmup": warmup,
        "chunk_attention": dict(sc, tflops=round(tfs, 2), pct_mfma_peak=round(100 * tfs / MFMA_PEAK_TFS, 2),
                                flops=flops),
        "roofline": {"kernel": "chunk_kernel (+ chunk_merge_kernel)", "bound": "mfma",
                     "achieved": round(tfs_mean, 2), "peak": MFMA_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": round(tfs_mean / MFMA_PEAK_TFS, 4),
                     "traffic": _counter_traffic(CHUNK_COUNTERS[name]), "time": "mean per call"}})
    if Kn is not None:
        sa = _stats([e[1].elapsed_time(e[2]) * 1e-3 for e in evs])
        rec["quantize_append"] = dict(sa, tokens=Lq, mtok_s=round(Lq / (sa["median_us"] * 1e-6) / 1e6, 2))
    host = {"d": d, "cent0": cache.centroids[0, 0].cpu().numpy() if kmeans_rounds else None,
            "kmeans_rounds": kmeans_rounds}
    del cache, Kd, Vd, qd, Kn, Vn, out, ws
    torch.cuda.empty_cache()
    return rec, host


def cpu_chunk_baseline(name: str, host) -> dict:
    """The oracle on head 0 of a chunk workload: its own calibration for that
    head (k-means from the same seeded picks; w and U from the calibration
    queries), the append of the head's history, then fp64 attention of the
    first CPU_CHUNK_ROWS query rows against all cached tokens.  value = the
    attention's TFLOP/s at the chunk's flop count for those rows."""
    import numpy as np

    import oracle
    import synth

    d = host["d"]
    Tn, Lq = d["T"], d["Lq"]
    R = min(CPU_CHUNK_ROWS, Lq)
    K = np.ascontiguousarray(d["K"][:, :, :1])
    V = np.ascontiguousarray(d["V"][:, :, :1])
    cap = ((Tn + 63) // 64) * 64
    t0 = time.perf_counter()
    if name == "long_history":
        o = oracle.Cache(1, 1, D, cap, oracle.KEY_WINDOW, oracle.VAL_GROUP)
    else:
        Kf = np.ascontiguousarray(synth.bf16_bits_to_f32(K)[0, :, 0])
        cent, _ = oracle.kmeans(Kf, 256, d["kmeans_init"][0, 0], host["kmeans_rounds"])
        if name == "video_chunk":
            o = oracle.Cache(1, 1, D, cap, oracle.KEY_CENTROID, oracle.VAL_HADAMARD, C=256)
        else:
            o = oracle.Cache(1, 1, D, cap, oracle.KEY_CENTROID_QSAC, oracle.VAL_HADAMARD, C=256,
                             topk=4, R=8)
            qc = synth.bf16_bits_to_f32(d["q_cal"])[:, 0].astype(np.float64)
            o.sens_w[0, 0] = oracle.sens_weights(qc)
            o.psac_basis[0, 0] = oracle.pca(qc, 8)[0]
        o.centroids[0, 0] = cent
    t_cal = time.perf_counter() - t0
    t0 = time.perf_counter()
    o.append(K, V, 0)
    t_app = time.perf_counter() - t0
    q = synth.bf16_bits_to_f32(np.ascontiguousarray(d["q"][:, :R, :1])).astype(np.float64)
    t0 = time.perf_counter()
    o.attention(q, Tn, 1.0 / math.sqrt(D))
    t_att = time.perf_counter() - t0
    flops = 4.0 * R * Tn * D
    return {"value": round(flops / t_att / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "quantize_mtok_s": round(Tn / t_app / 1e6 / d["Hkv"], 6),
            "sample": f"head 0 of {d['Hkv']}, query rows 0-{R - 1} of {Lq}, all {Tn} cached tokens: "
                      f"fp64 attention {t_att:.2f} s; append of the head's history {t_app:.2f} s "
                      f"(quantize_mtok_s scaled to {d['Hkv']} heads); calibration {t_cal:.2f} s untimed"}


KMEANS_SAMPLE_HEADS = 16   # oracle leg: this many heads, one round each


def kmeans_workload(steps: int, warmup: int, with_cpu: bool = True) -> dict:
    """Calibration: Lloyd rounds of kv_kmeans over the video workload's
    cached keys (40 heads x 31200 keys, 256 centroids, head_dim 128); one
    step = one round for every head (one call), each head starting from its
    picks.  The roofline is the assignment kernel's, timed on its own (a call
    with zero rounds is exactly one assignment launch)."""
    import numpy as np
    import torch

    import bit_kv_cache_int2_amd as kv
    import synth

    d = synth.video_chunk()
    H, T = d["Hkv"], d["T"]
    C = 256
    kd = torch.from_numpy(np.ascontiguousarray(d["K"]).view(np.int16)).view(torch.bfloat16).cuda()
    K = synth.bf16_bits_to_f32(d["K"])[0]
    Dh = K.shape[-1]
    init = torch.from_numpy(np.ascontiguousarray(
        np.stack([K[d["kmeans_init"][0, h], h] for h in range(H)]))).cuda()[None]   # [1][H][C][D]
    cent = init.clone()
    asg = torch.empty((1, H, T), dtype=torch.int32, device="cuda")
    ws = torch.empty(kv.lib().kv_kmeans_workspace(1, H, T), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def timed(fn, n):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record()
        for _ in range(n):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e-3 / n, time.perf_counter() - t0

    def step():    # one call: every head's round
        cent.copy_(init)
        kv.kv_kmeans(kd, cent, 1, assign_out=asg, workspace=ws)

    def assign_only():
        kv.kv_kmeans(kd, init, 0, assign_out=asg, workspace=ws)

    for _ in range(warmup):
        step()
        assign_only()
    t, wall = timed(step, steps)
    t_as, _ = timed(assign_only, steps)
    # the products k.c of every (key, centroid) pair, 2 flops each
    flops = 2.0 * H * T * C * Dh
    tfs = flops / t_as / 1e12
    rec = {"metric": "k-means round time (all heads)", "value": round(t * 1e6, 1), "unit": "us",
           "n_gpus": 1, "steps": steps, "warmup": warmup,
           "ms_per_step": round(wall / steps * 1e3, 4), "higher_is_better": False,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16+fp32", "data": "synthetic",
           "config": {"workload": "kmeans", "heads": H, "keys_per_head": T, "centroids": C,
                      "head_dim": Dh, "rule": "exact fp32 assignment, fp64 key-order means"},
           "kmeans": {"us_per_round": round(t * 1e6, 1), "assign_us": round(t_as * 1e6, 1),
                      "update_us": round((t - t_as) * 1e6, 1),
                      "g_key_assignments_s": round(H * T / t_as / 1e9, 3)},
           "roofline": {"kernel": "centroid_kernel", "bound": "mfma", "achieved": round(tfs, 2),
                        "peak": MFMA_PEAK_TFS, "unit": "TFLOP/s", "frac": round(tfs / MFMA_PEAK_TFS, 4),
                        "traffic": None}}
    if with_cpu:
        import oracle
        S = KMEANS_SAMPLE_HEADS
        t0 = time.perf_counter()
        for h in range(S):
            oracle.kmeans(np.ascontiguousarray(K[:, h]), C, d["kmeans_init"][0, h], 1)
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(dt * H / S * 1e6, 1), "unit": "us",
                               "cores": oracle.num_threads(), "kind": "oracle",
                               "sample": f"{S} of {H} heads, one round each ({T} keys, {C} centroids): "
                                         f"{dt:.2f} s, scaled to {H} heads"}
    return rec


def variants_workload(steps: int, warmup: int) -> dict:
    """The QuantWM variants side by side on the sensitivity-aware workload
    (40 heads, 65,536 cached tokens, 1,560 query rows, 256 centroids fitted
    by four kv_kmeans rounds from the seeded picks): plain centroid keys,
    QSAC with the exact and the range-based estimate, PSAC with fp16 and
    INT8 coefficients.  Per variant: cache bytes per token-head, append and
    chunk-attention time, and the attention error against fp32 attention
    over the unquantized bf16 keys and values (torch, sampled heads)."""
    import numpy as np
    import torch

    import bit_kv_cache_int2_amd as kv
    import synth

    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    d = synth.sensitivity_aware()
    H, T, Lq, C = d["Hkv"], d["T"], d["Lq"], 256
    Tcap = ((T + 63) // 64) * 64
    Kd, Vd, qd = to_dev(d["K"]), to_dev(d["V"]), to_dev(d["q"])
    scale = 1.0 / math.sqrt(D)
    # calibration inputs: centroids by GPU k-means, w and U from the calibration queries
    K = synth.bf16_bits_to_f32(d["K"])[0]
    cent = torch.from_numpy(np.ascontiguousarray(
        np.stack([K[d["kmeans_init"][0, h], h] for h in range(H)])[None])).cuda()
    kv.kv_kmeans(Kd, cent, 4)
    del K
    qc = synth.bf16_bits_to_f32(d["q_cal"]).astype(np.float64)
    w = torch.from_numpy((qc ** 2).mean(0).astype(np.float32)[None]).cuda()
    U = torch.from_numpy(np.ascontiguousarray(np.stack(
        [np.linalg.eigh(qc[:, h].T @ qc[:, h] / qc.shape[0])[1][:, ::-1][:, :8]
         for h in range(H)]).astype(np.float32)[None])).cuda()
    # reference: fp32 attention over the unquantized keys and values, and each
    # row's top-1 token (the first of the largest fp32 logit)
    heads = (0, 13, 27, 39)
    ref, ref_top = {}, {}
    for h in heads:
        q = qd[0, :, h].float()
        k = Kd[0, :, h].float().contiguous()
        v = Vd[0, :, h].float().contiguous()
        s_ = q @ k.t()
        ref_top[h] = torch.argmax(s_, dim=-1).to(torch.int32)
        p = torch.softmax(s_ * scale, dim=-1)
        ref[h] = p @ v
        del p, s_
    torch.cuda.synchronize()
    variants = [("centroid", kv.KEY_CENTROID, 0, kv.QSAC_EXACT, kv.PSAC_F16),
                ("qsac_exact", kv.KEY_CENTROID_QSAC, 0, kv.QSAC_EXACT, kv.PSAC_F16),
                ("qsac_range", kv.KEY_CENTROID_QSAC, 0, kv.QSAC_RANGE, kv.PSAC_F16),
                ("qsac_exact+psac_f16", kv.KEY_CENTROID_QSAC, 8, kv.QSAC_EXACT, kv.PSAC_F16),
                ("qsac_exact+psac_int8", kv.KEY_CENTROID_QSAC, 8, kv.QSAC_EXACT, kv.PSAC_INT8),
                ("qsac_range+psac_int8", kv.KEY_CENTROID_QSAC, 8, kv.QSAC_RANGE, kv.PSAC_INT8)]
    calib = ("centroids", "sens_w", "psac_basis")

    def timed(fn, n):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(n):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e-3 / n

    out = torch.empty((1, Lq, H, D), dtype=torch.float32, device="cuda")
    table = {}
    t0 = time.perf_counter()
    for name, mode, R, score, fmt in variants:
        c = kv.KVCache(1, H, D, Tcap, key_mode=mode, n_centroids=C, qsac_topk=4, psac_rank=R,
                       value_mode=kv.VAL_HADAMARD, qsac_score=score, psac_format=fmt)
        c.centroids.copy_(cent)
        if c.sens_w is not None:
            c.sens_w.copy_(w)
        if c.psac_basis is not None:
            c.psac_basis.copy_(U)
        app = lambda: kv.kv_quantize_append(c, Kd, Vd, 0)
        att = lambda: kv.attn_int2_chunk(c, T, qd, scale, out=out)
        for _ in range(warmup):
            app()
            att()
        t_app = timed(app, steps)
        t_att = timed(att, steps)
        # attention shift: rows whose top-1 cached token differs from bf16's
        top = kv.attn_int2_top1(c, T, qd)
        torch.cuda.synchronize()
        shifted = sum(int((top[0, h] != ref_top[h]).sum().item()) for h in heads)
        err_max, num, den, abs_sum, cnt = 0.0, 0.0, 0.0, 0.0, 0
        for h in heads:
            dlt = out[0, :, h] - ref[h]
            err_max = max(err_max, dlt.abs().max().item())
            num += (dlt * dlt).sum().item()
            den += (ref[h] * ref[h]).sum().item()
            abs_sum += dlt.abs().sum().item()
            cnt += dlt.numel()
        cache_bytes = sum(t.numel() * t.element_size() for n_, t in c.buffers.items() if n_ not in calib)
        table[name] = {"bytes_per_token_head": round(cache_bytes / (H * Tcap), 2),
                       "compression_vs_bf16": round(512 * H * Tcap / cache_bytes, 3),
                       "append_us": round(t_app * 1e6, 1), "chunk_us": round(t_att * 1e6, 1),
                       "attn_err_max": float(f"{err_max:.4g}"),
                       "attn_err_mean": float(f"{abs_sum / cnt:.4g}"),
                       "attn_rel_l2": float(f"{math.sqrt(num / den):.4g}"),
                       "top1_shift_pct": round(100.0 * shifted / (len(heads) * Lq), 2)}
        del c
        torch.cuda.empty_cache()
    wall = time.perf_counter() - t0
    best = table["qsac_range+psac_int8"]
    return {"metric": "INT2 cache variants: attention rel. L2 error vs bf16 (QSAC range + INT8 PSAC)",
            "value": best["attn_rel_l2"], "unit": "rel_l2", "n_gpus": 1, "steps": steps,
            "warmup": warmup, "ms_per_step": round(wall / (steps * len(variants)) * 1e3, 4),
            "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
            "data": "synthetic",
            "config": {"workload": "variants", "heads": H, "head_dim": D, "context": T, "q_len": Lq,
                       "centroids": "256 per head, 4 GPU k-means rounds from the seeded picks",
                       "values": "Walsh-Hadamard rotated, int2 per token, groups of 32",
                       "error_reference": "fp32 attention over the bf16 keys/values, heads "
                                          + ",".join(map(str, heads)) + ", all query rows",
                       "top1_shift": "share of those rows whose highest-logit cached token "
                                     "differs from the bf16 one"},
            "variants": table}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="all",
                    choices=["all", "llm_decode", "toy", "long_history", "video_chunk", "sensitivity",
                             "kmeans", "variants", "copy"])
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the path has no multi-GPU leg "
              "(each GPU would hold whole heads or sequences of the cache); run with --gpus 1",
              file=sys.stderr)
        return 2
    if args.workload == "copy":
        return copy_calibration(args.steps)
    import torch
    torch.cuda.set_device(0)
    with_cpu = not args.no_cpu_baseline
    if args.workload == "kmeans":
        print(json.dumps(kmeans_workload(args.steps, args.warmup, with_cpu)), flush=True)
        return 0
    if args.workload == "variants":
        print(json.dumps(variants_workload(args.steps, args.warmup)), flush=True)
        return 0
    if args.workload in ("toy", "long_history", "video_chunk", "sensitivity"):
        if args.workload == "toy":
            rec = toy_leg(args.steps, args.warmup, with_cpu)
        else:
            rec, host = chunk_leg(args.workload, args.steps, args.warmup)
            if with_cpu:
                rec["cpu_baseline"] = cpu_chunk_baseline(args.workload, host)
        print(json.dumps(rec), flush=True)
        return 0

    # the default line: the chunk workloads and the toy first (GPU work at
    # full clocks before the decode line is timed), then the decode line,
    # then the oracle legs on the host cores
    legs, hosts = {}, {}
    if args.workload == "all":
        legs["toy_single_head"] = toy_leg(args.steps, args.warmup, False)
        for name in ("video_chunk", "long_history", "sensitivity"):
            legs[name], hosts[name] = chunk_leg(name, args.steps, args.warmup)
    rec, d = decode_leg(args.steps, args.warmup)
    rec.update(legs)
    if args.workload == "all":
        # the measured denominators beside the vendor peaks of each roofline
        peaks = measured_peaks()
        rec["peaks_measured"] = peaks
        for r in [rec] + [v for v in legs.values() if isinstance(v, dict)]:
            for key in ("roofline", "roofline_append"):
                roof = r.get(key)
                if isinstance(roof, dict):
                    m = peaks["hbm_gbs"] if roof["bound"] == "hbm" else peaks["mfma_fp16_tflops"]
                    roof["peak_measured"] = m
                    roof["frac_of_measured"] = round(roof["achieved"] / m, 4)
        rec["generator"] = _generator_constants()
    if with_cpu:
        t0 = time.perf_counter()
        rec["cpu_baseline"] = cpu_decode_baseline(d)
        if "toy_single_head" in rec:
            import synth
            rec["toy_single_head"]["cpu_baseline"] = cpu_toy_baseline(synth.toy_single_head())
        for name, host in hosts.items():
            rec[name]["cpu_baseline"] = cpu_chunk_baseline(name, host)
        host_info = {"cpu_model": _cpu_model(), "nproc": os.cpu_count()}
        for r in [rec] + [v for v in legs.values() if isinstance(v, dict)]:
            if isinstance(r.get("cpu_baseline"), dict):
                r["cpu_baseline"].update(host_info)
        print(f"oracle legs: {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
