"""Seeded random configurations through the whole path: quantize-append in
one to three calls, decode and chunk attention, against the oracle.  Each
case draws the key mode (window, centroid, QSAC with the exact or the range
estimate), the value mode (plain, rotated, or rotated per modality with
one to three modalities), head_dim 64 / 128, PSAC off /
fp16 / INT8, batch, heads, GQA, the centroid count (1 .. 256), ragged
lengths and capacities, and the query dtype.  Caches must match bit for bit;
attention within 2e-3.  A draw that failed once is fixed in the code, not
dropped from the list: case 13 (nine copies of a centroid in a 256-entry
table overflowing the QSAC shortlist) is the tie-order regression of the
exact scan."""
import math
import os

import numpy as np
import pytest
import torch

import bit_kv_cache_int2_amd as kv
import oracle
import synth
from gpu_helpers import TOL, assert_cache_equal, dev_bf16, oracle_like, to_oracle

pytestmark = pytest.mark.gpu

CASES = int(os.environ.get("KVQ_SWEEP_CASES", "300"))   # more for a deeper one-off sweep


def _draw(case: int, seed0: int = 9000, t_range=(1, 700), lq_range=(1, 150), g_choices=(1, 2, 4)):
    r = np.random.default_rng(seed0 + case)
    cfg = dict(D=int(r.choice([64, 128])), key_mode=int(r.integers(0, 3)),
               value_mode=int(r.integers(0, 3)), B=int(r.integers(1, 3)), H=int(r.integers(1, 4)),
               G=int(r.choice(list(g_choices))), T=int(r.integers(*t_range)))
    cfg["cap_extra"] = int(r.integers(0, 2)) * 64
    centroid = cfg["key_mode"] != kv.KEY_WINDOW
    cfg["C"] = int(r.choice([1, 5, 32, 256])) if centroid else 0
    cfg["topk"] = min(4, cfg["C"]) if cfg["key_mode"] == kv.KEY_CENTROID_QSAC else 1
    cfg["R"] = 8 if centroid and r.random() < 0.5 else 0
    cfg["fmt"] = kv.PSAC_INT8 if cfg["R"] and r.random() < 0.5 else kv.PSAC_F16
    cfg["score"] = kv.QSAC_RANGE if cfg["key_mode"] == kv.KEY_CENTROID_QSAC and r.random() < 0.5 else kv.QSAC_EXACT
    cuts = sorted(r.choice(np.arange(1, cfg["T"]), size=min(int(r.integers(0, 3)), cfg["T"] - 1), replace=False)) \
        if cfg["T"] > 1 else []
    cfg["chunks"] = [int(x) for x in np.diff([0] + [int(x) for x in cuts] + [cfg["T"]])]
    cfg["Lq"] = int(r.integers(*lq_range))
    cfg["q_f32"] = bool(r.random() < 0.5)
    cfg["split"] = bool(centroid and r.random() < 0.5)
    cfg["M"] = int(r.integers(1, 4)) if cfg["value_mode"] == kv.VAL_HADAMARD_MODAL else 1
    return cfg, r


@pytest.mark.parametrize("case", range(CASES))
def test_random_configuration(case):
    _run(*_draw(case), f"case {case}")


@pytest.mark.parametrize("case", range(24))
def test_random_long_configuration(case):
    """Longer caches (700 to 6,000 tokens) and 100 to 600 query rows: decode
    over many token splits and chunk attention over several row blocks and
    token splits, so the split merges see random shapes too.  Chunk rows are
    sampled (every fifth row and the last) to bound the oracle's time."""
    cfg, r = _draw(case, seed0=19000, t_range=(700, 6000), lq_range=(100, 600), g_choices=(1, 2, 4, 8))
    _run(cfg, r, f"long case {case}", chunk_rows=slice(None, None, 5))


@pytest.mark.parametrize("case", range(20))
def test_random_streaming_appends(case):
    """Tokens arrive a few at a time (1 to 17 per call, as in decoding or a
    frame arriving in pieces): every call lands in a partly filled value
    tile and window, through the merge with earlier codes and the key
    tail; the cache must still equal the oracle's bit for bit."""
    cfg, r = _draw(case, seed0=27000, t_range=(60, 400))
    sizes = []
    while sum(sizes) < cfg["T"]:
        sizes.append(int(min(r.integers(1, 18), cfg["T"] - sum(sizes))))
    cfg["chunks"] = sizes
    _run(cfg, r, f"streaming case {case}")


def _run(cfg, r, name, chunk_rows=None):
    D, B, H, T, G = cfg["D"], cfg["B"], cfg["H"], cfg["T"], cfg["G"]
    Hq = H * G
    tag = f"{name}: {cfg}"
    # keys: per-channel scales to 5 and offsets of sd 1.5 (rms about 2.4,
    # peaks near 20) for every key mode, so window ranges and centroid
    # residuals both see spread; values at 0.5 to 2 times unit scale
    # (peaks to about 9)
    sc = np.exp(r.uniform(np.log(0.2), np.log(5.0), (1, 1, H, D)))
    off = r.normal(0, 1.5, (1, 1, H, D))
    K = synth.to_bf16_bits((r.standard_normal((B, T, H, D)) * sc + off).astype(np.float32))
    V = synth.to_bf16_bits((r.standard_normal((B, T, H, D)) * r.uniform(0.5, 2.0)).astype(np.float32))
    cap = ((T + 63) // 64) * 64 + cfg["cap_extra"]
    c = kv.KVCache(B, H, D, cap, key_mode=cfg["key_mode"], value_mode=cfg["value_mode"],
                   n_centroids=cfg["C"], qsac_topk=cfg["topk"], psac_rank=cfg["R"],
                   qsac_score=cfg["score"], psac_format=cfg["fmt"], centroid_key_split=cfg["split"],
                   n_modalities=cfg["M"])
    if c.v_signs is not None:          # per-modality rotations: random signs and modality runs
        c.v_signs.copy_(torch.from_numpy(
            r.integers(0, 1 << 32, size=(H, cfg["M"], D // 32), dtype=np.uint64).astype(np.uint32).view(np.int32)))
        runs = np.repeat(r.integers(0, cfg["M"], size=cap // 16 + 1), 16)[:cap]
        c.v_modality.copy_(torch.from_numpy(np.tile(runs.astype(np.uint8), (B, 1))))
    if c.centroids is not None:        # calibration inputs: keys picked at random, weights, a basis
        Kf = synth.bf16_bits_to_f32(K)
        cent = np.stack([np.stack([Kf[b, r.integers(0, T, cfg["C"]), h] for h in range(H)])
                         for b in range(B)])
        c.centroids.copy_(torch.from_numpy(np.ascontiguousarray(cent, np.float32)))
    if c.sens_w is not None:
        c.sens_w.copy_(torch.from_numpy(r.uniform(0.1, 3.0, (B, H, D)).astype(np.float32)))
    if c.psac_basis is not None:
        U = np.stack([np.stack([np.linalg.qr(r.standard_normal((D, 8)))[0] for _ in range(H)])
                      for _ in range(B)])
        c.psac_basis.copy_(torch.from_numpy(np.ascontiguousarray(U, np.float32)))
    o = oracle_like(c)
    pos = 0
    for n in cfg["chunks"]:
        k, v = np.ascontiguousarray(K[:, pos:pos + n]), np.ascontiguousarray(V[:, pos:pos + n])
        kv.kv_quantize_append(c, dev_bf16(k), dev_bf16(v), pos)
        o.append(k, v, pos)
        pos += n
    torch.cuda.synchronize()
    g = to_oracle(c)
    assert_cache_equal(g, o, T, tag)
    scale = 1.0 / math.sqrt(D)

    # decode: one query per sequence and query head
    qd = r.standard_normal((B, Hq, D)).astype(np.float32)
    if cfg["q_f32"]:
        q_dev, q64 = torch.from_numpy(qd).cuda(), qd.astype(np.float64)
    else:
        qb = synth.to_bf16_bits(qd)
        q_dev, q64 = dev_bf16(qb), synth.bf16_bits_to_f32(qb).astype(np.float64)
    out = kv.attn_int2_decode(c, T, q_dev, scale)
    torch.cuda.synchronize()
    ref, _ = g.attention(q64.reshape(B, 1, Hq, D), T, scale)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref[:, 0])
    assert np.all(err <= TOL), f"{tag}: decode max err {err.max():.3e}"

    # chunk: Lq query rows per sequence
    Lq = cfg["Lq"]
    qc = synth.to_bf16_bits(r.standard_normal((B, Lq, Hq, D)).astype(np.float32))
    outc = kv.attn_int2_chunk(c, T, dev_bf16(qc), scale)
    torch.cuda.synchronize()
    rows = np.arange(Lq) if chunk_rows is None else np.unique(np.r_[np.arange(Lq)[chunk_rows], Lq - 1])
    refc, _ = g.attention(np.ascontiguousarray(synth.bf16_bits_to_f32(qc[:, rows]).astype(np.float64)), T, scale)
    errc = np.abs(outc.cpu().numpy()[:, rows].astype(np.float64) - refc)
    assert np.all(errc <= TOL), f"{tag}: chunk max err {errc.max():.3e}"
