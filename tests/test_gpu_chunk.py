"""GPU parity of attn_int2_chunk (MFMA chunk attention over the packed
cache): every output within 2e-3 (max |delta|) of the oracle's fp64
attention over the same cache, after the cache bytes matched the oracle's."""
import math

import numpy as np
import pytest
import torch

import bit_kv_cache_int2_amd as kv
import oracle
import synth
from gpu_helpers import TOL, assert_cache_equal, calibrate, dev_bf16, oracle_like, to_oracle

pytestmark = pytest.mark.gpu


def _chunk_check(c, o, n, q_bits, tag, rows=None, out_dtype=torch.float32, check_cache=True):
    B, Lq, Hq, D = q_bits.shape
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device="cuda")
    out = kv.attn_int2_chunk(c, n, dev_bf16(q_bits), 1 / math.sqrt(D), out_dtype=out_dtype, lse=lse)
    torch.cuda.synchronize()
    g = to_oracle(c)
    if check_cache:
        assert_cache_equal(g, o, n, tag)
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    q64 = synth.bf16_bits_to_f32(q_bits[:, rows]).astype(np.float64)
    ref, rlse = g.attention(np.ascontiguousarray(q64), n, 1 / math.sqrt(D))
    got = out.float().cpu().numpy()[:, rows].astype(np.float64)
    tol = TOL + (np.abs(ref) * 2.0 ** -8 if out_dtype == torch.bfloat16 else 0.0)
    err = np.abs(got - ref)
    assert np.all(err <= tol), f"{tag}: max err {err.max():.3e}"
    lerr = np.abs(lse.cpu().numpy()[:, :, rows] - rlse).max()
    assert lerr < 1e-3, f"{tag}: lse err {lerr}"
    return float(err.max())


@pytest.mark.parametrize("T,Lq", [(64, 1), (1000, 130), (2047, 300), (1, 5), (130, 129)])
@pytest.mark.parametrize("G", [1, 4])
def test_window_chunk(T, Lq, G):
    H = 2
    d = synth.long_history(H=H, T=T, Lq=Lq)
    c = kv.KVCache(1, H, 128, 2048)
    o = oracle_like(c)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    o.append(d["K"], d["V"], 0)
    q = np.repeat(d["q"], G, axis=2) if G > 1 else d["q"]
    _chunk_check(c, o, T, np.ascontiguousarray(q), f"T={T} Lq={Lq} G={G}")


@pytest.mark.parametrize("mode,R,had,fmt", [(kv.KEY_CENTROID, 0, True, 0), (kv.KEY_CENTROID, 0, False, 0),
                                            (kv.KEY_CENTROID_QSAC, 8, True, 0),
                                            (kv.KEY_CENTROID_QSAC, 8, True, kv.PSAC_INT8)])
def test_centroid_chunk(mode, R, had, fmt):
    d = synth.sensitivity_aware(H=2, T=1000, Lq=200, C=64, n_cal=256)
    c = kv.KVCache(1, 2, 128, 1024, key_mode=mode, n_centroids=64, qsac_topk=4, psac_rank=R,
                   value_mode=kv.VAL_HADAMARD if had else kv.VAL_GROUP,
                   qsac_score=kv.QSAC_RANGE if fmt else kv.QSAC_EXACT, psac_format=fmt)
    calibrate(c, d["K"], d["kmeans_init"], 2, d["q_cal"])
    o = oracle_like(c)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    o.append(d["K"], d["V"], 0)
    _chunk_check(c, o, 1000, d["q"], f"mode={mode} R={R} had={had} fmt={fmt}")


@pytest.mark.parametrize("D,C", [(64, 1), (128, 256)])
@pytest.mark.parametrize("mode", [kv.KEY_WINDOW, kv.KEY_CENTROID, kv.KEY_CENTROID_QSAC])
@pytest.mark.parametrize("vscale", [2.0, 2.5])
def test_chunk_large_keys_and_values(D, C, mode, vscale):
    """Keys far above unit rms (per-channel scales to 5, offsets of sd 1.5:
    rms about 2.4, peaks near 20) and values with peaks of 8 to 12, for
    every key mode: within 2e-3 of the oracle's exact attention over the
    same cache.  Keys enter the MFMAs as fp16 hi + lo; values centred on
    their group midpoint, whose sums come out exact."""
    rng = np.random.default_rng(31 + D + 7 * mode)
    B, H, G, T, Lq = 1, 2, 2, 391, 144
    sc = np.exp(rng.uniform(np.log(0.2), np.log(5.0), (1, 1, H, D)))
    off = rng.normal(0, 1.5, (1, 1, H, D))
    K = synth.to_bf16_bits((rng.standard_normal((B, T, H, D)) * sc + off).astype(np.float32))
    V = synth.to_bf16_bits((rng.standard_normal((B, T, H, D)) * vscale).astype(np.float32))
    assert np.abs(synth.bf16_bits_to_f32(V)).max() > 7.5
    centroid = mode != kv.KEY_WINDOW
    c = kv.KVCache(B, H, D, 448, key_mode=mode, n_centroids=C if centroid else 0,
                   qsac_topk=min(4, C), psac_rank=8 if mode == kv.KEY_CENTROID_QSAC else 0,
                   value_mode=kv.VAL_GROUP)
    Kf = synth.bf16_bits_to_f32(K)
    if centroid:
        c.centroids.copy_(torch.from_numpy(np.ascontiguousarray(
            np.stack([[Kf[0, rng.integers(0, T, C), h] for h in range(H)]]), np.float32)))
    if c.sens_w is not None:
        c.sens_w.copy_(torch.from_numpy(rng.uniform(0.1, 3.0, (B, H, D)).astype(np.float32)))
    if c.psac_basis is not None:
        c.psac_basis.copy_(torch.from_numpy(np.ascontiguousarray(np.stack(
            [[np.linalg.qr(rng.standard_normal((D, 8)))[0] for _ in range(H)]]), np.float32)))
    o = oracle_like(c)
    kv.kv_quantize_append(c, dev_bf16(K), dev_bf16(V), 0)
    o.append(K, V, 0)
    q = synth.to_bf16_bits(rng.standard_normal((B, Lq, H * G, D)).astype(np.float32))
    _chunk_check(c, o, T, q, f"D={D} C={C} mode={mode} vscale={vscale}")


def test_centroid_chunk_ignores_rows_past_the_length():
    """Index rows past the cached length are unspecified; filled with 255
    (beyond the 32 centroids) they must change nothing in the ragged tile."""
    d = synth.video_chunk(H=2, T=1000, Lq=70, C=32)
    c = kv.KVCache(1, 2, 128, 1088, key_mode=kv.KEY_CENTROID, n_centroids=32,
                   value_mode=kv.VAL_HADAMARD)
    calibrate(c, d["K"], d["kmeans_init"], 1)
    o = oracle_like(c)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    o.append(d["K"], d["V"], 0)
    c.k_idx[:, :, 1000:] = 255
    _chunk_check(c, o, 1000, d["q"], "stale indices past the length", check_cache=False)


def test_chunk_bf16_out_and_determinism():
    d = synth.video_chunk(H=2, T=700, Lq=150, C=32)
    c = kv.KVCache(1, 2, 128, 704, key_mode=kv.KEY_CENTROID, n_centroids=32,
                   value_mode=kv.VAL_HADAMARD)
    calibrate(c, d["K"], d["kmeans_init"], 1)
    o = oracle_like(c)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    o.append(d["K"], d["V"], 0)
    _chunk_check(c, o, 700, d["q"], "bf16 out", out_dtype=torch.bfloat16)
    qd = dev_bf16(d["q"])
    a = kv.attn_int2_chunk(c, 700, qd, 0.1)
    b = kv.attn_int2_chunk(c, 700, qd, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _sample_rows(Lq):
    r = set(range(0, Lq, max(1, Lq // 40))) | {Lq - 1, Lq - 2, 127, 128}
    return sorted(x for x in r if 0 <= x < Lq)


@pytest.mark.slow
def test_long_history_full_size_sampled():
    """40 heads, 93600 cached tokens (1462 windows + 32-token tail), a
    1560-row query frame; sampled heads and rows against the oracle."""
    d = synth.long_history()
    H, T, Lq = d["Hkv"], d["T"], d["Lq"]
    c = kv.KVCache(1, H, 128, ((T + Lq + 63) // 64) * 64)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    torch.cuda.synchronize()
    rows = _sample_rows(Lq)
    worst = 0.0
    g = to_oracle(c)
    for h in (0, 17, 39):
        o = oracle.Cache(1, 1, 128, c.layout.capacity)
        o.append(np.ascontiguousarray(d["K"][:, :, h:h + 1]), np.ascontiguousarray(d["V"][:, :, h:h + 1]), 0)
        assert_cache_equal(g.slice_bh(0, h), o, T, f"h={h}")
    out = kv.attn_int2_chunk(c, T, dev_bf16(d["q"]), 1 / math.sqrt(128)).cpu().numpy()
    for h in (0, 17, 39):
        gs = g.slice_bh(0, h)
        q64 = synth.bf16_bits_to_f32(d["q"][:, rows, h:h + 1]).astype(np.float64)
        ref, _ = gs.attention(np.ascontiguousarray(q64), T, 1 / math.sqrt(128))
        err = np.abs(out[:, rows, h:h + 1] - ref).max()
        worst = max(worst, err)
        assert err <= TOL, f"h={h} err {err}"
    print(f"long-history chunk worst |delta| {worst:.3e}")


@pytest.mark.slow
@pytest.mark.parametrize("which", ["video", "sensitivity"])
def test_centroid_workloads_full_size_sampled(which):
    """Video chunk (31200 cached, 4680 queries, 256 centroids, rotated
    values) and the sensitivity-aware variant (65536 cached, 1560 queries,
    QSAC top-4, PSAC rank 8): sampled heads and rows."""
    if which == "video":
        d = synth.video_chunk()
        c = kv.KVCache(1, d["Hkv"], 128, ((d["T"] + 63) // 64) * 64, key_mode=kv.KEY_CENTROID,
                       n_centroids=256, value_mode=kv.VAL_HADAMARD)
        calibrate(c, d["K"], d["kmeans_init"], 0)
    else:
        d = synth.sensitivity_aware()
        c = kv.KVCache(1, d["Hkv"], 128, ((d["T"] + 63) // 64) * 64, key_mode=kv.KEY_CENTROID_QSAC,
                       n_centroids=256, qsac_topk=4, psac_rank=8, value_mode=kv.VAL_HADAMARD)
        calibrate(c, d["K"], d["kmeans_init"], 0, d["q_cal"])
    T, Lq = d["T"], d["Lq"]
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    out = kv.attn_int2_chunk(c, T, dev_bf16(d["q"]), 1 / math.sqrt(128)).cpu().numpy()
    g = to_oracle(c)
    rows = _sample_rows(Lq)
    for h in (3, 38):
        gs = g.slice_bh(0, h)
        o = oracle.Cache(1, 1, 128, gs.Tcap, gs.key_mode, gs.value_mode, gs.C, gs.topk, gs.R,
                         centroids=gs.centroids.copy(), sens_w=gs.sens_w.copy(),
                         psac_basis=gs.psac_basis.copy())
        o.append(np.ascontiguousarray(d["K"][:, :, h:h + 1]), np.ascontiguousarray(d["V"][:, :, h:h + 1]), 0)
        assert_cache_equal(gs, o, T, f"{which} h={h}")
        q64 = synth.bf16_bits_to_f32(d["q"][:, rows, h:h + 1]).astype(np.float64)
        ref, _ = gs.attention(np.ascontiguousarray(q64), T, 1 / math.sqrt(128))
        err = np.abs(out[:, rows, h:h + 1] - ref).max()
        assert err <= TOL, f"{which} h={h} err {err}"
