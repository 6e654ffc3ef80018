"""GPU parity of attn_int2_decode: the output (fp32) must be within 2e-3
(max |delta|) of the oracle's fp64 attention over the same packed cache,
whose bytes are first checked bit-exact against the oracle's own."""
import math

import numpy as np
import pytest
import torch

import bit_kv_cache_int2_amd as kv
import oracle
import synth
from gpu_helpers import TOL, assert_cache_equal, calibrate, dev_bf16, oracle_like, to_oracle

pytestmark = pytest.mark.gpu


def _decode_check(c, o, n, q_dev, q64, scale, tag, out_dtype=torch.float32):
    lse = torch.empty(q_dev.shape[0] * q_dev.shape[1], dtype=torch.float32, device="cuda")
    out = kv.attn_int2_decode(c, n, q_dev, scale, out_dtype=out_dtype, lse=lse)
    torch.cuda.synchronize()
    g = to_oracle(c)
    assert_cache_equal(g, o, n, tag)
    B, Hq, D = q_dev.shape
    ref, rlse = g.attention(q64.reshape(B, 1, Hq, D), n, scale)
    got = out.float().cpu().numpy().astype(np.float64)
    tol = TOL
    if out_dtype == torch.bfloat16:                       # + half a bf16 ulp of the output
        tol = TOL + np.abs(ref[:, 0]) * 2.0 ** -8
    err = np.abs(got - ref[:, 0])
    assert np.all(err <= tol), f"{tag}: max err {err.max():.3e}"
    lerr = np.abs(lse.cpu().numpy().reshape(B, Hq) - rlse[:, :, 0]).max()
    assert lerr < 1e-3, f"{tag}: lse err {lerr}"
    return out, float(err.max())


def test_toy_single_head_decode():
    d = synth.toy_single_head()
    c = kv.KVCache(1, 1, 64, 512, key_mode=kv.KEY_CENTROID, n_centroids=16)
    calibrate(c, d["K"], d["kmeans_init"], 4)
    o = oracle_like(c)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    o.append(d["K"], d["V"], 0)
    q = torch.from_numpy(d["q"]).cuda()                  # fp32 [1][1][64]
    _decode_check(c, o, 512, q, d["q"].astype(np.float64), 0.125, "toy")
    # ragged lengths inside the cache
    for n in (1, 63, 64, 65, 300):
        _decode_check(c, o, n, q, d["q"].astype(np.float64), 0.125, f"toy n={n}")


@pytest.mark.parametrize("T", [1, 40, 64, 65, 1000, 2047])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_window_decode_lengths_and_groups(T, G):
    H = 2
    d = synth.llm_decode(B=2, Hkv=H, Hq=H * G, D=128, T=T)
    c = kv.KVCache(2, H, 128, 2048)
    o = oracle_like(c)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    o.append(d["K"], d["V"], 0)
    qd = dev_bf16(d["q"])
    q64 = synth.bf16_bits_to_f32(d["q"]).astype(np.float64)
    _decode_check(c, o, T, qd, q64, 1 / math.sqrt(128), f"T={T} G={G}")


def test_window_decode_bf16_output_and_determinism():
    d = synth.llm_decode(B=3, Hkv=2, Hq=8, D=128, T=1500)
    c = kv.KVCache(3, 2, 128, 1536)
    o = oracle_like(c)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    o.append(d["K"], d["V"], 0)
    qd = dev_bf16(d["q"])
    q64 = synth.bf16_bits_to_f32(d["q"]).astype(np.float64)
    a, _ = _decode_check(c, o, 1500, qd, q64, 1 / math.sqrt(128), "f32")
    b, _ = _decode_check(c, o, 1500, qd, q64, 1 / math.sqrt(128), "bf16", torch.bfloat16)
    a2 = kv.attn_int2_decode(c, 1500, qd, 1 / math.sqrt(128))
    torch.cuda.synchronize()
    assert torch.equal(a, a2)


def test_window_decode_reused_workspace():
    """Rotated values with window keys against the oracle, then one
    workspace reused across calls of different lengths: every call matches
    a call on a fresh workspace bit for bit."""
    d = synth.llm_decode(B=2, Hkv=2, Hq=8, D=128, T=3000)
    c = kv.KVCache(2, 2, 128, 3008, value_mode=kv.VAL_HADAMARD)
    o = oracle_like(c)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    o.append(d["K"], d["V"], 0)
    qd = dev_bf16(d["q"])
    q64 = synth.bf16_bits_to_f32(d["q"]).astype(np.float64)
    _decode_check(c, o, 3000, qd, q64, 1 / math.sqrt(128), "rotated values")
    ws = kv.decode_workspace(c, 8, 3000)
    for n in (3000, 700, 64, 3000, 1999):
        lse_a = torch.empty(16, dtype=torch.float32, device="cuda")
        lse_b = torch.empty(16, dtype=torch.float32, device="cuda")
        a = kv.attn_int2_decode(c, n, qd, 1 / math.sqrt(128), lse=lse_a, workspace=ws)
        b = kv.attn_int2_decode(c, n, qd, 1 / math.sqrt(128), lse=lse_b)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"n={n}"
        assert torch.equal(lse_a, lse_b), f"n={n}"


@pytest.mark.parametrize("mode,R,had,fmt", [(kv.KEY_CENTROID, 0, True, 0), (kv.KEY_CENTROID_QSAC, 8, True, 0),
                                            (kv.KEY_CENTROID_QSAC, 8, False, 0),
                                            (kv.KEY_CENTROID_QSAC, 8, True, kv.PSAC_INT8)])
def test_centroid_decode_psac_hadamard(mode, R, had, fmt):
    d = synth.sensitivity_aware(H=2, T=900, Lq=4, C=32, n_cal=256)
    c = kv.KVCache(1, 2, 128, 960, key_mode=mode, n_centroids=32, qsac_topk=4, psac_rank=R,
                   value_mode=kv.VAL_HADAMARD if had else kv.VAL_GROUP,
                   qsac_score=kv.QSAC_RANGE if fmt else kv.QSAC_EXACT, psac_format=fmt)
    calibrate(c, d["K"], d["kmeans_init"], 2, d["q_cal"])
    o = oracle_like(c)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    o.append(d["K"], d["V"], 0)
    qbits = np.ascontiguousarray(d["q"][0, :2])           # two query heads per kv head
    qbits = np.ascontiguousarray(qbits.transpose(1, 0, 2).reshape(1, 4, 128))
    # query head 2h+g -> kv head h: heads (0,1) use q rows of kv head 0 ...
    q64 = synth.bf16_bits_to_f32(qbits).astype(np.float64)
    _decode_check(c, o, 900, dev_bf16(qbits), q64, 1 / math.sqrt(128), f"mode={mode} R={R} fmt={fmt}")


@pytest.mark.slow
def test_llm_decode_full_size_sampled():
    """B=16, 32 query / 8 KV heads, 32768 cached tokens: the benchmark's
    launch configuration; cache bytes and outputs of sampled (sequence, kv
    head) groups checked against the oracle."""
    d = synth.llm_decode()
    B, H, Hq, T = d["B"], d["Hkv"], d["Hq"], d["T"]
    c = kv.KVCache(B, H, 128, T)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    qd = dev_bf16(d["q"])
    out = kv.attn_int2_decode(c, T, qd, 1 / math.sqrt(128))
    torch.cuda.synchronize()
    g = to_oracle(c)
    got = out.cpu().numpy()
    q64 = synth.bf16_bits_to_f32(d["q"]).astype(np.float64)
    worst = 0.0
    for b, h in [(0, 0), (5, 2), (15, 7), (9, 4)]:
        o = oracle.Cache(1, 1, 128, T)
        o.append(np.ascontiguousarray(d["K"][b:b + 1, :, h:h + 1]),
                 np.ascontiguousarray(d["V"][b:b + 1, :, h:h + 1]), 0)
        gs = g.slice_bh(b, h)
        assert_cache_equal(gs, o, T, f"b={b} h={h}")
        qs = q64[b:b + 1, 4 * h:4 * h + 4].reshape(1, 1, 4, 128)
        ref, _ = gs.attention(np.ascontiguousarray(qs), T, 1 / math.sqrt(128))
        err = np.abs(got[b, 4 * h:4 * h + 4] - ref[0, 0]).max()
        worst = max(worst, err)
        assert err <= TOL, f"b={b} h={h} err {err}"
    print(f"full-size decode worst |delta| {worst:.3e}")
