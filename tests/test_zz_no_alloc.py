"""attn_int2_decode_noalloc (the allocation-free decode: split partials in
the library's fixed per-device scratch buffer) against attn_int2_decode
(caller workspace) through the C ABI: bit-identical outputs and lse, and
within 2e-3 of the oracle, on two calls in a row, the second smaller, so
partials the first call left in the scratch buffer must not leak into the
second."""
import math

import numpy as np
import pytest
import torch

import bit_kv_cache_int2_amd as kv
import synth
from gpu_helpers import TOL, calibrate, dev_bf16, to_oracle

pytestmark = pytest.mark.gpu


def _window_cache(B, H, G, T, seed_T=None):
    d = synth.llm_decode(B=B, Hkv=H, Hq=H * G, D=128, T=T)
    c = kv.KVCache(B, H, 128, ((T + 63) // 64) * 64)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    return c, d["q"]


def _centroid_cache(T):
    d = synth.video_chunk(H=2, T=T, Lq=1, C=32)
    c = kv.KVCache(1, 2, 128, ((T + 63) // 64) * 64, key_mode=kv.KEY_CENTROID, n_centroids=32,
                   value_mode=kv.VAL_HADAMARD)
    calibrate(c, d["K"], d["kmeans_init"], 1)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    q = synth.to_bf16_bits(np.random.default_rng(T).standard_normal((1, 4, 128)).astype(np.float32))
    return c, q


def _both(c, n, q_bits, tag):
    qd = dev_bf16(q_bits)
    B, Hq, D = qd.shape
    scale = 1 / math.sqrt(D)
    out_a = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse_a = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    kv.attn_int2_decode(c, n, qd, scale, out=out_a, lse=lse_a)
    out_b = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    lse_b = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    kv.attn_int2_decode_noalloc(c, n, qd, scale, out_b, lse=lse_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b), f"{tag}: outputs differ"
    assert torch.equal(lse_a, lse_b), f"{tag}: lse differs"
    ref, _ = to_oracle(c).attention(
        synth.bf16_bits_to_f32(q_bits).astype(np.float64).reshape(B, 1, Hq, D), n, scale)
    err = np.abs(out_b.cpu().numpy().astype(np.float64) - ref[:, 0]).max()
    assert err <= TOL, f"{tag}: {err:.3e} from the oracle"


def test_noalloc_matches_workspace_decode_window_keys():
    c1, q1 = _window_cache(4, 4, 4, 6000)     # many splits, MFMA decode
    _both(c1, 6000, q1, "first call (4 x 4 kv heads, 6000 tokens)")
    c2, q2 = _window_cache(1, 2, 4, 700)      # smaller: stale partials in the scratch
    _both(c2, 700, q2, "second call (1 x 2 kv heads, 700 tokens)")


def test_noalloc_matches_workspace_decode_centroid_keys():
    c1, q1 = _centroid_cache(3000)
    _both(c1, 3000, q1, "first call (centroid keys, 3000 tokens)")
    c2, q2 = _centroid_cache(200)
    _both(c2, 130, q2, "second call (centroid keys, 130 of 200 tokens)")
