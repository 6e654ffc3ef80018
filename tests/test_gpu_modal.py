"""GPU parity of the per-modality value rotation ("OmniKVQuant: KV Cache
Quantization for Omni-LLMs", English abstract: values rotated separately
per modality; read as R_m = diag(sigma_m) H per kv head and modality):
append (rotation, signs, INT2) bit-exact against the oracle, decode and
chunk attention (each value signed by its token's modality, one inverse
Walsh-Hadamard transform at the end) within 2e-3 of the oracle's
attention, over window and centroid keys, head_dim 64 / 128, one to three
modalities, ragged appends and GQA."""
import math

import numpy as np
import pytest
import torch

import bit_kv_cache_int2_amd as kv
import synth
from gpu_helpers import TOL, assert_cache_equal, dev_bf16, oracle_like, to_oracle

pytestmark = pytest.mark.gpu


def _modal_cache(rng, B, H, D, T, M, key_mode, signs=None):
    cap = ((T + 63) // 64) * 64
    C = 32 if key_mode != kv.KEY_WINDOW else 0
    c = kv.KVCache(B, H, D, cap, key_mode=key_mode, n_centroids=C, value_mode=kv.VAL_HADAMARD_MODAL,
                   n_modalities=M)
    if signs is None:
        signs = rng.integers(0, 1 << 32, size=(H, M, D // 32), dtype=np.uint64).astype(np.uint32)
    c.v_signs.copy_(torch.from_numpy(signs.view(np.int32)))
    # modality runs, as interleaved text / audio / video spans
    modal = np.zeros((B, cap), np.uint8)
    for b in range(B):
        t = 0
        while t < T:
            n = int(rng.integers(1, 90))
            modal[b, t:t + n] = rng.integers(0, M)
            t += n
    c.v_modality.copy_(torch.from_numpy(modal))
    return c


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("key_mode", [kv.KEY_WINDOW, kv.KEY_CENTROID])
@pytest.mark.parametrize("M", [1, 2, 3])
def test_modal_append_decode_chunk(D, key_mode, M):
    rng = np.random.default_rng(100 * D + 10 * key_mode + M)
    B, H, G, T, Lq = 2, 2, 4, 700, 150
    K = synth.to_bf16_bits((rng.standard_normal((B, T, H, D)) * 2).astype(np.float32))
    V = synth.to_bf16_bits((rng.standard_normal((B, T, H, D)) * 1.5).astype(np.float32))
    c = _modal_cache(rng, B, H, D, T, M, key_mode)
    if c.centroids is not None:
        Kf = synth.bf16_bits_to_f32(K)
        c.centroids.copy_(torch.from_numpy(np.ascontiguousarray(
            np.stack([[Kf[b, rng.integers(0, T, 32), h] for h in range(H)] for b in range(B)]), np.float32)))
    o = oracle_like(c)
    for lo, hi in ((0, 130), (130, 511), (511, T)):
        k, v = np.ascontiguousarray(K[:, lo:hi]), np.ascontiguousarray(V[:, lo:hi])
        kv.kv_quantize_append(c, dev_bf16(k), dev_bf16(v), lo)
        o.append(k, v, lo)
    torch.cuda.synchronize()
    g = to_oracle(c)
    tag = f"D={D} key_mode={key_mode} M={M}"
    assert_cache_equal(g, o, T, tag)
    scale = 1 / math.sqrt(D)
    qd = synth.to_bf16_bits(rng.standard_normal((B, H * G, D)).astype(np.float32))
    out = kv.attn_int2_decode(c, T, dev_bf16(qd), scale)
    torch.cuda.synchronize()
    ref, _ = g.attention(synth.bf16_bits_to_f32(qd).astype(np.float64).reshape(B, 1, H * G, D), T, scale)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref[:, 0]).max()
    assert err <= TOL, f"{tag}: decode {err:.3e}"
    qc = synth.to_bf16_bits(rng.standard_normal((B, Lq, H * G, D)).astype(np.float32))
    outc = kv.attn_int2_chunk(c, T, dev_bf16(qc), scale)
    torch.cuda.synchronize()
    refc, _ = g.attention(synth.bf16_bits_to_f32(qc).astype(np.float64), T, scale)
    errc = np.abs(outc.cpu().numpy().astype(np.float64) - refc).max()
    assert errc <= TOL, f"{tag}: chunk {errc:.3e}"


def test_modal_with_plus_signs_is_the_single_rotation():
    """Every sign +1: the cache bytes equal the single-rotation mode's and
    both attention outputs agree with it."""
    rng = np.random.default_rng(9)
    B, H, D, T, Lq = 1, 2, 128, 333, 70
    K = synth.to_bf16_bits(rng.standard_normal((B, T, H, D)).astype(np.float32))
    V = synth.to_bf16_bits(rng.standard_normal((B, T, H, D)).astype(np.float32))
    m = _modal_cache(rng, B, H, D, T, 3, kv.KEY_WINDOW, signs=np.zeros((H, 3, D // 32), np.uint32))
    h = kv.KVCache(B, H, D, m.layout.capacity, value_mode=kv.VAL_HADAMARD)
    for c in (m, h):
        kv.kv_quantize_append(c, dev_bf16(K), dev_bf16(V), 0)
    torch.cuda.synchronize()
    for name in ("v_codes", "v_params", "k_codes", "k_params"):
        assert torch.equal(getattr(m, name), getattr(h, name)), name
    qd = dev_bf16(synth.to_bf16_bits(rng.standard_normal((B, H, D)).astype(np.float32)))
    qc = dev_bf16(synth.to_bf16_bits(rng.standard_normal((B, Lq, H, D)).astype(np.float32)))
    s = 1 / math.sqrt(D)
    assert torch.allclose(kv.attn_int2_decode(m, T, qd, s), kv.attn_int2_decode(h, T, qd, s), atol=1e-5)
    assert torch.allclose(kv.attn_int2_chunk(m, T, qc, s), kv.attn_int2_chunk(h, T, qc, s), atol=1e-5)
