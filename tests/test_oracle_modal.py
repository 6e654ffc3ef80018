"""Pins for the oracle's per-modality value rotation ("OmniKVQuant: KV Cache
Quantization for Omni-LLMs", English abstract: values are rotated
separately per modality).  Reading: modality m of a head rotates a value
row by R_m = diag(sigma_m) H (H the orthonormal Walsh-Hadamard transform,
sigma_m a sign vector), so R_m^T = H diag(sigma_m).  Checked against what
the mathematics fixes, with independent numpy arithmetic: with every sign
+1 the mode is the single-rotation mode byte for byte; each R_m is
orthogonal (scipy's Sylvester matrix with the signs applied); the cache's
values rotated back with each token's own R_m^T stay within the INT2
bound of the inputs (a sign applied before H, or another modality's signs,
breaks it); attention equals the per-modality sum
o = sum_m R_m^T (sum_{t in m} p_t vhat_t) formed in numpy."""
import math

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth

f32 = synth.bf16_bits_to_f32


def _signs(rng, H, M, D, zero_first=False):
    s = rng.integers(0, 1 << 32, size=(H, M, D // 32), dtype=np.uint64).astype(np.uint32)
    if zero_first:
        s[:, 0] = 0
    return s


def _sigma(words, D):
    """+1 / -1 per channel from sign words u32 [D/32] (bit c%32 of word c/32)."""
    bits = (words[np.arange(D) // 32] >> (np.arange(D) % 32).astype(np.uint32)) & 1
    return 1.0 - 2.0 * bits.astype(np.float64)


def _cache(mode, B, H, D, T, M=1, signs=None, modal=None):
    c = oracle.Cache(B, H, D, ((T + 63) // 64) * 64, oracle.KEY_WINDOW, mode, M=M)
    if signs is not None:
        c.v_signs[:] = signs
    if modal is not None:
        c.v_modal[:, :T] = modal
    return c


@pytest.mark.parametrize("D", [64, 128])
def test_all_plus_signs_equal_the_single_rotation(D):
    rng = np.random.default_rng(D)
    B, H, T, M = 2, 2, 150, 3
    K = synth.to_bf16_bits(rng.standard_normal((B, T, H, D)).astype(np.float32))
    V = synth.to_bf16_bits((rng.standard_normal((B, T, H, D)) * 2).astype(np.float32))
    had = _cache(oracle.VAL_HADAMARD, B, H, D, T)
    mod = _cache(oracle.VAL_HADAMARD_MODAL, B, H, D, T, M=M, signs=np.zeros((H, M, D // 32), np.uint32),
                 modal=rng.integers(0, M, (B, T)).astype(np.uint8))
    had.append(K, V, 0)
    mod.append(K, V, 0)
    assert np.array_equal(had.v_codes, mod.v_codes)
    assert np.array_equal(had.v_params, mod.v_params)
    q = f32(synth.to_bf16_bits(rng.standard_normal((B, 7, H, D)).astype(np.float32))).astype(np.float64)
    oh, lh = had.attention(q, T, 1 / math.sqrt(D))
    om, lm = mod.attention(q, T, 1 / math.sqrt(D))
    assert np.array_equal(oh, om) and np.array_equal(lh, lm)


@pytest.mark.parametrize("D", [64, 128])
def test_each_signed_hadamard_is_orthogonal_and_matches_the_row_rotation(D):
    rng = np.random.default_rng(3 + D)
    Hn = scipy.linalg.hadamard(D).astype(np.float64) / math.sqrt(D)
    for words in _signs(rng, 1, 4, D)[0]:
        R = np.diag(_sigma(words, D)) @ Hn
        assert np.abs(R @ R.T - np.eye(D)).max() < 1e-12
        x = rng.standard_normal(D).astype(np.float32)
        y = oracle.rotate_modal_f32(x, words).astype(np.float64)
        assert np.abs(y - R @ x.astype(np.float64)).max() <= 1e-5 * np.abs(x).max()


@pytest.mark.parametrize("D", [64, 128])
def test_values_rotated_back_per_token_modality_are_within_the_int2_bound(D):
    rng = np.random.default_rng(11 + D)
    B, H, T, M = 1, 2, 200, 3
    signs = _signs(rng, H, M, D)
    modal = rng.integers(0, M, (B, T)).astype(np.uint8)
    V = synth.to_bf16_bits((rng.standard_normal((B, T, H, D)) * 1.5).astype(np.float32))
    K = synth.to_bf16_bits(rng.standard_normal((B, T, H, D)).astype(np.float32))
    c = _cache(oracle.VAL_HADAMARD_MODAL, B, H, D, T, M=M, signs=signs, modal=modal)
    c.append(K, V, 0)
    Hn = scipy.linalg.hadamard(D).astype(np.float64) / math.sqrt(D)
    for h in range(H):
        vh = c.values(0, h, T)                      # rotated basis
        prm = c.v_params[0, h, :T].astype(np.uint32)
        step = np.vectorize(oracle.f16_to_f64)(prm & 0xFFFF)          # [T][D/32]
        for t in range(T):
            sig = _sigma(signs[h, modal[0, t]], D)
            back = Hn @ (sig * vh[t])
            err = np.linalg.norm(back - f32(V[0, t, h]).astype(np.float64))
            # orthogonal: the error norm is the rotated-space error norm, at
            # most half a step per element (plus the fp16 zero's rounding)
            bound = math.sqrt(np.sum((np.repeat(step[t], 32) * 0.5 + 1e-3) ** 2)) + 1e-4
            assert err <= bound, (h, t, err, bound)
            wrong = Hn @ (_sigma(signs[h, (modal[0, t] + 1) % M], D) * vh[t])
            if not np.array_equal(signs[h, modal[0, t]], signs[h, (modal[0, t] + 1) % M]):
                assert np.linalg.norm(wrong - f32(V[0, t, h])) > bound


def test_attention_is_the_per_modality_sum():
    rng = np.random.default_rng(77)
    B, H, D, T, M, G = 1, 2, 128, 300, 3, 2
    signs = _signs(rng, H, M, D)
    modal = rng.integers(0, M, (B, T)).astype(np.uint8)
    K = synth.to_bf16_bits(rng.standard_normal((B, T, H, D)).astype(np.float32))
    V = synth.to_bf16_bits(rng.standard_normal((B, T, H, D)).astype(np.float32))
    c = _cache(oracle.VAL_HADAMARD_MODAL, B, H, D, T, M=M, signs=signs, modal=modal)
    c.append(K, V, 0)
    q = f32(synth.to_bf16_bits(rng.standard_normal((B, 5, H * G, D)).astype(np.float32))).astype(np.float64)
    scale = 1 / math.sqrt(D)
    out, lse = c.attention(q, T, scale)
    Hn = scipy.linalg.hadamard(D).astype(np.float64) / math.sqrt(D)
    for hq in range(H * G):
        h = hq // G
        kh, vh = c.keys(0, h, T), c.values(0, h, T)
        lg = scale * q[0, :, hq] @ kh.T
        p = np.exp(lg - lg.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        ref = np.zeros((q.shape[1], D))
        for m in range(M):
            sel = modal[0, :T] == m
            R = np.diag(_sigma(signs[h, m], D)) @ Hn
            ref += (p[:, sel] @ vh[sel]) @ R          # row form of R_m^T (sum p v)
        assert np.abs(out[0, :, hq] - ref).max() < 1e-12


def test_modality_out_of_range_is_refused():
    rng = np.random.default_rng(1)
    c = _cache(oracle.VAL_HADAMARD_MODAL, 1, 1, 64, 64, M=2, signs=_signs(rng, 1, 2, 64),
               modal=np.full((1, 64), 2, np.uint8))
    z = np.zeros((1, 64, 1, 64), np.uint16)
    with pytest.raises(ValueError):
        c.append(z, z, 0)
