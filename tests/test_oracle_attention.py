"""Pins for the oracle's attention over the dequantised cache, the split
merge and the calibration statistics.  References are independent numpy
fp64 code, library routines (numpy eigh, scipy logsumexp/hadamard) and
closed forms."""
import math

import numpy as np
import pytest
import scipy.linalg
import scipy.special

import oracle
import synth

f32 = synth.bf16_bits_to_f32


def _cache_llm(B=2, H=2, Hq=4, T=300):
    d = synth.llm_decode(B=B, Hkv=H, Hq=Hq, D=128, T=T)
    c = oracle.Cache(B, H, 128, ((T + 63) // 64) * 64)
    c.append(d["K"], d["V"], 0)
    return d, c


def _numpy_attention(q, K, V, scale):
    lg = scale * (K @ q)
    p = np.exp(lg - lg.max())
    return (p / p.sum()) @ V, scipy.special.logsumexp(lg)


def test_attention_matches_two_pass_numpy_softmax():
    d, c = _cache_llm()
    q = f32(d["q"]).astype(np.float64).reshape(2, 1, 4, 128)
    out, lse = c.attention(q, 300, 1 / math.sqrt(128))
    for b in range(2):
        for hq in range(4):
            h = hq // 2                                   # contiguous GQA groups
            o, l = _numpy_attention(q[b, 0, hq], c.keys(b, h, 300), c.values(b, h, 300),
                                    1 / math.sqrt(128))
            assert np.allclose(out[b, 0, hq], o, rtol=0, atol=1e-12)
            assert abs(lse[b, hq, 0] - l) < 1e-10


def test_attention_special_cases():
    d, c = _cache_llm(B=1, H=1, Hq=1, T=130)
    q = np.random.default_rng(0).standard_normal((1, 3, 1, 128))
    # one cached token: the output is that token's value
    out, lse = c.attention(q, 1, 0.1)
    assert np.array_equal(out[0, 0, 0], c.values(0, 0, 1)[0])
    # q = 0: every logit is 0, uniform weights -> the mean value, lse = log n
    out, lse = c.attention(np.zeros((1, 1, 1, 128)), 130, 0.1)
    assert np.allclose(out[0, 0, 0], c.values(0, 0, 130).mean(0), atol=1e-12)
    assert abs(lse[0, 0, 0] - math.log(130)) < 1e-12
    # weights sum to one: identical value rows come back unchanged (every
    # token gets token 0's codes: value codes are stored per 64-token tile,
    # channel-major, 2 bits per token)
    first = c.v_codes[:, :, 0, :, 0] & 3                   # token 0, every channel
    c.v_codes[:] = (first * 0x55).astype(np.uint8)[:, :, None, :, None]
    c.v_params[:] = c.v_params[:, :, :1]
    out, _ = c.attention(q, 130, 0.5)
    for i in range(3):
        assert np.allclose(out[0, i, 0], c.values(0, 0, 1)[0], rtol=0, atol=1e-12)


def test_attention_rotated_values_and_psac_term():
    d = synth.sensitivity_aware(H=1, T=192, Lq=4, C=8, n_cal=128)
    c = oracle.Cache(1, 1, 128, 192, key_mode=oracle.KEY_CENTROID_QSAC,
                     value_mode=oracle.VAL_HADAMARD, C=8, topk=4, R=8)
    K = f32(d["K"])[0, :, 0]
    qc = f32(d["q_cal"])[:, 0].astype(np.float64)
    c.centroids[0, 0] = oracle.kmeans(K, 8, d["kmeans_init"][0, 0], 1)[0]
    c.sens_w[0, 0] = oracle.sens_weights(qc)
    c.psac_basis[0, 0] = oracle.pca(qc, 8)[0]
    c.append(d["K"], d["V"], 0)
    q = f32(d["q"]).astype(np.float64)
    out, lse = c.attention(q, 192, 1 / math.sqrt(128))
    Hm = scipy.linalg.hadamard(128) / math.sqrt(128)
    U = c.psac_basis[0, 0].astype(np.float64)
    a = oracle.f16_array_to_f64(c.k_psac[0, 0, :192])
    Kt = c.keys(0, 0, 192) + a @ U.T        # compensated keys
    for i in range(4):
        o, l = _numpy_attention(q[0, i, 0], Kt, c.values(0, 0, 192), 1 / math.sqrt(128))
        assert np.allclose(out[0, i, 0], Hm @ o, atol=1e-12)
        assert abs(lse[0, 0, i] - l) < 1e-10


def test_merge_of_any_partition_equals_unsplit():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal(200) * 3
    V = rng.standard_normal((200, 16))
    p = np.exp(lg - lg.max())
    ref = (p / p.sum()) @ V
    for cuts in ([100], [1, 2, 3, 199], [50, 51, 150], list(range(10, 200, 10))):
        parts = np.split(np.arange(200), cuts)
        m = np.array([lg[s].max() for s in parts])
        l = np.array([np.exp(lg[s] - lg[s].max()).sum() for s in parts])
        o = np.stack([np.exp(lg[s] - lg[s].max()) @ V[s] for s in parts])
        out, lse = oracle.merge(m, l, o)
        assert np.allclose(out, ref, atol=1e-12)
        assert abs(lse - scipy.special.logsumexp(lg)) < 1e-12


# ----------------------------------------------------------------- calibration
def test_kmeans_closed_form_and_monotone():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((600, 32)) + 3 * rng.integers(0, 4, (600, 1))).astype(np.float32)
    init = synth.kmeans_init(99, 600, 8)
    cent0, a0 = oracle.kmeans(x, 8, init, 0)
    assert np.array_equal(cent0, x[init])
    prev = None
    for it in range(1, 6):
        cent, a = oracle.kmeans(x, 8, init, it)
        cprev, _ = oracle.kmeans(x, 8, init, it - 1)
        # the update step: each centroid is the fp64 mean of the members
        # assigned to it under the previous centroids (empty clusters keep
        # their centroid)
        aprev = np.array([oracle.assign_plain(v, cprev) for v in x])
        assert np.array_equal(a, aprev)
        for j in range(8):
            mem = x[aprev == j].astype(np.float64)
            if len(mem):
                assert np.array_equal(cent[j], mem.mean(0).astype(np.float32))
            else:
                assert np.array_equal(cent[j], cprev[j])
        obj = ((x.astype(np.float64) - cent[[oracle.assign_plain(v, cent) for v in x]]) ** 2).sum()
        if prev is not None:
            assert obj <= prev * (1 + 1e-9)
        prev = obj


def test_sensitivity_weights_closed_form():
    a = np.linspace(0.5, 3.0, 16)
    q = np.stack([a, -a, a, -a])                       # q_d^2 = a_d^2 exactly
    assert np.array_equal(oracle.sens_weights(q), (a * a).astype(np.float32))


def test_pca_against_eigh_and_energy():
    d = synth.sensitivity_aware(H=2, T=64, Lq=4, C=4, n_cal=1024)
    for h in range(2):
        q = f32(d["q_cal"])[:, h].astype(np.float64)
        U, ev, sweeps = oracle.pca(q, 8)
        M = q.T @ q / q.shape[0]
        w, V = np.linalg.eigh(M)
        assert np.allclose(ev, w[::-1], rtol=1e-10, atol=1e-12)
        U64 = U.astype(np.float64)
        assert np.allclose(U64.T @ U64, np.eye(8), atol=1e-6)
        for m in range(8):
            v = V[:, -1 - m]
            v = v * np.sign(v[np.argmax(np.abs(v))])
            assert np.allclose(U64[:, m], v, atol=1e-6)
            assert U64[np.argmax(np.abs(U64[:, m])), m] > 0
        # ~71% of the query energy lies in the top 8 directions (the page's figure)
        frac = ev[:8].sum() / ev.sum()
        assert 0.66 < frac < 0.76
