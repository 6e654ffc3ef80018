"""Pins for the oracle's two QuantWM variants: QSAC's range-based
perturbation estimate ("QuantWM Framework" 1: the estimate considers the
residual groups' dynamic range and the query sensitivity) and INT8 PSAC
coefficients with a per-token scale ("QuantWM Framework" 2: the
compensation coefficients are quantized to INT8).  Checks use exactly
representable constructions, independent fp64 numpy evaluation, the
symmetric INT8 error bound, and the compensated-key attention identity."""
import math

import numpy as np
import pytest

import oracle
import synth

f32 = synth.bf16_bits_to_f32


def _dist64(k, cent, w):
    t = k.astype(np.float64)[None, :] - cent.astype(np.float64)
    return (w.astype(np.float64)[None, :] * t * t).sum(1)


def _range_estimate64(k, c, w):
    """sum_g s_g^2 W_g in fp64, s_g the fp16 step numpy's IEEE conversion
    gives for (max - min) / 3 computed in fp32."""
    r = (k - c).astype(np.float32).reshape(-1, 32)
    s = ((r.max(1) - r.min(1)) / np.float32(3)).astype(np.float16).astype(np.float64)
    W = w.astype(np.float64).reshape(-1, 32).sum(1)
    return float((s * s * W).sum())


def test_range_estimate_dyadic_closed_form():
    """Residual ranges 3 * 2^e_g and integer weights make every step, weight
    sum and product exact: E = sum_g 4^e_g W_g.  With every candidate in the
    shortlist the oracle must take the smallest such E."""
    rng = np.random.default_rng(31)
    D, C = 128, 12
    w = rng.integers(1, 5, D).astype(np.float32)
    W = w.reshape(4, 32).sum(1).astype(np.int64)
    k = np.zeros(D, np.float32)
    exps = rng.integers(-6, 3, (C, 4))
    cent = np.empty((C, D), np.float32)
    for j in range(C):
        for g in range(4):
            s = 2.0 ** int(exps[j, g])
            r = rng.choice([0.0, s, 2 * s, 3 * s], 32).astype(np.float32)
            r[0], r[1] = 0.0, 3 * s          # the range is exactly 3 s
            cent[j, 32 * g:32 * g + 32] = -r
    E = [sum(4.0 ** int(exps[j, g]) * W[g] for g in range(4)) for j in range(C)]
    best = min(range(C), key=lambda j: (E[j], j))
    assert oracle.assign_qsac(k, cent, w, C, oracle.QSAC_RANGE) == best
    # residuals on the INT2 grid have zero quantization error: the exact rule
    # is indifferent and takes the lowest index, the range rule need not
    assert oracle.assign_qsac(k, cent, w, C, oracle.QSAC_EXACT) == 0


def test_range_and_exact_estimates_choose_differently():
    """Candidate 0: large range, every residual on the INT2 grid (no error).
    Candidate 1: small range, residuals halfway between levels.  The exact
    error prefers 0, the range estimate prefers 1."""
    D = 128
    k = np.zeros(D, np.float32)
    w = np.ones(D, np.float32)
    r0 = np.tile(np.array([0.0, 1.0, 2.0, 3.0], np.float32), D // 4)          # step 1, on grid
    r1 = np.tile(np.array([0.0, 0.125, 0.375, 0.75], np.float32), D // 4)      # step 0.25, off grid
    cent = np.stack([-r0, -r1]).astype(np.float32)
    assert oracle.assign_qsac(k, cent, w, 2, oracle.QSAC_EXACT) == 0
    assert oracle.assign_qsac(k, cent, w, 2, oracle.QSAC_RANGE) == 1


def _cand(steps, D=128):
    """Centroid whose residual against a zero key has, in group g, the
    range 3 * steps[g] (values on that group's INT2 grid)."""
    c = np.empty(D, np.float32)
    for g, st in enumerate(steps):
        r = np.tile(np.array([0.0, 1.0, 2.0, 3.0], np.float32), 8) * np.float32(st)
        c[32 * g:32 * g + 32] = -r
    return c


def _pick(steps_list, w):
    k = np.zeros(128, np.float32)
    cent = np.stack([_cand(st) for st in steps_list]).astype(np.float32)
    return oracle.assign_qsac(k, cent, w.astype(np.float32), len(steps_list), oracle.QSAC_RANGE)


def test_range_estimate_discriminates_its_terms():
    """Exact constructions whose winner flips under a plausible slip in the
    estimate: the step unsquared, the weights squared or dropped, or the
    fp32 step used instead of the fp16 step the quantizer stores."""
    ones = np.ones(128)
    # squared steps: (1,1,1,1) -> 4 beats (2,1/4,1/4,1/4) -> 4.1875; linear sums would flip it
    assert _pick([(2, .25, .25, .25), (1, 1, 1, 1)], ones) == 1
    # group weights W_g = sum of w: group 1 all 2 (W 64, sum w^2 128), group 2
    # half 0.5 half 3 (W 56, sum w^2 148); a large step in group 2 costs less
    w = np.ones(128)
    w[32:64] = 2.0
    w[64:80], w[80:96] = 0.5, 3.0
    assert _pick([(.5, 2, .5, .5), (.5, .5, 2, .5)], w) == 1
    # unweighted sums would prefer (1, 2, 1/2, 1/2) (5.5 < 7); with W = (32, 128, 128, 128)
    # it costs 608 against 512 for (2, 1, 1, 1)
    w = np.full(128, 4.0)
    w[:32] = 1.0
    assert _pick([(1, 2, .5, .5), (2, 1, 1, 1)], w) == 1
    # fp32 steps 1 + 2^-12 and 1 round to the same fp16 step: a tie, which
    # the lower index wins (the fp32 step would pick index 1)
    assert _pick([(1 + 2.0 ** -12, 1, 1, 1), (1, 1, 1, 1)], ones) == 0


@pytest.mark.parametrize("topk", [1, 4, 16])
def test_range_estimate_against_fp64(topk):
    """Random keys, candidates and weights: the choice is the fp64 argmin of
    sum_g s_g^2 W_g over the topk nearest centroids by the weighted distance
    (near ties, within 1e-5 relative, accept either)."""
    rng = np.random.default_rng(32 + topk)
    C, D = 16, 128
    cent = rng.standard_normal((C, D)).astype(np.float32)
    w = rng.uniform(0.1, 3, D).astype(np.float32)
    for _ in range(80):
        k = (cent[rng.integers(C)] + 0.8 * rng.standard_normal(D) *
             rng.uniform(0.2, 2.0, D)).astype(np.float32)
        j = oracle.assign_qsac(k, cent, w, topk, oracle.QSAC_RANGE)
        dw = _dist64(k, cent, w)
        short = np.argsort(dw, kind="stable")[:topk]
        E = {int(i): _range_estimate64(k, cent[i], w) for i in short}
        best = min(E, key=lambda i: (E[i], i))
        assert j in E
        assert j == best or abs(E[j] - E[best]) <= 1e-5 * E[best]


def test_range_estimate_scale_and_permutation_invariance():
    """Scaling all weights by 2 and permuting channels inside each group
    (with the key and centroids permuted alike) leaves the choice unchanged."""
    rng = np.random.default_rng(33)
    C, D = 8, 128
    cent = rng.standard_normal((C, D)).astype(np.float32)
    w = rng.integers(1, 9, D).astype(np.float32)       # exact sums in any order
    perm = np.concatenate([32 * g + rng.permutation(32) for g in range(4)])
    for _ in range(40):
        k = (cent[rng.integers(C)] + rng.standard_normal(D)).astype(np.float32)
        j = oracle.assign_qsac(k, cent, w, C, oracle.QSAC_RANGE)
        assert oracle.assign_qsac(k, cent, 2 * w, C, oracle.QSAC_RANGE) == j
        assert oracle.assign_qsac(k[perm], np.ascontiguousarray(cent[:, perm]), w[perm], C,
                                  oracle.QSAC_RANGE) == j


def _psac_cache(psac_fmt, qsac_score=oracle.QSAC_EXACT, T=640, H=2):
    d = synth.sensitivity_aware(H=H, T=T, Lq=16, C=16, n_cal=256)
    K = f32(d["K"])[0]
    c = oracle.Cache(1, H, 128, T, key_mode=oracle.KEY_CENTROID_QSAC,
                     value_mode=oracle.VAL_HADAMARD, C=16, topk=4, R=8,
                     qsac_score=qsac_score, psac_fmt=psac_fmt)
    qc = f32(d["q_cal"]).astype(np.float64)
    for h in range(H):
        c.centroids[0, h] = oracle.kmeans(K[:, h], 16, d["kmeans_init"][0, h], 2)[0]
        c.sens_w[0, h] = oracle.sens_weights(qc[:, h])
        c.psac_basis[0, h] = oracle.pca(qc[:, h], 8)[0]
    c.append(d["K"], d["V"], 0)
    return c, d, K


def test_psac_int8_against_fp64_coefficients():
    """q * sc is within half a step of the fp64 coefficients U^T e; the
    largest coefficient of every token lands on +-127; signs are kept; the
    scale is max |a| / 127 to fp16 precision."""
    c, d, K = _psac_cache(oracle.PSAC_INT8)
    for h in range(2):
        kh = c.keys(0, h, 640)
        U = c.psac_basis[0, h].astype(np.float64)
        want = (K[:, h].astype(np.float64) - kh) @ U              # [T][8]
        q = c.k_psac8[0, h, :640].astype(np.float64)
        sc = oracle.f16_array_to_f64(c.k_psac_sc[0, h, :640])
        amax = np.abs(want).max(1)
        assert np.all(sc > 0)
        assert np.all(np.abs(sc - amax / 127) <= 2.0 ** -10 * amax / 127 + 1e-9)
        assert np.all(np.abs(q).max(1) == 127)
        assert np.all(np.abs(q * sc[:, None] - want) <= 0.5 * sc[:, None] * (1 + 1e-3) + 1e-7)
        nz = q != 0
        assert np.all(np.sign(q[nz]) == np.sign(want[nz]))


def test_psac_format_changes_only_the_coefficients():
    """The INT8 format leaves indices, codes and parameters as the fp16
    format makes them; the fp16 buffer stays untouched."""
    a, _, _ = _psac_cache(oracle.PSAC_F16)
    b, _, _ = _psac_cache(oracle.PSAC_INT8)
    for name in ("k_idx", "k_codes", "k_params", "v_codes", "v_params"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    assert not b.k_psac.any()
    # fp16 vs INT8 coefficients agree to the INT8 step
    fa = oracle.f16_array_to_f64(a.k_psac[0, :, :640])
    fb = b.k_psac8[0, :, :640].astype(np.float64) * oracle.f16_array_to_f64(b.k_psac_sc[0, :, :640])[..., None]
    step = oracle.f16_array_to_f64(b.k_psac_sc[0, :, :640])[..., None]
    assert np.all(np.abs(fa - fb) <= 0.5 * step * 1.01 + np.abs(fa) * 2.0 ** -10 + 1e-7)


def test_psac_int8_attention_is_compensated_keys():
    """Attention with INT8 coefficients equals fp64 softmax attention over the
    keys khat + U (q * sc), values rotated back."""
    import scipy.linalg
    c, d, K = _psac_cache(oracle.PSAC_INT8, T=192, H=1)
    q = f32(d["q"])[:, :4].astype(np.float64)
    scale = 1 / math.sqrt(128)
    out, lse = c.attention(q, 192, scale)
    U = c.psac_basis[0, 0].astype(np.float64)
    a = c.k_psac8[0, 0, :192].astype(np.float64) * oracle.f16_array_to_f64(c.k_psac_sc[0, 0, :192])[:, None]
    Kt = c.keys(0, 0, 192) + a @ U.T
    V = c.values(0, 0, 192)
    Hm = scipy.linalg.hadamard(128) / math.sqrt(128)
    for i in range(4):
        lg = scale * (Kt @ q[0, i, 0])
        m = lg.max()
        p = np.exp(lg - m)
        o = (p / p.sum()) @ V
        assert np.allclose(out[0, i, 0], Hm @ o, atol=1e-12)
        assert abs(lse[0, 0, i] - (m + math.log(p.sum()))) < 1e-10


def test_psac_int8_still_reduces_logit_error():
    """INT8 coefficients keep most of the compensation: the mean |logit error|
    drops below 0.8x the uncompensated one, and stays within 5% of fp16's."""
    errs = {}
    for fmt in (oracle.PSAC_F16, oracle.PSAC_INT8):
        c, d, K = _psac_cache(fmt, T=1024, H=1)
        kh = c.keys(0, 0, 1024)
        U = c.psac_basis[0, 0].astype(np.float64)
        if fmt == oracle.PSAC_F16:
            a = oracle.f16_array_to_f64(c.k_psac[0, 0, :1024])
        else:
            a = c.k_psac8[0, 0, :1024].astype(np.float64) * oracle.f16_array_to_f64(c.k_psac_sc[0, 0, :1024])[:, None]
        q = f32(d["q"])[0, :, 0].astype(np.float64)
        K0 = K[:, 0].astype(np.float64)
        errs[fmt] = (np.abs(q @ (K0 - kh).T).mean(), np.abs(q @ (K0 - kh - a @ U.T).T).mean())
    base, comp16 = errs[oracle.PSAC_F16]
    _, comp8 = errs[oracle.PSAC_INT8]
    assert comp8 < 0.8 * base
    assert comp8 <= 1.05 * comp16


def test_qsac_range_cache_keys_within_bounds():
    """A cache built with the range estimate quantizes every key within half
    a step of its chosen centroid's residual, and its chosen centroid is
    among the 4 nearest by the weighted distance."""
    c, d, K = _psac_cache(oracle.PSAC_F16, qsac_score=oracle.QSAC_RANGE)
    for h in range(2):
        kh = c.keys(0, h, 640)
        prm = c.k_params[0, h, :640]
        s = oracle.f16_array_to_f64((prm & 0xFFFF).astype(np.uint16))
        err = np.abs(kh - K[:, h]).reshape(640, 4, 32)
        assert np.all(err <= (0.5 * s + 4e-3 * s + 1e-6)[:, :, None] + 1e-6)
        w = c.sens_w[0, h]
        for t in range(0, 640, 29):
            dw = _dist64(K[t, h], c.centroids[0, h], w)
            assert int(c.k_idx[0, h, t]) in np.argsort(dw, kind="stable")[:4]


def test_top1_against_numpy_and_attention_limit():
    """Top-1 tokens equal the numpy argmax of the compensated fp64 logits
    over the oracle's dequantised keys, for fp16 and INT8 coefficients and
    window keys; a very sharp softmax returns the top-1 token's value; a
    duplicated key ties and the lower index wins."""
    for fmt in (oracle.PSAC_F16, oracle.PSAC_INT8):
        c, d, K = _psac_cache(fmt, T=192, H=1)
        q = f32(d["q"])[:, :6].astype(np.float64)           # [1][6][1][D]
        idx, lg = c.top1(q, 192)
        U = c.psac_basis[0, 0].astype(np.float64)
        if fmt == oracle.PSAC_F16:
            a = oracle.f16_array_to_f64(c.k_psac[0, 0, :192])
        else:
            a = c.k_psac8[0, 0, :192].astype(np.float64) * oracle.f16_array_to_f64(c.k_psac_sc[0, 0, :192])[:, None]
        Kt = c.keys(0, 0, 192) + a @ U.T
        want = Kt @ q[0, :, 0].T                             # [T][6]
        assert np.array_equal(idx[0, 0], np.argmax(want, axis=0))
        assert np.allclose(lg[0, 0], want.max(0), rtol=1e-12, atol=1e-12)
        # softmax at a huge scale picks the top-1 value (rotated back)
        out, _ = c.attention(q, 192, 1e6)
        import scipy.linalg
        Hm = scipy.linalg.hadamard(128) / math.sqrt(128)
        V = c.values(0, 0, 192)
        for i in range(6):
            if np.sort(want[:, i])[-1] - np.sort(want[:, i])[-2] > 1e-4:
                assert np.allclose(out[0, i, 0], Hm @ V[idx[0, 0, i]], atol=1e-9)
    # window keys, GQA 2
    d = synth.llm_decode(B=1, T=128, Hq=4, Hkv=2)
    c = oracle.Cache(1, 2, 128, 128)
    c.append(d["K"], d["V"], 0)
    q = f32(d["q"]).astype(np.float64)[:, None]                          # [1][1][4][D]
    idx, lg = c.top1(q, 128)
    for hq in range(4):
        want = c.keys(0, hq // 2, 128) @ q[0, 0, hq]
        assert idx[0, hq, 0] == int(np.argmax(want))
    # an exact tie (token 70 repeats token 5; centroid keys have per-token
    # parameters, so both dequantise alike): the lower index wins
    Kb = np.array(d["K"][:, :, :1])
    Kb[:, 70] = Kb[:, 5]
    c = oracle.Cache(1, 1, 128, 128, key_mode=oracle.KEY_CENTROID, C=4)
    c.centroids[0, 0] = f32(Kb[0, [0, 1, 2, 3], 0])
    c.append(np.ascontiguousarray(Kb), np.ascontiguousarray(d["V"][:, :, :1]), 0)
    kh = c.keys(0, 0, 128)
    assert np.array_equal(kh[5], kh[70])
    q = kh[5][None, None, None, :] * 4.0
    idx, lg = c.top1(q, 128)
    want = kh @ q[0, 0, 0]
    assert want[5] == want.max() and idx[0, 0, 0] == 5
