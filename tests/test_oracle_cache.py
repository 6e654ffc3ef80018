"""Pins for the oracle's cache update: key-range windows and the bf16 tail,
per-token value groups (plain and rotated), centroid + residual keys, QSAC
and PSAC.  Checks are against error bounds, brute force with independent
fp64 numpy arithmetic, and append-order invariance."""
import math
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth

f32 = synth.bf16_bits_to_f32


def _params(words):
    s = oracle.f16_array_to_f64((words & 0xFFFF).astype(np.uint16))
    z = oracle.f16_array_to_f64((words >> 16).astype(np.uint16))
    return s, z


def _bound(s):
    # half a step, plus slack for fp16 rounding of scale/zero (<= 2^-11
    # relative of the group range) -- generous but far below a wrong group
    return 0.5 * s + 4e-3 * s + 1e-6


def _valid_tail(c: oracle.Cache, n: int):
    r = n % oracle.WINDOW
    return c.k_tail[:, :, :r]


def test_window_keys_error_bound_and_tail():
    d = synth.llm_decode(B=2, Hkv=2, Hq=4, D=128, T=1000)
    c = oracle.Cache(2, 2, 128, 1024)
    c.append(d["K"], d["V"], 0)
    K = f32(d["K"])
    for b in range(2):
        for h in range(2):
            kh = c.keys(b, h, 1000)
            ref = K[b, :, h, :].astype(np.float64)
            s, _ = _params(c.k_params[b, h, :1000 // 64])          # [W][D]
            err = np.abs(kh[:960] - ref[:960]).reshape(15, 64, 128)
            assert np.all(err <= _bound(s)[:, None, :])
            # the unfinished window waits verbatim in the tail
            assert (c.k_tail[b, h, :40] == d["K"][b, 960:1000, h]).all()
            assert (kh[960:] == ref[960:]).all()
    # a wrong window index would give errors of the key's own size
    assert np.abs(kh[:960] - ref[:960]).max() < 0.3 * np.abs(ref).max()


def test_window_params_are_per_channel_min_max():
    d = synth.llm_decode(B=1, Hkv=1, Hq=1, D=128, T=256)
    c = oracle.Cache(1, 1, 128, 256)
    c.append(d["K"], d["V"], 0)
    K = f32(d["K"])[0, :, 0, :]
    s, z = _params(c.k_params[0, 0])
    for w in range(4):
        blk = K[64 * w:64 * w + 64]
        # bf16 minima are fp16-exact: the stored zero point is the column min
        assert np.array_equal(z[w], blk.min(0).astype(np.float64))
        rng = (blk.max(0) - blk.min(0)).astype(np.float64)
        assert np.allclose(s[w] * 3, rng, rtol=2e-3)


@pytest.mark.parametrize("chunks", [[1] * 70 + [930], [7] * 142 + [6], [64] * 15 + [40],
                                    [1560 - 1500, 940], [1000]])
def test_append_split_invariance(chunks):
    d = synth.llm_decode(B=2, Hkv=2, Hq=4, D=128, T=1000)
    one = oracle.Cache(2, 2, 128, 1024)
    one.append(d["K"], d["V"], 0)
    many = oracle.Cache(2, 2, 128, 1024)
    pos = 0
    for n in chunks:
        many.append(np.ascontiguousarray(d["K"][:, pos:pos + n]),
                    np.ascontiguousarray(d["V"][:, pos:pos + n]), pos)
        pos += n
    assert pos == 1000
    full = 960
    assert (one.k_codes[:, :, :full] == many.k_codes[:, :, :full]).all()
    assert (one.k_params[:, :, :15] == many.k_params[:, :, :15]).all()
    assert (_valid_tail(one, 1000) == _valid_tail(many, 1000)).all()
    assert (one.v_codes[:, :, :1000] == many.v_codes[:, :, :1000]).all()
    assert (one.v_params[:, :, :1000] == many.v_params[:, :, :1000]).all()


@pytest.mark.parametrize("hadamard", [False, True])
def test_value_groups_error_bound(hadamard):
    d = synth.video_chunk(H=2, D=128, T=320, Lq=8, C=4)
    c = oracle.Cache(1, 2, 128, 320, value_mode=oracle.VAL_HADAMARD if hadamard else oracle.VAL_GROUP,
                     key_mode=oracle.KEY_CENTROID, C=4)
    c.append(d["K"], d["V"], 0)
    V = f32(d["V"])[0].astype(np.float64)
    Hm = scipy.linalg.hadamard(128) / math.sqrt(128)
    for h in range(2):
        vh = c.values(0, h, 320)
        ref = V[:, h, :] @ Hm.T if hadamard else V[:, h, :]
        s, _ = _params(c.v_params[0, h, :320])          # [T][4]
        err = np.abs(vh - ref).reshape(320, 4, 32)
        assert np.all(err <= _bound(s)[:, :, None] + 1e-6)
        if hadamard:   # the rotation is orthogonal: row errors keep their norm
            back = np.linalg.norm(vh @ Hm - V[:, h, :], axis=1)
            assert np.allclose(back, np.linalg.norm(vh - ref, axis=1), rtol=1e-9)


def _dist64(k, cent, w=None):
    t = k[None, :].astype(np.float64) - cent.astype(np.float64)
    return (t * t if w is None else w.astype(np.float64) * t * t).sum(1)


def test_centroid_assign_brute_force():
    rng = np.random.default_rng(5)
    cent = rng.standard_normal((64, 128)).astype(np.float32)
    near_ties = 0
    for _ in range(400):
        k = (cent[rng.integers(64)] + 0.8 * rng.standard_normal(128)).astype(np.float32)
        j = oracle.assign_plain(k, cent)
        d = _dist64(k, cent)
        best = int(np.argmin(d))
        if j != best:
            near_ties += 1
            assert abs(d[j] - d[best]) <= 1e-5 * d[best]
    assert near_ties <= 2
    # C = 1, and duplicated centroids -> the lower index
    assert oracle.assign_plain(cent[3], cent[:1]) == 0
    dup = np.concatenate([cent[:5], cent[:5]])
    for i in range(5):
        assert oracle.assign_plain(cent[i], dup) == i
    # exact ties at equal distance go to the lower index
    two = np.array([[1.0] * 4, [-1.0] * 4], np.float32)
    assert oracle.assign_plain(np.zeros(4, np.float32), two) == 0


def test_qsac_special_cases():
    rng = np.random.default_rng(11)
    cent = rng.standard_normal((32, 128)).astype(np.float32)
    ones = np.ones(128, np.float32)
    w = rng.uniform(0.1, 3, 128).astype(np.float32)
    for _ in range(100):
        k = (cent[rng.integers(32)] + rng.standard_normal(128)).astype(np.float32)
        # unit weights, one candidate: plain nearest centroid
        assert oracle.assign_qsac(k, cent, ones, 1) == oracle.assign_plain(k, cent)
        # one candidate: the weighted-distance argmin (fp64 brute force)
        j = oracle.assign_qsac(k, cent, w, 1)
        dw = _dist64(k, cent, w)
        assert j == int(np.argmin(dw)) or abs(dw[j] - dw.min()) <= 1e-5 * dw.min()


def _residual_error(k, c):
    """Weighted INT2 residual error of candidate centroid c, fp64 from the
    oracle's (pinned) group quantizer outputs."""
    r = (k - c).astype(np.float32)
    e = np.empty(128)
    for g in range(4):
        codes, sb, zb = oracle.q2(r[32 * g:32 * g + 32])
        s, z = oracle.f16_to_f64(sb), oracle.f16_to_f64(zb)
        e[32 * g:32 * g + 32] = r[32 * g:32 * g + 32].astype(np.float64) - (codes * s + z)
    return e


def test_qsac_all_candidates_is_brute_force():
    rng = np.random.default_rng(12)
    C = 16
    cent = rng.standard_normal((C, 128)).astype(np.float32)
    w = rng.uniform(0.1, 3, 128).astype(np.float32)
    for _ in range(60):
        k = (cent[rng.integers(C)] + 0.7 * rng.standard_normal(128)).astype(np.float32)
        j = oracle.assign_qsac(k, cent, w, C)
        E = np.array([(w.astype(np.float64) * _residual_error(k, cent[i]) ** 2).sum() for i in range(C)])
        best = int(np.argmin(E))
        assert j == best or abs(E[j] - E[best]) <= 1e-5 * E[best]
    # QSAC never increases the weighted residual error over plain assignment
    worse = 0
    for _ in range(60):
        k = (cent[rng.integers(C)] + 0.7 * rng.standard_normal(128)).astype(np.float32)
        jq = oracle.assign_qsac(k, cent, w, 4)
        jp = oracle.assign_plain(k, cent)
        eq = (w * _residual_error(k, cent[jq]) ** 2).sum()
        ep = (w * _residual_error(k, cent[jp]) ** 2).sum()
        dw = _dist64(k, cent, w)
        if jp in np.argsort(dw, kind="stable")[:4]:
            worse += eq > ep * (1 + 1e-6)
    assert worse == 0


@pytest.mark.parametrize("mode", [oracle.KEY_CENTROID, oracle.KEY_CENTROID_QSAC])
def test_centroid_cache_keys(mode):
    d = synth.sensitivity_aware(H=2, T=640, Lq=16, C=16, n_cal=256)
    K = f32(d["K"])[0]
    c = oracle.Cache(1, 2, 128, 640, key_mode=mode, value_mode=oracle.VAL_HADAMARD, C=16, topk=4, R=8)
    qc = f32(d["q_cal"]).astype(np.float64)
    for h in range(2):
        cent, _ = oracle.kmeans(K[:, h], 16, d["kmeans_init"][0, h], 2)
        c.centroids[0, h] = cent
        c.sens_w[0, h] = oracle.sens_weights(qc[:, h])
        c.psac_basis[0, h] = oracle.pca(qc[:, h], 8)[0]
    c.append(d["K"], d["V"], 0)
    for h in range(2):
        kh = c.keys(0, h, 640)
        s, _ = _params(c.k_params[0, h, :640])
        err = np.abs(kh - K[:, h]).reshape(640, 4, 32)
        assert np.all(err <= _bound(s)[:, :, None] + 1e-6)
        if mode == oracle.KEY_CENTROID:
            cent = c.centroids[0, h]
            for t in range(0, 640, 37):
                dd = _dist64(K[t, h], cent)
                j = int(c.k_idx[0, h, t])
                assert j == int(np.argmin(dd)) or abs(dd[j] - dd.min()) <= 1e-5 * dd.min()
        # PSAC coefficients: fp16 of U^T e with e the key's residual error
        U = c.psac_basis[0, h].astype(np.float64)
        e = K[:, h].astype(np.float64) - kh
        a = oracle.f16_array_to_f64(c.k_psac[0, h, :640])
        want = e @ U
        assert np.all(np.abs(a - want) <= 2.0 ** -10 * np.abs(want) + 2e-6)


def test_psac_reduces_logit_error():
    d = synth.sensitivity_aware(H=1, T=1024, Lq=256, C=16, n_cal=512)
    K = f32(d["K"])[0, :, 0]
    qc = f32(d["q_cal"])[:, 0].astype(np.float64)
    c = oracle.Cache(1, 1, 128, 1024, key_mode=oracle.KEY_CENTROID_QSAC, C=16, topk=4, R=8)
    c.centroids[0, 0] = oracle.kmeans(K, 16, d["kmeans_init"][0, 0], 2)[0]
    c.sens_w[0, 0] = oracle.sens_weights(qc)
    U, ev, _ = oracle.pca(qc, 8)
    c.psac_basis[0, 0] = U
    c.append(d["K"], d["V"], 0)
    kh = c.keys(0, 0, 1024)
    a = oracle.f16_array_to_f64(c.k_psac[0, 0, :1024])
    kt = kh + a @ U.astype(np.float64).T
    q = f32(d["q"])[0, :, 0].astype(np.float64)
    base = np.abs(q @ (K.astype(np.float64) - kh).T).mean()
    comp = np.abs(q @ (K.astype(np.float64) - kt).T).mean()
    assert comp < 0.8 * base


def _read_value_tile_fixture():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "value_tile_bytes.txt")
    values, bytes_, params = [], [], None
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        f = [x.strip() for x in line.split("|")]
        if f[0] == "value":
            values.append((f[1], int(f[2]), float(f[3])))
        elif f[0] == "byte":
            lo, _, hi = f[1].partition("..")
            bytes_.append((int(lo), int(hi or lo), int(f[2], 16)))
        elif f[0] == "param":
            params = int(f[2], 16)
    return values, bytes_, params


def test_value_tile_byte_order_golden():
    """The channel-major value tile against hand-derived bytes
    (tests/golden/value_tile_bytes.txt): writer and reader cannot share a
    transposition that this fixture would not see."""
    values, bytes_, params = _read_value_tile_fixture()
    D, T = 64, 64
    V = np.zeros((1, T, 1, D), np.float32)
    for tok, ch, val in values:
        if tok == "all":
            V[0, :, 0, ch] = val
        else:
            V[0, int(tok), 0, ch] = val
    K = np.zeros((1, T, 1, D), np.float32)
    c = oracle.Cache(1, 1, D, T, oracle.KEY_WINDOW, oracle.VAL_GROUP)
    c.append(synth.to_bf16_bits(K), synth.to_bf16_bits(V), 0)
    want = np.zeros(T * D // 4, np.uint8)
    for lo, hi, b in bytes_:
        want[lo:hi + 1] = b
    got = np.ascontiguousarray(c.v_codes).reshape(-1)
    assert got.size == want.size
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:10]
    assert np.all(np.ascontiguousarray(c.v_params).reshape(-1) == params)
