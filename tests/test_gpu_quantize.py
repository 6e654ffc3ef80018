"""GPU parity of kv_quantize_append and kv_cluster_assign against the
oracle: packed codes, parameter words, the bf16 tail, centroid indices and
PSAC words must be bit-identical."""
import numpy as np
import pytest
import torch

import bit_kv_cache_int2_amd as kv
import oracle
import synth
from gpu_helpers import assert_cache_equal, calibrate, dev_bf16, oracle_like, to_oracle

pytestmark = pytest.mark.gpu


def _append_both(c, o, K, V, chunks):
    pos = 0
    for n in chunks:
        k = np.ascontiguousarray(K[:, pos:pos + n])
        v = np.ascontiguousarray(V[:, pos:pos + n])
        kv.kv_quantize_append(c, dev_bf16(k), dev_bf16(v), pos)
        o.append(k, v, pos)
        pos += n
    torch.cuda.synchronize()
    return pos


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("chunks", [[1000], [1, 7, 56, 64, 100, 500, 272], [63, 1, 64, 65, 807]])
def test_window_keys_and_values(D, chunks):
    d = synth.llm_decode(B=2, Hkv=3, Hq=6, D=D, T=1000)
    c = kv.KVCache(2, 3, D, 1024)
    o = oracle_like(c)
    n = _append_both(c, o, d["K"], d["V"], chunks)
    assert_cache_equal(to_oracle(c), o, n, f"D={D} chunks={chunks}")


def test_window_keys_chunked_equals_one_shot_on_gpu():
    d = synth.llm_decode(B=1, Hkv=2, Hq=2, D=128, T=2000)
    a = kv.KVCache(1, 2, 128, 2048)
    b = kv.KVCache(1, 2, 128, 2048)
    kv.kv_quantize_append(a, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    pos = 0
    for n in [1560 - 1500, 1, 1499, 440]:
        kv.kv_quantize_append(b, dev_bf16(d["K"][:, pos:pos + n]), dev_bf16(d["V"][:, pos:pos + n]), pos)
        pos += n
    torch.cuda.synchronize()
    assert_cache_equal(to_oracle(a), to_oracle(b), 2000, "one-shot vs chunked")


@pytest.mark.parametrize("hadamard", [False, True])
def test_toy_centroid_keys(hadamard):
    d = synth.toy_single_head()
    c = kv.KVCache(1, 1, 64, 512, key_mode=kv.KEY_CENTROID, n_centroids=16,
                   value_mode=kv.VAL_HADAMARD if hadamard else kv.VAL_GROUP)
    calibrate(c, d["K"], d["kmeans_init"], 4)
    o = oracle_like(c)
    n = _append_both(c, o, d["K"], d["V"], [512])
    assert_cache_equal(to_oracle(c), o, n, "toy")


@pytest.mark.parametrize("mode,R,score,fmt", [
    (kv.KEY_CENTROID, 0, 0, 0), (kv.KEY_CENTROID, 8, 0, 0), (kv.KEY_CENTROID_QSAC, 0, 0, 0),
    (kv.KEY_CENTROID_QSAC, 8, 0, 0),
    # the QuantWM variants: range-based QSAC estimate, INT8 PSAC coefficients
    (kv.KEY_CENTROID_QSAC, 0, kv.QSAC_RANGE, 0), (kv.KEY_CENTROID_QSAC, 8, kv.QSAC_RANGE, kv.PSAC_INT8),
    (kv.KEY_CENTROID_QSAC, 8, kv.QSAC_EXACT, kv.PSAC_INT8), (kv.KEY_CENTROID, 8, 0, kv.PSAC_INT8)])
def test_centroid_qsac_psac_hadamard(mode, R, score, fmt):
    d = synth.sensitivity_aware(H=2, T=700, Lq=8, C=32, n_cal=256)
    c = kv.KVCache(1, 2, 128, 768, key_mode=mode, value_mode=kv.VAL_HADAMARD, n_centroids=32,
                   qsac_topk=4, psac_rank=R, qsac_score=score, psac_format=fmt)
    calibrate(c, d["K"], d["kmeans_init"][:, :, :32], 2, d["q_cal"])
    o = oracle_like(c)
    n = _append_both(c, o, d["K"], d["V"], [300, 1, 399])
    assert_cache_equal(to_oracle(c), o, n, f"mode={mode} R={R} score={score} fmt={fmt}")


def test_qsac_range_estimate_decides_differently_on_gpu():
    """The range estimate is a different rule: on these keys some tokens pick
    another centroid than with the exact error (both sides bit-exact)."""
    d = synth.sensitivity_aware(H=1, T=640, Lq=8, C=32, n_cal=256)
    idx = []
    for score in (kv.QSAC_EXACT, kv.QSAC_RANGE):
        c = kv.KVCache(1, 1, 128, 640, key_mode=kv.KEY_CENTROID_QSAC, n_centroids=32, qsac_topk=4,
                       qsac_score=score)
        calibrate(c, d["K"], d["kmeans_init"][:, :, :32], 2, d["q_cal"])
        kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
        idx.append(c.k_idx.cpu().numpy())
    assert (idx[0] != idx[1]).sum() > 0


def test_cluster_assign_plain_and_qsac():
    rng = np.random.default_rng(3)
    C, D, n = 200, 128, 3000
    cent = rng.standard_normal((C, D)).astype(np.float32)
    cent[150] = cent[17]                                  # duplicate: lower index wins
    keys = synth.to_bf16_bits(cent[rng.integers(0, C, n)] + 0.9 * rng.standard_normal((n, D)))
    keys[5] = synth.to_bf16_bits(cent[17])                # exact hit of a duplicated centroid
    w = rng.uniform(0.2, 2.0, D).astype(np.float32)
    # rows strided inside a wider matrix
    wide = np.zeros((n, 3 * D), np.uint16)
    wide[:, D:2 * D] = keys
    kt = dev_bf16(wide)[:, D:2 * D]
    ct = torch.from_numpy(cent).cuda()
    got = kv.kv_cluster_assign(kt, ct).cpu().numpy()
    gq = kv.kv_cluster_assign(kt, ct, torch.from_numpy(w).cuda(), topk=4).cpu().numpy()
    kf = synth.bf16_bits_to_f32(keys)
    want = np.array([oracle.assign_plain(kf[i], cent) for i in range(n)])
    wq = np.array([oracle.assign_qsac(kf[i], cent, w, 4) for i in range(n)])
    assert np.array_equal(got, want)
    assert np.array_equal(gq, wq)
    assert got[5] == 17


def _assign_check(keys_bits, cent, w=None, topk=1, tag=""):
    """kv_cluster_assign on the GPU equals the oracle's rule key by key."""
    kt = dev_bf16(np.ascontiguousarray(keys_bits))
    ct = torch.from_numpy(np.ascontiguousarray(cent, np.float32)).cuda()
    wt = None if w is None else torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    got = kv.kv_cluster_assign(kt, ct, wt, topk=topk).cpu().numpy()
    kf = synth.bf16_bits_to_f32(keys_bits)
    if w is None:
        want = np.array([oracle.assign_plain(kf[i], cent) for i in range(len(kf))])
    else:
        want = np.array([oracle.assign_qsac(kf[i], cent, w, topk) for i in range(len(kf))])
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{tag}: {bad.size} keys differ, first {bad[:5]} got {got[bad[:5]]} want {want[bad[:5]]}"
    return got


@pytest.mark.parametrize("D", [128, 64])
def test_cluster_assign_near_ties(D):
    """Keys on the bisector of two centroids (up to bf16 rounding) and tiny
    offsets from it: the MFMA shortlist must keep both and the rule decide."""
    rng = np.random.default_rng(11)
    C = 96
    cent = rng.standard_normal((C, D)).astype(np.float32)
    a, b = rng.integers(0, C, 400), rng.integers(0, C, 400)
    mid = 0.5 * (cent[a] + cent[b])
    keys = np.concatenate([mid, mid + 1e-3 * rng.standard_normal(mid.shape),
                           mid + 1e-6 * rng.standard_normal(mid.shape)])
    _assign_check(synth.to_bf16_bits(keys.astype(np.float32)), cent, tag=f"near ties D={D}")
    w = rng.uniform(0.0, 2.0, D).astype(np.float32)
    w[:5] = 0.0
    _assign_check(synth.to_bf16_bits(keys.astype(np.float32)), cent, w, 4, tag=f"near ties qsac D={D}")


@pytest.mark.parametrize("scale", [1e-3, 1.0, 3e3])
def test_cluster_assign_scales_and_shapes(scale):
    """Magnitudes far from 1, centroid counts that leave partial chunks and
    tiles, key counts that leave partial waves and blocks."""
    rng = np.random.default_rng(12)
    D = 128
    for C, n in ((1, 5), (3, 65), (70, 257), (256, 300)):
        cent = (scale * rng.standard_normal((C, D))).astype(np.float32)
        keys = cent[rng.integers(0, C, n)] + 0.5 * scale * rng.standard_normal((n, D))
        kb = synth.to_bf16_bits(keys.astype(np.float32))
        _assign_check(kb, cent, tag=f"scale={scale} C={C} n={n}")
        w = rng.uniform(0.1, 3.0, D).astype(np.float32)
        for topk in (1, 4):
            if topk <= C:
                _assign_check(kb, cent, w, topk, tag=f"qsac scale={scale} C={C} n={n} topk={topk}")


def test_cluster_assign_exact_scan_paths():
    """All-equal centroids (every centroid ties: the rescoring queue and the
    QSAC lists overflow), topk above 4 and a negative weight all take the
    exact scan; results must still follow the rule."""
    rng = np.random.default_rng(13)
    D, n = 128, 200
    same = np.tile(rng.standard_normal((1, D)).astype(np.float32), (40, 1))
    keys = synth.to_bf16_bits((rng.standard_normal((n, D))).astype(np.float32))
    got = _assign_check(keys, same, tag="all equal")
    assert np.all(got == 0)
    w = rng.uniform(0.5, 1.5, D).astype(np.float32)
    _assign_check(keys, same, w, 4, tag="all equal qsac")
    cent = rng.standard_normal((64, D)).astype(np.float32)
    _assign_check(keys, cent, w, 8, tag="topk 8")
    wn = w.copy()
    wn[3] = -0.25
    _assign_check(keys, cent, wn, 4, tag="negative weight")


@pytest.mark.parametrize("D", [128, 64])
def test_exact_scan_keeps_tie_order(D):
    """Nine copies of one centroid fill the QSAC shortlist (its capacity is
    eight), then a strictly closer centroid arrives last: the displaced
    copies must stay in (distance, index) order, so the lowest-index copy is
    the one kept and chosen whenever that centroid has the smaller score.
    Checked through kv_cluster_assign (exact score, topk 4 overflows the
    list, topk 8 scans outright) and through the cache with both scores."""
    rng = np.random.default_rng(14)
    n = 600
    A, B = rng.standard_normal((2, D)).astype(np.float32)
    cent = np.stack([A] * 9 + [B]).astype(np.float32)
    al = rng.uniform(0.3, 0.7, (n, 1))
    keys = synth.to_bf16_bits((al * A + (1 - al) * B + 0.3 * rng.standard_normal((n, D))).astype(np.float32))
    w = rng.uniform(0.5, 1.5, D).astype(np.float32)
    kf = synth.bf16_bits_to_f32(keys).astype(np.float64)
    closer_b = (w * (kf - B) ** 2).sum(1) < (w * (kf - A) ** 2).sum(1) * (1 - 1e-4)
    for topk in (4, 8):
        got = _assign_check(keys, cent, w, topk, tag=f"tie order D={D} topk={topk}")
        assert np.any((got == 0) & closer_b), "the construction must displace the copies"
    for score in (kv.QSAC_EXACT, kv.QSAC_RANGE):
        c = kv.KVCache(1, 1, D, 640, key_mode=kv.KEY_CENTROID_QSAC, n_centroids=10, qsac_topk=4,
                       qsac_score=score)
        c.centroids.copy_(torch.from_numpy(cent.reshape(1, 1, 10, D)))
        c.sens_w.copy_(torch.from_numpy(w.reshape(1, 1, D)))
        o = oracle_like(c)
        K = np.ascontiguousarray(keys.reshape(1, n, 1, D))
        V = synth.to_bf16_bits(rng.standard_normal((1, n, 1, D)).astype(np.float32))
        kv.kv_quantize_append(c, dev_bf16(K), dev_bf16(V), 0)
        o.append(K, V, 0)
        torch.cuda.synchronize()
        g = to_oracle(c)
        assert_cache_equal(g, o, n, f"tie order cache D={D} score={score}")
        assert np.any((g.k_idx[0, 0, :n] == 0) & closer_b)


@pytest.mark.parametrize("D,C,n,iters", [(128, 64, 3000, 3), (64, 16, 512, 4), (128, 256, 4100, 2),
                                         (128, 32, 700, 0)])
def test_kmeans_matches_oracle(D, C, n, iters):
    """GPU Lloyd rounds give the oracle's centroids and last assignment bit
    for bit; duplicated starting picks leave a centroid without members."""
    rng = np.random.default_rng(21 + C)
    base = rng.standard_normal((C, D)).astype(np.float32)
    keys = synth.to_bf16_bits((base[rng.integers(0, C, n)] + 0.7 * rng.standard_normal((n, D))).astype(np.float32))
    kf = synth.bf16_bits_to_f32(keys)
    init = rng.choice(n, C, replace=False).astype(np.int64)
    init[C - 1] = init[0]                       # a duplicate pick: its cluster stays empty
    want_c, want_a = oracle.kmeans(kf, C, init, iters)
    cent = torch.from_numpy(np.ascontiguousarray(kf[init])).cuda()
    # rows strided inside a wider matrix
    wide = np.zeros((n, 2 * D), np.uint16)
    wide[:, :D] = keys
    kt = dev_bf16(wide)[:, :D]
    got_c, got_a = kv.kv_kmeans(kt, cent, iters)
    got_c, got_a = got_c.cpu().numpy(), got_a.cpu().numpy()
    assert np.array_equal(got_a, want_a), f"assignment: {np.sum(got_a != want_a)} keys differ"
    assert np.array_equal(got_c.view(np.uint32), want_c.view(np.uint32)), \
        f"centroids: {np.sum(got_c != want_c)} values differ"


def test_kmeans_batched_heads_match_oracle():
    """One call over [B, n, H, D] keys runs every (sequence, head) table's
    rounds; each equals the oracle's k-means of that key set."""
    B, n, H, D, C, iters = 2, 1500, 3, 128, 48, 2
    rng = np.random.default_rng(77)
    keys = synth.to_bf16_bits(rng.standard_normal((B, n, H, D)).astype(np.float32) *
                              rng.uniform(0.5, 2.0, (1, 1, H, 1)).astype(np.float32))
    kf = synth.bf16_bits_to_f32(keys)
    init = np.stack([np.stack([rng.choice(n, C, replace=False) for _ in range(H)]) for _ in range(B)])
    start = np.stack([np.stack([kf[b, init[b, h], h] for h in range(H)]) for b in range(B)])
    cent = torch.from_numpy(np.ascontiguousarray(start)).cuda()
    got_c, got_a = kv.kv_kmeans(dev_bf16(keys), cent, iters)
    got_c, got_a = got_c.cpu().numpy(), got_a.cpu().numpy()
    for b in range(B):
        for h in range(H):
            want_c, want_a = oracle.kmeans(np.ascontiguousarray(kf[b, :, h]), C, init[b, h], iters)
            assert np.array_equal(got_a[b, h], want_a), f"(b={b}, h={h}) assignment"
            assert np.array_equal(got_c[b, h].view(np.uint32), want_c.view(np.uint32)), \
                f"(b={b}, h={h}) centroids"


@pytest.mark.slow
def test_kmeans_video_full_size_sampled():
    """One Lloyd round over the video workload's keys at full size (40 heads
    x 31,200 keys, 256 centroids, one call, as the benchmark times it):
    sampled heads equal the oracle's k-means bit for bit."""
    d = synth.video_chunk()
    H, T, C = d["Hkv"], d["T"], 256
    K = synth.bf16_bits_to_f32(d["K"])[0]                      # [T][H][D]
    start = np.stack([K[d["kmeans_init"][0, h], h] for h in range(H)])[None]
    cent = torch.from_numpy(np.ascontiguousarray(start)).cuda()
    got_c, got_a = kv.kv_kmeans(dev_bf16(d["K"]), cent, 1)
    got_c, got_a = got_c.cpu().numpy(), got_a.cpu().numpy()
    for h in (0, 17, 39):
        want_c, want_a = oracle.kmeans(np.ascontiguousarray(K[:, h]), C, d["kmeans_init"][0, h], 1)
        assert np.array_equal(got_a[0, h], want_a), f"h={h}: {np.sum(got_a[0, h] != want_a)} keys differ"
        assert np.array_equal(got_c[0, h].view(np.uint32), want_c.view(np.uint32)), f"h={h} centroids"


@pytest.mark.slow
def test_llm_decode_build_full_size_sampled():
    """Full 16 x 32768 x 8-head window-key build (the benchmark's launch
    configuration); all bytes of sampled (sequence, head) pairs compared."""
    d = synth.llm_decode()
    B, H, T = d["B"], d["Hkv"], d["T"]
    c = kv.KVCache(B, H, 128, T)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    torch.cuda.synchronize()
    g = to_oracle(c)
    for b, h in [(0, 0), (7, 3), (15, 7), (11, 5)]:
        o = oracle.Cache(1, 1, 128, T)
        o.append(np.ascontiguousarray(d["K"][b:b + 1, :, h:h + 1]),
                 np.ascontiguousarray(d["V"][b:b + 1, :, h:h + 1]), 0)
        assert_cache_equal(g.slice_bh(b, h), o, T, f"b={b} h={h}")


def test_append_of_more_than_65535_windows():
    """One call that touches 65,601 windows (more than a 16-bit grid
    dimension holds), after a 32-token append, so the call also completes
    the first window from the tail and leaves 17 tokens in it; the whole
    cache equals the oracle's."""
    T = 65600 * 64 + 17
    d = synth.llm_decode(B=1, Hkv=1, Hq=1, D=64, T=T)
    c = kv.KVCache(1, 1, 64, ((T + 63) // 64) * 64)
    o = oracle_like(c)
    n = _append_both(c, o, d["K"], d["V"], [32, T - 32])
    assert_cache_equal(to_oracle(c), o, n, "65601-window append")
