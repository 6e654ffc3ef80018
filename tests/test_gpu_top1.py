"""attn_int2_top1 (the attention-shift diagnostic) against the oracle's
fp64 top-1 token.  The GPU forms logits in fp32, so its choice is checked
where it is unique: the reported logit is within the fp32 error bound of the
exact logit of the reported token, that token is within twice the bound of
the exact maximum, and wherever the exact top-1 leads the runner-up by more
than twice the bound the two indices agree."""
import numpy as np
import pytest
import torch

import bit_kv_cache_int2_amd as kv
import oracle
import synth
from gpu_helpers import calibrate, dev_bf16, oracle_like, to_oracle

pytestmark = pytest.mark.gpu


def _exact_logits(o: oracle.Cache, b: int, h: int, n: int, q: np.ndarray):
    """fp64 logits [rows][n] and the sum of |terms| per (row, token)."""
    kh = o.keys(b, h, n)
    lg, mag = q @ kh.T, np.abs(q) @ np.abs(kh).T
    if o.R > 0:
        U = o.psac_basis[b, h].astype(np.float64)
        if o.psac_fmt == oracle.PSAC_INT8:
            a = o.k_psac8[b, h, :n].astype(np.float64) * oracle.f16_array_to_f64(o.k_psac_sc[b, h, :n])[:, None]
        else:
            a = oracle.f16_array_to_f64(o.k_psac[b, h, :n])
        qp = q @ U
        lg, mag = lg + qp @ a.T, mag + np.abs(qp) @ np.abs(a).T
    return lg, mag


def _check(c: kv.KVCache, n: int, qbits: np.ndarray, tag: str):
    qd = dev_bf16(qbits)
    idx, lg = kv.attn_int2_top1(c, n, qd, logits=True)
    torch.cuda.synchronize()
    idx, lg = idx.cpu().numpy(), lg.cpu().numpy()
    o = to_oracle(c)
    q64 = synth.bf16_bits_to_f32(qbits).astype(np.float64)      # [B][Lq][Hq][D]
    oi, ol = o.top1(q64, n)
    B, Lq, Hq, D = qbits.shape
    G = Hq // o.H
    agree = 0
    for b in range(B):
        for hq in range(Hq):
            ex, mag = _exact_logits(o, b, hq // G, n, q64[b, :, hq])
            for r in range(Lq):
                j = int(idx[b, hq, r])
                assert 0 <= j < n, f"{tag}: index {j}"
                tol = 1e-5 * mag[r, j] + 1e-6
                assert abs(lg[b, hq, r] - ex[r, j]) <= tol, f"{tag} b={b} hq={hq} r={r}: logit"
                mx = ex[r].max()
                assert ex[r, j] >= mx - 2 * tol - 1e-5 * mag[r].max(), f"{tag} b={b} hq={hq} r={r}: not a maximum"
                srt = np.sort(ex[r])
                if n == 1 or srt[-1] - srt[-2] > 2e-5 * mag[r].max() + 2e-6:
                    assert j == oi[b, hq, r], f"{tag} b={b} hq={hq} r={r}: {j} vs {oi[b, hq, r]}"
                    agree += 1
                assert abs(ol[b, hq, r] - mx) < 1e-9 * max(1.0, abs(mx))
    assert agree > 0.9 * B * Hq * Lq, f"{tag}: only {agree} unique maxima"


@pytest.mark.parametrize("D,n,G", [(128, 1000, 1), (128, 256, 2), (64, 333, 4), (128, 1, 1)])
def test_top1_window_keys(D, n, G):
    d = synth.llm_decode(B=2, T=max(n, 64), Hq=2 * G, Hkv=2, D=D)
    c = kv.KVCache(2, 2, D, ((n + 63) // 64) * 64 + 64)
    kv.kv_quantize_append(c, dev_bf16(d["K"][:, :n]), dev_bf16(d["V"][:, :n]), 0)
    rng = np.random.default_rng(n + D)
    q = synth.to_bf16_bits(rng.standard_normal((2, 70, 2 * G, D)).astype(np.float32))
    _check(c, n, q, f"window D={D} n={n} G={G}")


@pytest.mark.parametrize("mode,R,score,fmt", [(kv.KEY_CENTROID, 0, 0, 0),
                                              (kv.KEY_CENTROID_QSAC, 8, kv.QSAC_EXACT, kv.PSAC_F16),
                                              (kv.KEY_CENTROID_QSAC, 8, kv.QSAC_RANGE, kv.PSAC_INT8)])
def test_top1_centroid_psac(mode, R, score, fmt):
    d = synth.sensitivity_aware(H=2, T=900, Lq=130, C=32, n_cal=256)
    c = kv.KVCache(1, 2, 128, 960, key_mode=mode, n_centroids=32, qsac_topk=4, psac_rank=R,
                   value_mode=kv.VAL_HADAMARD, qsac_score=score, psac_format=fmt)
    calibrate(c, d["K"], d["kmeans_init"], 2, d["q_cal"])
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    _check(c, 900, np.ascontiguousarray(d["q"]), f"mode={mode} R={R} fmt={fmt}")


def test_top1_validation():
    c = kv.KVCache(1, 2, 128, 128)
    q = torch.zeros((1, 4, 3, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kv.KVQError):
        kv.attn_int2_top1(c, 64, q)                 # 3 query heads over 2 kv heads
    q = torch.zeros((1, 4, 2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kv.KVQError):
        kv.attn_int2_top1(c, 0, q)
    with pytest.raises(kv.KVQError):
        kv.attn_int2_top1(c, 129, q)


@pytest.mark.slow
def test_top1_video_full_size_sampled():
    """The video workload at full size (40 heads, 31,200 cached tokens,
    4,680 query rows, 256 centroids, one call): sampled heads and rows
    against the oracle's top-1 over that head's dequantised cache."""
    d = synth.video_chunk()
    H, T, Lq = d["Hkv"], d["T"], d["Lq"]
    c = kv.KVCache(1, H, 128, ((T + 63) // 64) * 64, key_mode=kv.KEY_CENTROID, n_centroids=256,
                   value_mode=kv.VAL_HADAMARD)
    calibrate(c, d["K"], d["kmeans_init"], 0)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    idx, lg = kv.attn_int2_top1(c, T, dev_bf16(d["q"]), logits=True)
    torch.cuda.synchronize()
    idx, lg = idx.cpu().numpy(), lg.cpu().numpy()
    g = to_oracle(c)
    rows = sorted(set(range(0, Lq, Lq // 12)) | {Lq - 1})
    for h in (5, 33):
        o = g.slice_bh(0, h)
        q64 = synth.bf16_bits_to_f32(d["q"][:, rows, h:h + 1]).astype(np.float64)
        oi, ol = o.top1(q64, T)
        kh = o.keys(0, 0, T)
        for r_i, r in enumerate(rows):
            ex = kh @ q64[0, r_i, 0]
            mag = np.abs(kh) @ np.abs(q64[0, r_i, 0])
            j = int(idx[0, h, r])
            tol = 1e-5 * mag[j] + 1e-6
            assert abs(lg[0, h, r] - ex[j]) <= tol, f"h={h} r={r}: logit"
            assert ex[j] >= ex.max() - 2 * tol - 1e-5 * mag.max(), f"h={h} r={r}: not a maximum"
            srt = np.sort(ex)
            if srt[-1] - srt[-2] > 2e-5 * mag.max() + 2e-6:
                assert j == oi[0, 0, r_i], f"h={h} r={r}: {j} vs {oi[0, 0, r_i]}"


@pytest.mark.parametrize("case", range(20))
def test_top1_random_configuration(case):
    """Seeded random layouts (key mode, head_dim, PSAC off / fp16 / INT8,
    batch, heads, GQA, cached length, query rows) through the same checks."""
    r = np.random.default_rng(52000 + case)
    D = int(r.choice([64, 128]))
    mode = int(r.integers(0, 3))
    B, H, G = int(r.integers(1, 3)), int(r.integers(1, 4)), int(r.choice([1, 2, 4]))
    n, Lq = int(r.integers(1, 1500)), int(r.integers(1, 150))
    C = int(r.choice([1, 8, 64])) if mode != kv.KEY_WINDOW else 0
    R = 8 if mode != kv.KEY_WINDOW and r.random() < 0.5 else 0
    fmt = kv.PSAC_INT8 if R and r.random() < 0.5 else kv.PSAC_F16
    K = synth.to_bf16_bits((r.standard_normal((B, n, H, D)) * r.uniform(0.5, 2.0, (1, 1, H, D))).astype(np.float32))
    V = synth.to_bf16_bits(r.standard_normal((B, n, H, D)).astype(np.float32))
    c = kv.KVCache(B, H, D, ((n + 63) // 64) * 64, key_mode=mode, n_centroids=C,
                   qsac_topk=min(4, C) if mode == kv.KEY_CENTROID_QSAC else 1, psac_rank=R, psac_format=fmt)
    if c.centroids is not None:
        Kf = synth.bf16_bits_to_f32(K)
        cent = np.stack([np.stack([Kf[b, r.integers(0, n, C), h] for h in range(H)]) for b in range(B)])
        c.centroids.copy_(torch.from_numpy(np.ascontiguousarray(cent, np.float32)))
    if c.sens_w is not None:
        c.sens_w.copy_(torch.from_numpy(r.uniform(0.1, 3.0, (B, H, D)).astype(np.float32)))
    if c.psac_basis is not None:
        U = np.stack([np.stack([np.linalg.qr(r.standard_normal((D, 8)))[0] for _ in range(H)]) for _ in range(B)])
        c.psac_basis.copy_(torch.from_numpy(np.ascontiguousarray(U, np.float32)))
    kv.kv_quantize_append(c, dev_bf16(K), dev_bf16(V), 0)
    q = synth.to_bf16_bits(r.standard_normal((B, Lq, H * G, D)).astype(np.float32))
    _check(c, n, q, f"case {case}: D={D} mode={mode} B={B} H={H} G={G} n={n} Lq={Lq} C={C} R={R} fmt={fmt}")
