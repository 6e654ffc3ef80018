"""Seeded random kv_cluster_assign cases against the oracle's rules, built
to reach every path of the fast assignment: duplicated centroids (ties the
lowest index must win, including runs longer than the QSAC shortlist),
keys on the bisector of two centroids and just off it, keys equal to a
centroid, magnitudes from 1e-3 to 1e3, centroid counts 1 to 256 that leave
partial chunks, key counts that leave partial waves, and the QSAC rule
with topk 1 to 8 and weights that may be zero.  Indices must match bit
for bit."""
import os

import numpy as np
import pytest
import torch

import bit_kv_cache_int2_amd as kv
import oracle
import synth
from gpu_helpers import dev_bf16

pytestmark = pytest.mark.gpu


def _draw(case: int):
    r = np.random.default_rng(31000 + case)
    D = int(r.choice([64, 128]))
    C = int(r.choice([1, 2, 7, 33, 64, 65, 200, 256]))
    n = int(r.integers(1, 700))
    scale = float(np.exp(r.uniform(np.log(1e-3), np.log(1e3))))
    cent = (scale * r.standard_normal((C, D))).astype(np.float32)
    if C > 1 and r.random() < 0.5:                      # duplicated centroids, some in long runs
        n_dup = int(r.integers(1, min(C, 12) + 1))
        src = int(r.integers(0, C))
        cent[r.choice(C, n_dup, replace=False)] = cent[src]
    kind = r.integers(0, 4, n)
    a, b = r.integers(0, C, n), r.integers(0, C, n)
    keys = cent[a] + 0.5 * scale * r.standard_normal((n, D))          # ordinary keys
    mid = 0.5 * (cent[a] + cent[b])
    keys[kind == 1] = mid[kind == 1]                                   # on a bisector
    keys[kind == 2] = mid[kind == 2] + 1e-3 * scale * r.standard_normal((int((kind == 2).sum()), D))
    keys[kind == 3] = cent[a][kind == 3]                               # on a centroid
    kb = synth.to_bf16_bits(keys.astype(np.float32))
    qsac = r.random() < 0.5
    topk = int(r.integers(1, min(8, C) + 1)) if qsac else 1
    w = None
    if qsac:
        w = r.uniform(0.0, 3.0, D).astype(np.float32)
        w[r.random(D) < 0.1] = 0.0
    return kb, cent, w, topk


CASES = int(os.environ.get("KVQ_ASSIGN_CASES", "200"))   # more for a deeper one-off sweep


@pytest.mark.parametrize("case", range(CASES))
def test_random_assignment(case):
    kb, cent, w, topk = _draw(case)
    kt = dev_bf16(np.ascontiguousarray(kb))
    ct = torch.from_numpy(np.ascontiguousarray(cent)).cuda()
    wt = None if w is None else torch.from_numpy(w).cuda()
    got = kv.kv_cluster_assign(kt, ct, wt, topk=topk).cpu().numpy()
    kf = synth.bf16_bits_to_f32(kb)
    if w is None:
        want = np.array([oracle.assign_plain(kf[i], cent) for i in range(len(kf))])
    else:
        want = np.array([oracle.assign_qsac(kf[i], cent, w, topk) for i in range(len(kf))])
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (f"case {case} (C={len(cent)}, D={cent.shape[1]}, n={len(kb)}, topk={topk}, "
                           f"qsac={w is not None}): {bad.size} differ, first {bad[:5]} got {got[bad[:5]]} "
                           f"want {want[bad[:5]]}")


def _draw_kmeans(case: int):
    r = np.random.default_rng(41000 + case)
    D = int(r.choice([64, 128]))
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    n = int(r.integers(1, 2500))
    C = int(r.integers(1, min(256, n) + 1))
    iters = int(r.integers(0, 4))
    scale = float(np.exp(r.uniform(np.log(1e-2), np.log(1e2))))
    centers = scale * r.standard_normal((max(C // 2, 1), D))
    keys = centers[r.integers(0, len(centers), (B, n, H))] + 0.6 * scale * r.standard_normal((B, n, H, D))
    kb = synth.to_bf16_bits(keys.astype(np.float32))
    init = np.stack([np.stack([r.choice(n, C, replace=False) for _ in range(H)]) for _ in range(B)])
    if C > 2 and r.random() < 0.5:          # a duplicated starting pick: one cluster stays empty
        init[:, :, C - 1] = init[:, :, 0]
    return kb, init, C, iters


@pytest.mark.parametrize("case", range(40))
def test_random_kmeans(case):
    """kv_kmeans over random batches, heads, key counts, centroid counts
    (with empty clusters) and round counts: every (sequence, head) table and
    its last assignment equal the oracle's Lloyd rounds bit for bit."""
    kb, init, C, iters = _draw_kmeans(case)
    B, n, H, D = kb.shape
    kf = synth.bf16_bits_to_f32(kb)
    start = np.stack([np.stack([kf[b, init[b, h], h] for h in range(H)]) for b in range(B)])
    got_c, got_a = kv.kv_kmeans(dev_bf16(kb), torch.from_numpy(np.ascontiguousarray(start)).cuda(), iters)
    got_c, got_a = got_c.cpu().numpy(), got_a.cpu().numpy()
    for b in range(B):
        for h in range(H):
            want_c, want_a = oracle.kmeans(np.ascontiguousarray(kf[b, :, h]), C, init[b, h], iters)
            tag = f"case {case} (B={B}, n={n}, H={H}, D={D}, C={C}, iters={iters}) b={b} h={h}"
            assert np.array_equal(got_a[b, h], want_a), f"{tag}: assignment"
            assert np.array_equal(got_c[b, h].view(np.uint32), want_c.view(np.uint32)), f"{tag}: centroids"
