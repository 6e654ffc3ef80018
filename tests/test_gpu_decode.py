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
from test_gpu_top1 import _exact_logits

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


def test_window_decode_uninitialised_workspace():
    """A workspace full of random bytes, reused across calls whose split
    counts differ, gives the fresh-workspace results bit for bit (bf16
    output and lse included), and the oracle's within tolerance: nothing in
    it is read before this call writes it."""
    d = synth.llm_decode(B=3, Hkv=2, Hq=8, D=128, T=5000)
    c = kv.KVCache(3, 2, 128, 5056, value_mode=kv.VAL_HADAMARD)
    o = oracle_like(c)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    o.append(d["K"], d["V"], 0)
    qd = dev_bf16(d["q"])
    q64 = synth.bf16_bits_to_f32(d["q"]).astype(np.float64)
    ws = kv.decode_workspace(c, 8, 5000)
    gen = torch.Generator(device="cpu").manual_seed(7)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, generator=gen))
    g = to_oracle(c)
    for n in (5000, 777, 64, 5000, 4096):
        lse_a = torch.empty(24, dtype=torch.float32, device="cuda")
        lse_b = torch.empty(24, dtype=torch.float32, device="cuda")
        a = kv.attn_int2_decode(c, n, qd, 1 / math.sqrt(128), out_dtype=torch.bfloat16, lse=lse_a, workspace=ws)
        b = kv.attn_int2_decode(c, n, qd, 1 / math.sqrt(128), out_dtype=torch.bfloat16, lse=lse_b)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"n={n}"
        assert torch.equal(lse_a, lse_b), f"n={n}"
        ref, rlse = g.attention(q64.reshape(3, 1, 8, 128), n, 1 / math.sqrt(128))
        err = np.abs(a.float().cpu().numpy().astype(np.float64) - ref[:, 0])
        assert np.all(err <= TOL + np.abs(ref[:, 0]) * 2.0 ** -8), f"n={n}: max err {err.max():.3e}"
        assert np.abs(lse_a.cpu().numpy().reshape(3, 8) - rlse[:, :, 0]).max() < 1e-3, f"n={n}"


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


@pytest.mark.slow
def test_decode_long_ragged_sampled():
    """Many (sequence, kv head) groups over a long, ragged context (16 x 8
    heads, 16421 tokens: 256 full windows and a 37-token tail in the last
    split), in the MFMA decode's launch configuration; sampled groups
    against the oracle."""
    T = 16421
    d = synth.llm_decode(T=T)
    B, H = d["B"], d["Hkv"]
    c = kv.KVCache(B, H, 128, (T + 63) // 64 * 64)
    kv.kv_quantize_append(c, dev_bf16(d["K"]), dev_bf16(d["V"]), 0)
    qd = dev_bf16(d["q"])
    out = kv.attn_int2_decode(c, T, qd, 1 / math.sqrt(128))
    torch.cuda.synchronize()
    g = to_oracle(c)
    got = out.cpu().numpy()
    q64 = synth.bf16_bits_to_f32(d["q"]).astype(np.float64)
    for b, h in [(0, 0), (7, 3), (15, 7)]:
        gs = g.slice_bh(b, h)
        qs = q64[b:b + 1, 4 * h:4 * h + 4].reshape(1, 1, 4, 128)
        ref, _ = gs.attention(np.ascontiguousarray(qs), T, 1 / math.sqrt(128))
        err = np.abs(got[b, 4 * h:4 * h + 4] - ref[0, 0]).max()
        assert err <= TOL, f"b={b} h={h} err {err}"


def test_window_prefix_and_rewind():
    """Window keys under the header's length contract: after appends past a
    window boundary, attention over a prefix of whole windows reads only
    their codes (decode and chunk match the oracle's cache of that prefix);
    an append that rewinds to a window boundary overwrites the later tokens
    and leaves the cache equal to a one-shot build of the new sequence."""
    H, G, T, P = 2, 4, 300, 256
    d = synth.llm_decode(B=1, Hkv=H, Hq=H * G, D=128, T=T)
    c = kv.KVCache(1, H, 128, 320)
    kv.kv_quantize_append(c, dev_bf16(d["K"][:, :100]), dev_bf16(d["V"][:, :100]), 0)
    kv.kv_quantize_append(c, dev_bf16(d["K"][:, 100:]), dev_bf16(d["V"][:, 100:]), 100)
    o = oracle_like(c)
    o.append(np.ascontiguousarray(d["K"][:, :P]), np.ascontiguousarray(d["V"][:, :P]), 0)
    qd = dev_bf16(d["q"])
    q64 = synth.bf16_bits_to_f32(d["q"]).astype(np.float64)
    scale = 1 / math.sqrt(128)
    _decode_check(c, o, P, qd, q64, scale, "prefix of 4 windows")
    rng = np.random.default_rng(5)
    qc = synth.to_bf16_bits(rng.standard_normal((1, 40, H * G, 128)).astype(np.float32))
    outc = kv.attn_int2_chunk(c, P, dev_bf16(qc), scale)
    torch.cuda.synchronize()
    refc, _ = o.attention(synth.bf16_bits_to_f32(qc).astype(np.float64), P, scale)
    err = np.abs(outc.cpu().numpy().astype(np.float64) - refc).max()
    assert err <= TOL, f"chunk over the prefix: {err:.3e}"
    # rewind to the window boundary and append different tokens
    K2, V2 = d["K"].copy(), d["V"].copy()
    K2[:, P:] = synth.to_bf16_bits(rng.standard_normal(K2[:, P:].shape).astype(np.float32) * 3)
    V2[:, P:] = synth.to_bf16_bits(rng.standard_normal(V2[:, P:].shape).astype(np.float32))
    kv.kv_quantize_append(c, dev_bf16(K2[:, P:]), dev_bf16(V2[:, P:]), P)
    o2 = oracle_like(c)
    o2.append(K2, V2, 0)
    _decode_check(c, o2, T, qd, q64, scale, "after the rewind")


def _small_like(c: kv.KVCache, cap: int = 64) -> oracle.Cache:
    """An empty one-sequence, one-head oracle cache of capacity cap with the
    modes and calibration inputs of c (itself one sequence and head)."""
    L = c.layout
    o = oracle.Cache(1, 1, L.head_dim, cap, L.key_mode, L.value_mode, L.n_centroids, L.qsac_topk,
                     L.psac_rank, L.qsac_score, L.psac_format,
                     M=L.n_modalities if L.value_mode == kv.VAL_HADAMARD_MODAL else 1)
    for name in ("centroids", "sens_w", "psac_basis"):
        if getattr(c, name) is not None:
            getattr(o, name)[:] = getattr(c, name).cpu().numpy()
    if c.v_signs is not None:
        o.v_signs[:] = c.v_signs.cpu().numpy().view(np.uint32)
    return o


def _maximum_capacity_check(c, d, q_dec, q_chunk, tag, modal=None):
    """Fills c (capacity 2^24, one sequence and kv head) in one append with
    2^24 - 47 tokens: 262,143 full windows, window w a copy of window w % 7
    of the seven in d, then d's last 17 tokens.  Every window's cache bytes
    must equal the oracle's for its copy, decode (q_dec bf16 bits
    [1][Hq][D]) and chunk attention (q_chunk [1][Lq][Hq][D]) over all tokens
    the oracle's merge of the seven window attentions, each weighted by its
    number of copies, and the tail's, and the top-1 token of each chunk row
    the first copy of the oracle's choice.  modal (per-modality rotations):
    the modality of each of d's tokens, copied with them."""
    W, L = 7, c.layout
    D, T = L.head_dim, (1 << 24) - 47
    n_full, rem = T // 64, T % 64
    t = np.arange(T)
    w = t // 64
    src = torch.from_numpy(np.where(w < n_full, (w % W) * 64 + t % 64, W * 64 + t - n_full * 64)).cuda()
    del t, w
    if modal is not None:
        c.v_modality[0, :T] = torch.from_numpy(modal).cuda()[src]
    kv.kv_quantize_append(c, dev_bf16(d["K"])[:, src].contiguous(), dev_bf16(d["V"])[:, src].contiguous(), 0)
    torch.cuda.synchronize()
    del src
    torch.cuda.empty_cache()
    def small(lo, hi, cap=64):    # d's tokens [lo, hi) in a cache of their own
        o = _small_like(c, cap)
        if modal is not None:
            o.v_modal[0, :hi - lo] = modal[lo:hi]
        return o

    types = []
    for j in range(W):
        oj = small(64 * j, 64 * j + 64)
        oj.append(np.ascontiguousarray(d["K"][:, 64 * j:64 * j + 64]),
                  np.ascontiguousarray(d["V"][:, 64 * j:64 * j + 64]), 0)
        types.append(oj)
    ot = small(W * 64, W * 64 + rem)
    ot.append(np.ascontiguousarray(d["K"][:, W * 64:]), np.ascontiguousarray(d["V"][:, W * 64:]), 0)
    g = to_oracle(c)
    if L.key_mode == kv.KEY_WINDOW:
        per_token, per_window = ["k_codes", "v_params"], ["k_params", "v_codes"]
        assert np.array_equal(g.k_tail[0, 0, :rem], ot.k_tail[0, 0, :rem]), f"{tag}: k_tail"
    else:
        per_token, per_window = ["k_idx", "k_codes", "k_params", "v_params"], ["v_codes"]
        if L.psac_rank > 0:
            per_token += ["k_psac8", "k_psac_sc"] if L.psac_format == kv.PSAC_INT8 else ["k_psac"]
    for name in per_token:
        a = getattr(g, name)[0, 0]
        rows = a[:n_full * 64].reshape((n_full, 64) + a.shape[1:])
        for j, oj in enumerate(types):
            assert np.all(rows[j::W] == getattr(oj, name)[0, 0, :64]), f"{tag}: {name} of copies of window {j}"
        assert np.array_equal(a[n_full * 64:T], getattr(ot, name)[0, 0, :rem]), f"{tag}: {name} of the tail"
    for name in per_window:
        a = getattr(g, name)[0, 0]
        for j, oj in enumerate(types):
            assert np.all(a[j:n_full:W] == getattr(oj, name)[0, 0, 0]), f"{tag}: {name} of window {j}"
    bits = np.zeros(128, np.uint8)
    bits[:2 * rem] = 1
    mask = np.packbits(bits.reshape(16, 8)[:, ::-1], axis=1).reshape(16)
    assert np.array_equal(g.v_codes[0, 0, n_full] & mask, ot.v_codes[0, 0, 0] & mask), f"{tag}: tail v_codes"
    del g

    counts = [len(range(j, n_full, W)) for j in range(W)]
    scale = 1 / math.sqrt(D)
    Hq = q_dec.shape[1]

    def reference(q64):                      # q64 [1][Lq][Hq][D]
        parts = [oj.attention(q64, 64, scale) for oj in types] + [ot.attention(q64, rem, scale)]
        Lq = q64.shape[1]
        out = np.empty((Lq, Hq, D))
        lse = np.empty((Hq, Lq))
        for r in range(Lq):
            for hq in range(Hq):
                m = np.array([p[1][0, hq, r] for p in parts]) + np.log(np.array(counts + [1.0]))
                o = np.stack([p[0][0, r, hq] for p in parts])
                out[r, hq], lse[hq, r] = oracle.merge(m, np.ones(W + 1), o)
        return out, lse

    ref, rlse = reference(synth.bf16_bits_to_f32(q_dec).astype(np.float64).reshape(1, 1, Hq, D))
    lse = torch.empty(Hq, dtype=torch.float32, device="cuda")
    out = kv.attn_int2_decode(c, T, dev_bf16(q_dec), scale, lse=lse)
    torch.cuda.synchronize()
    err = np.abs(out.cpu().numpy()[0].astype(np.float64) - ref[0]).max()
    assert err <= TOL, f"{tag}: decode max err {err:.3e}"
    assert np.abs(lse.cpu().numpy() - rlse[:, 0]).max() < 1e-3, f"{tag}: decode lse"
    Lq = q_chunk.shape[1]
    ref, rlse = reference(synth.bf16_bits_to_f32(q_chunk).astype(np.float64))
    lse = torch.empty((1, Hq, Lq), dtype=torch.float32, device="cuda")
    out = kv.attn_int2_chunk(c, T, dev_bf16(q_chunk), scale, lse=lse)
    torch.cuda.synchronize()
    err = np.abs(out.cpu().numpy()[0].astype(np.float64) - ref).max()
    assert err <= TOL, f"{tag}: chunk max err {err:.3e}"
    assert np.abs(lse.cpu().numpy()[0] - rlse).max() < 1e-3, f"{tag}: chunk lse"
    # top-1 token of the chunk rows: the copies of a window have bit-identical
    # fp32 logits, so the first-on-ties rule must pick a token of the first
    # copy (or of the tail); checked against the oracle over the 7 * 64 + 17
    # distinct tokens as in test_gpu_top1
    nd = W * 64 + rem
    od = small(0, nd, 512)
    od.append(np.ascontiguousarray(d["K"]), np.ascontiguousarray(d["V"]), 0)
    idx, lg = kv.attn_int2_top1(c, T, dev_bf16(q_chunk), logits=True)
    torch.cuda.synchronize()
    idx, lg = idx.cpu().numpy()[0], lg.cpu().numpy()[0]             # [Hq][Lq]
    q64 = synth.bf16_bits_to_f32(q_chunk).astype(np.float64)        # [1][Lq][Hq][D]
    oi, _ = od.top1(q64, nd)
    to_full = lambda t: t if t < W * 64 else n_full * 64 + t - W * 64
    G = Hq // L.kv_heads
    for hq in range(Hq):
        ex, mag = _exact_logits(od, 0, hq // G, nd, q64[0, :, hq])
        for r in range(Lq):
            j = int(idx[hq, r])
            assert j < W * 64 or n_full * 64 <= j < T, f"{tag}: top-1 {j} is a later copy"
            t = j if j < W * 64 else W * 64 + j - n_full * 64
            tol = 1e-5 * mag[r, t] + 1e-6
            assert abs(lg[hq, r] - ex[r, t]) <= tol, f"{tag} hq={hq} r={r}: top-1 logit"
            assert ex[r, t] >= ex[r].max() - 2 * tol - 1e-5 * mag[r].max(), f"{tag}: not a maximum"
            srt = np.sort(ex[r])
            if srt[-1] - srt[-2] > 2e-5 * mag[r].max() + 2e-6:
                assert j == to_full(int(oi[0, hq, r])), f"{tag} hq={hq} r={r}: {j} vs the oracle"


@pytest.mark.slow
@pytest.mark.parametrize("D,Hq", [(128, 4), (64, 2)])
def test_window_keys_at_maximum_capacity(D, Hq):
    """Window keys: head_dim 128 with 4 query heads per kv head (the MFMA
    decode, 8,192 splits) and head_dim 64 with 2 (the VALU decode); the
    query, its negation and its channel reversal as chunk rows."""
    d = synth.llm_decode(B=1, Hkv=1, Hq=Hq, D=D, T=7 * 64 + 17)
    qc = np.ascontiguousarray(np.stack([d["q"][0], d["q"][0] ^ 0x8000, d["q"][0, :, ::-1]])[None])
    _maximum_capacity_check(kv.KVCache(1, 1, D, 1 << 24), d, d["q"], qc, f"window keys D={D}")


@pytest.mark.slow
def test_centroid_keys_at_maximum_capacity():
    """64 centroids with the QSAC choice, rank-8 PSAC and rotated values,
    calibrated on the seven distinct windows (two k-means rounds)."""
    d = synth.sensitivity_aware(H=1, T=7 * 64 + 17, Lq=3, C=64, n_cal=256)
    c = kv.KVCache(1, 1, 128, 1 << 24, key_mode=kv.KEY_CENTROID_QSAC, n_centroids=64, qsac_topk=4,
                   psac_rank=8, value_mode=kv.VAL_HADAMARD)
    calibrate(c, d["K"], d["kmeans_init"], 2, d["q_cal"])
    _maximum_capacity_check(c, d, np.ascontiguousarray(d["q"][:, 0]), d["q"], "centroid keys")


@pytest.mark.slow
def test_modal_values_at_maximum_capacity():
    """Window keys with values rotated per modality (three modalities in
    runs across the seven windows and the tail)."""
    d = synth.llm_decode(B=1, Hkv=1, Hq=4, D=128, T=7 * 64 + 17)
    rng = np.random.default_rng(31)
    c = kv.KVCache(1, 1, 128, 1 << 24, value_mode=kv.VAL_HADAMARD_MODAL, n_modalities=3)
    signs = rng.integers(0, 1 << 32, size=(1, 3, 4), dtype=np.uint64).astype(np.uint32)
    c.v_signs.copy_(torch.from_numpy(signs.view(np.int32)))
    modal = np.repeat(rng.integers(0, 3, 465 // 15 + 1), 15)[:465].astype(np.uint8)
    qc = np.ascontiguousarray(np.stack([d["q"][0], d["q"][0] ^ 0x8000, d["q"][0, :, ::-1]])[None])
    _maximum_capacity_check(c, d, d["q"], qc, "modal values", modal)
