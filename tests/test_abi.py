"""The C-ABI library loads, exports every function include/*.h declares,
and its host-side validation rejects bad arguments before any launch.  No
call here reaches the GPU (validation fails first), so this runs on machines
without one."""
import ctypes
import glob
import os
import re

import pytest

import bit_kv_cache_int2_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvint2.h")


def _declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_four_entry_points():
    names = _declared_functions()
    for n in ("kv_quantize_append", "kv_cluster_assign", "attn_int2_decode", "attn_int2_chunk"):
        assert n in names
    assert len(names) >= 9


def test_library_exports_every_declared_symbol():
    L = kv.lib()
    headers = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
    assert HEADER in headers
    for h in headers:
        for n in _declared_functions(h):
            assert hasattr(L, n), f"{os.path.basename(h)}: {n}"
    assert L.kvq_status_string(-3) == b"exceeds cache capacity"


def test_mfma_probe_validation_without_launch():
    L = kv.lib()
    p = ctypes.c_void_p(1 << 20)
    assert L.kvq_mfma_peak_probe(None, 1, 1, None) == kv.KVQ_EINVAL
    assert L.kvq_mfma_peak_probe(p, 0, 1, None) == kv.KVQ_EINVAL
    assert L.kvq_mfma_peak_probe(p, 1, 0, None) == kv.KVQ_EINVAL
    assert L.kvq_mfma_peak_probe(p, (1 << 20) + 1, 1, None) == kv.KVQ_EINVAL


def _layout(**kw):
    d = dict(batch=2, kv_heads=4, head_dim=128, capacity=1024, key_mode=kv.KEY_WINDOW,
             value_mode=kv.VAL_GROUP, n_centroids=0, qsac_topk=1, psac_rank=0, qsac_score=0,
             psac_format=0, centroid_key_split=0, n_modalities=1)
    d.update(kw)
    return kv.Layout(*[d[f] for f, _ in kv.Layout._fields_])


def test_layout_validation():
    chk = lambda **kw: kv.lib().kvq_layout_check(ctypes.byref(_layout(**kw)))
    assert chk() == kv.KVQ_OK
    assert chk(capacity=1000) == kv.KVQ_EINVAL
    assert chk(key_mode=kv.KEY_CENTROID, n_centroids=16, centroid_key_split=1) == kv.KVQ_OK
    assert chk(key_mode=kv.KEY_CENTROID, n_centroids=16, centroid_key_split=2) == kv.KVQ_EINVAL
    assert chk(centroid_key_split=2) == kv.KVQ_OK          # ignored for window keys
    assert chk(batch=0) == kv.KVQ_EINVAL
    assert chk(head_dim=96) == kv.KVQ_EUNSUPPORTED
    assert chk(key_mode=7) == kv.KVQ_EINVAL
    assert chk(key_mode=kv.KEY_CENTROID, n_centroids=0) == kv.KVQ_EUNSUPPORTED
    assert chk(key_mode=kv.KEY_CENTROID, n_centroids=300) == kv.KVQ_EUNSUPPORTED
    assert chk(key_mode=kv.KEY_CENTROID, n_centroids=16, psac_rank=8) == kv.KVQ_OK
    assert chk(key_mode=kv.KEY_CENTROID, n_centroids=16, psac_rank=4) == kv.KVQ_EUNSUPPORTED
    assert chk(psac_rank=8) == kv.KVQ_EUNSUPPORTED
    assert chk(key_mode=kv.KEY_CENTROID_QSAC, n_centroids=16, qsac_topk=9) == kv.KVQ_EINVAL
    assert chk(key_mode=kv.KEY_CENTROID_QSAC, n_centroids=2, qsac_topk=4) == kv.KVQ_EINVAL
    q = dict(key_mode=kv.KEY_CENTROID_QSAC, n_centroids=16, qsac_topk=4)
    assert chk(**q, qsac_score=kv.QSAC_RANGE) == kv.KVQ_OK
    assert chk(**q, qsac_score=2) == kv.KVQ_EINVAL
    assert chk(**q, psac_rank=8, psac_format=kv.PSAC_INT8) == kv.KVQ_OK
    assert chk(**q, psac_rank=8, psac_format=3) == kv.KVQ_EINVAL
    assert chk(key_mode=kv.KEY_CENTROID, n_centroids=16, qsac_score=5) == kv.KVQ_OK   # ignored
    # launch-grid and 32-bit row-offset limits
    assert chk(batch=1, kv_heads=1, capacity=1 << 24) == kv.KVQ_OK
    assert chk(batch=1, kv_heads=1, capacity=(1 << 24) + 64) == kv.KVQ_EUNSUPPORTED
    assert chk(batch=65535, kv_heads=1, capacity=64) == kv.KVQ_OK
    assert chk(batch=65536, kv_heads=1, capacity=64) == kv.KVQ_EUNSUPPORTED
    assert chk(batch=1, kv_heads=65536, capacity=64) == kv.KVQ_EUNSUPPORTED
    # per-modality rotations: 1..3 modalities
    assert chk(value_mode=kv.VAL_HADAMARD_MODAL, n_modalities=3) == kv.KVQ_OK
    assert chk(value_mode=kv.VAL_HADAMARD_MODAL, n_modalities=0) == kv.KVQ_EUNSUPPORTED
    assert chk(value_mode=kv.VAL_HADAMARD_MODAL, n_modalities=4) == kv.KVQ_EUNSUPPORTED
    assert chk(value_mode=3) == kv.KVQ_EINVAL
    assert chk(n_modalities=9) == kv.KVQ_OK                # ignored without the modal mode


def test_buffer_sizes():
    L = _layout()
    nb = lambda w: kv.lib().kvq_buffer_bytes(ctypes.byref(L), w)
    BH, T, D = 8, 1024, 128
    assert nb(0) == BH * T * D // 4                # k_codes
    assert nb(1) == BH * (T // 64) * D * 4         # window params
    assert nb(2) == BH * 64 * D * 2                # tail
    assert nb(3) == 0 and nb(4) == 0 and nb(7) == 0
    assert nb(8) == BH * T * D // 4 and nb(9) == BH * T * (D // 32) * 4
    L = _layout(key_mode=kv.KEY_CENTROID_QSAC, n_centroids=256, qsac_topk=4, psac_rank=8)
    assert nb(1) == BH * T * (D // 32) * 4
    assert nb(2) == 0 and nb(3) == BH * T and nb(4) == BH * 256 * D * 4
    assert nb(5) == BH * D * 4 and nb(6) == BH * D * 8 * 4 and nb(7) == BH * T * 8 * 2
    # INT8 PSAC: 8 codes + one fp16 scale per token-head
    L = _layout(key_mode=kv.KEY_CENTROID_QSAC, n_centroids=256, qsac_topk=4, psac_rank=8,
                psac_format=kv.PSAC_INT8)
    assert nb(7) == BH * T * 10
    assert nb(99) == 0
    assert nb(10) == 0 and nb(11) == 0
    L = _layout(value_mode=kv.VAL_HADAMARD_MODAL, n_modalities=3)
    assert nb(10) == 4 * 3 * (D // 32) * 4 and nb(11) == 2 * T


def _cache(**kw):
    L = _layout(**kw)
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced: validation fails first
    return kv.CacheStruct(L, *[fake] * len(kv.BUFFERS))


def test_append_validation_without_launch():
    L = kv.lib()
    c = _cache()
    p = ctypes.c_void_p(1 << 20)
    assert L.kv_quantize_append(None, p, p, 0, 1, None) == kv.KVQ_EINVAL
    assert L.kv_quantize_append(ctypes.byref(c), p, p, -1, 1, None) == kv.KVQ_EINVAL
    assert L.kv_quantize_append(ctypes.byref(c), p, p, 1000, 25, None) == kv.KVQ_ECAPACITY
    assert L.kv_quantize_append(ctypes.byref(c), None, p, 0, 1, None) == kv.KVQ_EINVAL
    assert L.kv_quantize_append(ctypes.byref(c), p, p, 5, 0, None) == kv.KVQ_OK   # no-op
    bad = _cache()
    bad.v_codes = None
    assert L.kv_quantize_append(ctypes.byref(bad), p, p, 0, 1, None) == kv.KVQ_EINVAL
    mis = _cache()
    mis.k_codes = ctypes.c_void_p((1 << 20) + 4)
    assert L.kv_quantize_append(ctypes.byref(mis), p, p, 0, 1, None) == kv.KVQ_EINVAL


def test_attention_validation_without_launch():
    L = kv.lib()
    c = _cache()
    p = ctypes.c_void_p(1 << 20)
    call = lambda n=100, hq=8, od=kv.F32, ws=p, wsb=1 << 30, qd=kv.F32: L.attn_int2_decode(
        ctypes.byref(c), n, p, qd, hq, 0.1, p, od, None, ws, wsb, None)
    assert call(hq=6) == kv.KVQ_EINVAL
    assert call(hq=4 * 3) == kv.KVQ_EUNSUPPORTED
    assert call(n=0) == kv.KVQ_EINVAL
    assert call(n=2000) == kv.KVQ_ECAPACITY
    assert call(od=7) == kv.KVQ_EINVAL
    assert call(qd=9) == kv.KVQ_EINVAL
    assert call(wsb=16) == kv.KVQ_EWORKSPACE
    assert call(ws=None) == kv.KVQ_EWORKSPACE
    need = L.attn_int2_decode_workspace(ctypes.byref(c.layout), 8, 100)
    assert need > 0 and need % 4 == 0
    assert L.attn_int2_chunk(ctypes.byref(c), 100, p, 0, 8, 0.1, p, kv.F32, None, p, 1 << 30,
                             None) == kv.KVQ_EINVAL
    # the top-1 diagnostic: same cache / head / length checks, no workspace
    top1 = lambda n=100, ql=5, hq=8, idx=p: L.attn_int2_top1(ctypes.byref(c), n, p, ql, hq, idx,
                                                             None, None)
    assert top1(ql=0) == kv.KVQ_EINVAL
    assert top1(hq=6) == kv.KVQ_EINVAL
    assert top1(n=0) == kv.KVQ_EINVAL
    assert top1(n=2000) == kv.KVQ_ECAPACITY
    assert top1(idx=None) == kv.KVQ_EINVAL
    # more than 65535 query heads (grid y) is refused before any launch
    wide = _cache(batch=1, kv_heads=16384, capacity=64)
    assert L.attn_int2_decode(ctypes.byref(wide), 64, p, kv.F32, 16384 * 8, 0.1, p, kv.F32, None,
                              p, 1 << 40, None) == kv.KVQ_EUNSUPPORTED
    assert L.attn_int2_chunk(ctypes.byref(wide), 64, p, 4, 16384 * 8, 0.1, p, kv.F32, None,
                             p, 1 << 40, None) == kv.KVQ_EUNSUPPORTED


def test_noalloc_decode_validation_without_launch():
    """The allocation-free decode checks like attn_int2_decode and refuses,
    before any launch, a call whose split partials exceed its fixed
    scratch buffer."""
    L = kv.lib()
    p = ctypes.c_void_p(1 << 20)
    c = _cache()
    call = lambda cc=c, n=100, hq=8, od=kv.F32, qd=kv.F32: L.attn_int2_decode_noalloc(
        ctypes.byref(cc), n, p, qd, hq, 0.1, p, od, None, None)
    assert call(hq=6) == kv.KVQ_EINVAL
    assert call(hq=12) == kv.KVQ_EUNSUPPORTED
    assert call(n=0) == kv.KVQ_EINVAL
    assert call(n=2000) == kv.KVQ_ECAPACITY
    assert call(od=7) == kv.KVQ_EINVAL
    assert call(qd=9) == kv.KVQ_EINVAL
    assert L.attn_int2_decode_noalloc(None, 100, p, kv.F32, 8, 0.1, p, kv.F32, None, None) == kv.KVQ_EINVAL
    big = _cache(batch=64, kv_heads=8, capacity=1 << 20)
    need = L.attn_int2_decode_workspace(ctypes.byref(big.layout), 64, 1 << 20)
    assert need > kv.NOALLOC_SCRATCH_BYTES
    assert call(cc=big, n=1 << 20, hq=64) == kv.KVQ_ESCRATCH
    assert L.kvq_status_string(kv.KVQ_ESCRATCH).startswith(b"exceeds the fixed scratch")


def test_python_wrappers_check_shapes_before_any_call():
    """The bindings size-check what the C ABI cannot (q, out, lse against
    the layout) and raise ValueError before reaching the library; CPU
    tensors suffice because the checks come first."""
    import torch
    c = kv.KVCache(2, 4, 128, 1024, device="cpu")
    q = torch.zeros((2, 8, 128))
    with pytest.raises(ValueError, match="batch"):
        kv.attn_int2_decode(c, 100, torch.zeros((3, 8, 128)), 0.1)
    with pytest.raises(ValueError, match="head_dim"):
        kv.attn_int2_decode(c, 100, torch.zeros((2, 8, 64)), 0.1)
    with pytest.raises(ValueError, match="dimensions"):
        kv.attn_int2_decode(c, 100, torch.zeros((2, 1, 8, 128)), 0.1)
    with pytest.raises(ValueError, match="out must have shape"):
        kv.attn_int2_decode(c, 100, q, 0.1, out=torch.zeros((2, 8, 64)))
    with pytest.raises(ValueError, match="out must be one of"):
        kv.attn_int2_decode(c, 100, q, 0.1, out=torch.zeros((2, 8, 128), dtype=torch.float16))
    with pytest.raises(ValueError, match="out must be contiguous"):
        kv.attn_int2_decode(c, 100, q, 0.1, out=torch.zeros((2, 128, 8)).transpose(1, 2))
    with pytest.raises(ValueError, match="lse must have shape"):
        kv.attn_int2_decode(c, 100, q, 0.1, lse=torch.zeros((2, 4)))
    with pytest.raises(ValueError, match="lse must be one of"):
        kv.attn_int2_decode(c, 100, q, 0.1, lse=torch.zeros((2, 8), dtype=torch.float64))
    with pytest.raises(ValueError, match="out must have shape"):
        kv.attn_int2_decode_noalloc(c, 100, q, 0.1, out=torch.zeros((2, 8, 127)))
    qc = torch.zeros((2, 5, 8, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="q must be one of"):
        kv.attn_int2_chunk(c, 100, qc.float(), 0.1)
    with pytest.raises(ValueError, match="batch"):
        kv.attn_int2_chunk(c, 100, torch.zeros((1, 5, 8, 128), dtype=torch.bfloat16), 0.1)
    with pytest.raises(ValueError, match="lse must have shape"):
        kv.attn_int2_chunk(c, 100, qc, 0.1, lse=torch.zeros((2, 5, 7)))
    with pytest.raises(ValueError, match="out must have shape"):
        kv.attn_int2_chunk(c, 100, qc, 0.1, out=torch.zeros((2, 5, 8, 64)))
    with pytest.raises(ValueError, match="head_dim"):
        kv.attn_int2_top1(c, 100, torch.zeros((2, 5, 8, 64), dtype=torch.bfloat16))
    # shapes right, but host tensors: refused by the device check
    with pytest.raises(ValueError, match="device"):
        kv.attn_int2_decode(c, 100, q, 0.1)


def test_assign_validation_without_launch():
    L = kv.lib()
    p = ctypes.c_void_p(1 << 20)
    assert L.kv_cluster_assign(p, -1, 128, 128, p, 16, None, 1, p, None) == kv.KVQ_EINVAL
    assert L.kv_cluster_assign(p, 10, 96, 96, p, 16, None, 1, p, None) == kv.KVQ_EUNSUPPORTED
    assert L.kv_cluster_assign(p, 10, 128, 128, p, 0, None, 1, p, None) == kv.KVQ_EUNSUPPORTED
    assert L.kv_cluster_assign(p, 10, 128, 100, p, 16, None, 1, p, None) == kv.KVQ_EINVAL
    assert L.kv_cluster_assign(p, 10, 128, 128, p, 16, p, 9, p, None) == kv.KVQ_EINVAL
    assert L.kv_cluster_assign(p, 0, 128, 128, p, 16, None, 1, p, None) == kv.KVQ_OK


def test_kmeans_validation_without_launch():
    L = kv.lib()
    p = ctypes.c_void_p(1 << 20)
    ws = L.kv_kmeans_workspace(2, 3, 1000)
    assert ws >= 24000 and ws % 256 == 0
    assert L.kv_kmeans_workspace(1, 1, -1) == 0

    def call(n=1000, B=2, H=3, D=128, ks=384, hs=128, bs=384000, C=16, it=2, w=p, wsb=ws):
        return L.kv_kmeans(p, B, n, H, D, ks, hs, bs, p, C, it, p, w, wsb, None)
    assert call(n=-1) == kv.KVQ_EINVAL
    assert call(it=-1) == kv.KVQ_EINVAL
    assert call(B=-1) == kv.KVQ_EINVAL
    assert call(D=96, ks=288) == kv.KVQ_EUNSUPPORTED
    assert call(C=300) == kv.KVQ_EUNSUPPORTED
    assert call(ks=100) == kv.KVQ_EINVAL
    assert call(hs=-8) == kv.KVQ_EINVAL
    assert call(wsb=ws - 256) == kv.KVQ_EWORKSPACE
    assert call(w=None) == kv.KVQ_EWORKSPACE
    assert call(n=0, w=None, wsb=0) == kv.KVQ_OK
    assert call(H=70000, bs=70000 * 128 * 1000) == kv.KVQ_EUNSUPPORTED
