"""kvint2: 2-bit KV cache for MI355X -- Python binding of libkvint2.so.

This module only marshals arguments: every step of quantisation and
attention runs in the HIP kernels behind the C ABI declared in
``include/kvint2.h``.  PyTorch provides device memory and the current
stream.  There is no fallback path: if ``libkvint2.so`` is missing or
cannot be loaded the calls raise.

Methods (web pages, cited by title and section):
  "QuantWM: Training-Free 2-bit KV Cache Quantization for Stable Video World
   Models" -- "QuantWM Framework" 1 (QSAC) and 2 (PSAC);
  "OmniKVQuant: KV Cache Quantization for Omni-LLMs" -- English abstract
   (per-window key ranges, rotated values, fused 2-bit decode).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvint2.so")

KVQ_OK, KVQ_EINVAL, KVQ_EUNSUPPORTED, KVQ_ECAPACITY, KVQ_EWORKSPACE, KVQ_EHIP = 0, -1, -2, -3, -4, -5
KVQ_ESCRATCH = -6
NOALLOC_SCRATCH_BYTES = 16 << 20   # KVQ_NOALLOC_SCRATCH_BYTES
KEY_WINDOW, KEY_CENTROID, KEY_CENTROID_QSAC = 0, 1, 2
VAL_GROUP, VAL_HADAMARD, VAL_HADAMARD_MODAL = 0, 1, 2
F32, BF16 = 0, 1
QSAC_EXACT, QSAC_RANGE = 0, 1     # QSAC perturbation estimate
PSAC_F16, PSAC_INT8 = 0, 1        # PSAC coefficient storage
GROUP, WINDOW = 32, 64

BUFFERS = ("k_codes", "k_params", "k_tail", "k_idx", "centroids", "sens_w", "psac_basis",
           "k_psac", "v_codes", "v_params", "v_signs", "v_modality")


class KVQError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = lib().kvq_status_string(status).decode()
        super().__init__(f"{what}: {msg} (status {status})")
        self.status = status


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "kv_heads", "head_dim", "capacity",
                                               "key_mode", "value_mode", "n_centroids",
                                               "qsac_topk", "psac_rank", "qsac_score",
                                               "psac_format", "centroid_key_split",
                                               "n_modalities")]


class CacheStruct(ctypes.Structure):
    _fields_ = [("layout", Layout)] + [(n, ctypes.c_void_p) for n in BUFFERS]


_lib = None


def lib():
    """The loaded libkvint2.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pL, pC = ctypes.POINTER(Layout), ctypes.POINTER(CacheStruct)
    L.kvq_status_string.argtypes = [ctypes.c_int]
    L.kvq_status_string.restype = ctypes.c_char_p
    L.kvq_layout_check.argtypes = [pL]
    L.kvq_layout_check.restype = ctypes.c_int
    L.kvq_buffer_bytes.argtypes = [pL, i32]
    L.kvq_buffer_bytes.restype = sz
    L.kv_quantize_append.argtypes = [pC, vp, vp, i32, i32, vp]
    L.kv_quantize_append.restype = ctypes.c_int
    L.kv_cluster_assign.argtypes = [vp, i64, i32, i64, vp, i32, vp, i32, vp, vp]
    L.kv_cluster_assign.restype = ctypes.c_int
    L.kv_kmeans_workspace.argtypes = [i32, i32, i64]
    L.kv_kmeans_workspace.restype = sz
    L.kv_kmeans.argtypes = [vp, i32, i64, i32, i32, i64, i64, i64, vp, i32, i32, vp, vp, sz, vp]
    L.kv_kmeans.restype = ctypes.c_int
    L.attn_int2_decode_workspace.argtypes = [pL, i32, i32]
    L.attn_int2_decode_workspace.restype = sz
    L.attn_int2_decode.argtypes = [pC, i32, vp, i32, i32, ctypes.c_float, vp, i32, vp, vp, sz, vp]
    L.attn_int2_decode.restype = ctypes.c_int
    L.attn_int2_decode_noalloc.argtypes = [pC, i32, vp, i32, i32, ctypes.c_float, vp, i32, vp, vp]
    L.attn_int2_decode_noalloc.restype = ctypes.c_int
    L.attn_int2_chunk_workspace.argtypes = [pL, i32, i32, i32]
    L.attn_int2_chunk_workspace.restype = sz
    L.attn_int2_chunk.argtypes = [pC, i32, vp, i32, i32, ctypes.c_float, vp, i32, vp, vp, sz, vp]
    L.attn_int2_chunk.restype = ctypes.c_int
    L.attn_int2_top1.argtypes = [pC, i32, vp, i32, i32, vp, vp, vp]
    L.attn_int2_top1.restype = ctypes.c_int
    L.kvq_mfma_peak_probe.argtypes = [vp, i32, i32, vp]
    L.kvq_mfma_peak_probe.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int, what: str) -> None:
    if status != KVQ_OK:
        raise KVQError(status, what)


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_cuda(t: torch.Tensor, name: str, dtype=None):
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device tensor")


def _need_shape(t: torch.Tensor, name: str, shape, dtypes) -> None:
    """Shape and dtype of a tensor the C ABI cannot size-check (it reads or
    writes exactly this many elements): checked before anything else."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _attention_io(cache: "KVCache", q: torch.Tensor, q_rank: int, qdtypes, out, out_dtype, lse,
                  lse_shape):
    """Validates q against the cache layout and the optional out / lse
    against q, and allocates out when it is None."""
    L = cache.layout
    if q.dim() != q_rank:
        raise ValueError(f"q must have {q_rank} dimensions, got {tuple(q.shape)}")
    if q.dtype not in qdtypes:
        raise ValueError(f"q must be one of {qdtypes}, got {q.dtype}")
    if q.shape[0] != L.batch or q.shape[-1] != L.head_dim:
        raise ValueError(f"q must be [batch={L.batch}, ..., head_dim={L.head_dim}], got {tuple(q.shape)}")
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=out_dtype, device=q.device)
    _need_shape(out, "out", q.shape, (torch.float32, torch.bfloat16))
    if lse is not None:   # any contiguous f32 tensor of that many elements
        want = 1
        for x in lse_shape:
            want *= int(x)
        if lse.numel() != want:
            raise ValueError(f"lse must have shape {tuple(lse_shape)} ({want} elements), "
                             f"got {tuple(lse.shape)}")
        _need_shape(lse, "lse", lse.shape, (torch.float32,))
    _need_cuda(q, "q")
    _need_cuda(out, "out")
    if lse is not None:
        _need_cuda(lse, "lse")
    return out


class KVCache:
    """One layer's packed INT2 cache: device buffers in the library layout.

    Buffers (views, C order): k_codes u8 [B,H,T,D/4]; k_params i32 (u32 words)
    [B,H,T/64,D] for window keys or [B,H,T,D/32] for centroid keys; k_tail
    i16 (bf16 bits) [B,H,64,D]; k_idx u8 [B,H,T]; centroids f32 [B,H,C,D];
    sens_w f32 [B,H,D]; psac_basis f32 [B,H,D,R]; k_psac i16 (fp16 bits)
    [B,H,T,R], or with psac_format PSAC_INT8 a u8 buffer of B*H*T*(R+2)
    bytes viewed as k_psac8 i8 [B,H,T,R] and k_psac_sc i16 (fp16 bits)
    [B,H,T]; v_codes u8 [B,H,T/64,D,16] (per 64-token tile, channel-major:
    token t of the tile, channel c in byte 16c + t/4, bits 2(t%4));
    v_params i32 [B,H,T,D/32]; with value_mode VAL_HADAMARD_MODAL, v_signs i32
    [H,M,D/32] (sign bits of each head's per-modality rotation, bit c % 32 of
    word c / 32 set = -1) and v_modality u8 [B,T] (modality of each token).
    Calibration inputs (centroids, sens_w, psac_basis) and the modal inputs
    (v_signs, and v_modality before each append) are filled by the caller.
    """

    def __init__(self, batch: int, kv_heads: int, head_dim: int, capacity: int,
                 key_mode: int = KEY_WINDOW, value_mode: int = VAL_GROUP,
                 n_centroids: int = 0, qsac_topk: int = 1, psac_rank: int = 0,
                 qsac_score: int = QSAC_EXACT, psac_format: int = PSAC_F16,
                 centroid_key_split: bool = False, n_modalities: int = 1, device="cuda"):
        self.layout = Layout(batch, kv_heads, head_dim, capacity, key_mode, value_mode,
                             n_centroids, qsac_topk, psac_rank, qsac_score, psac_format,
                             int(bool(centroid_key_split)), int(n_modalities))
        _check(lib().kvq_layout_check(ctypes.byref(self.layout)), "layout")
        B, H, D, T = batch, kv_heads, head_dim, capacity
        shapes = {
            "k_codes": ((B, H, T, D // 4), torch.uint8),
            "k_params": (((B, H, T // WINDOW, D) if key_mode == KEY_WINDOW
                          else (B, H, T, D // GROUP)), torch.int32),
            "k_tail": ((B, H, WINDOW, D), torch.int16),
            "k_idx": ((B, H, T), torch.uint8),
            "centroids": ((B, H, max(n_centroids, 1), D), torch.float32),
            "sens_w": ((B, H, D), torch.float32),
            "psac_basis": ((B, H, D, max(psac_rank, 1)), torch.float32),
            "k_psac": (((B * H * T * (psac_rank + 2),) if psac_format == PSAC_INT8
                        else (B, H, T, max(psac_rank, 1))),
                       torch.uint8 if psac_format == PSAC_INT8 else torch.int16),
            "v_codes": ((B, H, T // WINDOW, D, 16), torch.uint8),
            "v_params": ((B, H, T, D // GROUP), torch.int32),
            "v_signs": ((H, max(n_modalities, 1), D // 32), torch.int32),
            "v_modality": ((B, T), torch.uint8),
        }
        self.buffers = {}
        for i, name in enumerate(BUFFERS):
            nbytes = lib().kvq_buffer_bytes(ctypes.byref(self.layout), i)
            if nbytes == 0:
                setattr(self, name, None)
                continue
            shape, dt = shapes[name]
            t = torch.zeros(shape, dtype=dt, device=device)
            assert t.numel() * t.element_size() == nbytes, name
            setattr(self, name, t)
            self.buffers[name] = t
        self.k_psac8 = self.k_psac_sc = None
        if self.k_psac is not None and psac_format == PSAC_INT8:
            n8 = B * H * T * psac_rank
            self.k_psac8 = self.k_psac[:n8].view(torch.int8).view(B, H, T, psac_rank)
            self.k_psac_sc = self.k_psac[n8:].view(torch.int16).view(B, H, T)

    def struct(self) -> CacheStruct:
        return CacheStruct(self.layout, *[_ptr(getattr(self, n)) for n in BUFFERS])

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.buffers.values())


def kv_quantize_append(cache: KVCache, k: torch.Tensor, v: torch.Tensor, cur_len: int,
                       stream=None) -> None:
    """Quantise k, v (bf16 [B, n_new, H, D]) into positions cur_len.. of every
    sequence of the cache."""
    _need_cuda(k, "k", torch.bfloat16)
    _need_cuda(v, "v", torch.bfloat16)
    L = cache.layout
    if tuple(k.shape) != (L.batch, k.shape[1], L.kv_heads, L.head_dim) or v.shape != k.shape:
        raise ValueError("k/v must be [batch, n_new, kv_heads, head_dim]")
    cs = cache.struct()
    _check(lib().kv_quantize_append(ctypes.byref(cs), _ptr(k), _ptr(v), int(cur_len),
                                    int(k.shape[1]), _stream(stream)), "kv_quantize_append")


def kv_cluster_assign(keys: torch.Tensor, centroids: torch.Tensor, sens_w=None, topk: int = 1,
                      out=None, stream=None) -> torch.Tensor:
    """Centroid index (i32) of each bf16 key row keys[i, :D] (rows may be
    strided); centroids f32 [C, D]; sens_w f32 [D] selects the QSAC rule."""
    if keys.dtype != torch.bfloat16 or not keys.is_cuda or keys.dim() != 2 or keys.stride(1) != 1:
        raise ValueError("keys must be a bf16 device matrix with unit column stride")
    _need_cuda(centroids, "centroids", torch.float32)
    n, D = keys.shape
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=keys.device)
    if sens_w is not None:
        _need_cuda(sens_w, "sens_w", torch.float32)
    _check(lib().kv_cluster_assign(_ptr(keys), n, D, keys.stride(0), _ptr(centroids),
                                   centroids.shape[0], _ptr(sens_w), int(topk), _ptr(out),
                                   _stream(stream)), "kv_cluster_assign")
    return out


def kv_kmeans(keys: torch.Tensor, centroids: torch.Tensor, iters: int, assign_out=None,
              workspace=None, stream=None):
    """Lloyd k-means of bf16 keys [B, n, H, D] (one table per (b, h); any
    strides with a unit last one), or of one key matrix [n, D], starting from
    centroids f32 [B, H, C, D] (or [C, D]), which are updated in place.
    Returns (centroids, assignment i32 [B, H, n] (or [n]) of the last round)."""
    if keys.dtype != torch.bfloat16 or not keys.is_cuda or keys.stride(-1) != 1:
        raise ValueError("keys must be a bf16 device tensor with unit last stride")
    if keys.dim() == 2:
        k4 = keys[None, :, None, :]
        c4 = centroids[None, None]
    elif keys.dim() == 4:
        k4, c4 = keys, centroids
    else:
        raise ValueError("keys must be [n, D] or [B, n, H, D]")
    _need_cuda(centroids, "centroids", torch.float32)
    B, n, H, D = k4.shape
    if tuple(c4.shape[:2]) != (B, H) or c4.shape[3] != D or not centroids.is_contiguous():
        raise ValueError("centroids must be contiguous f32 [B, H, C, D] ([C, D] for 2-D keys)")
    if assign_out is None:
        assign_out = torch.empty((B, H, n) if keys.dim() == 4 else (n,), dtype=torch.int32,
                                 device=keys.device)
    if workspace is None:
        workspace = torch.empty(max(int(lib().kv_kmeans_workspace(B, H, n)), 16), dtype=torch.uint8,
                                device=keys.device)
    _check(lib().kv_kmeans(_ptr(keys), B, n, H, D, k4.stride(1), k4.stride(2), k4.stride(0),
                           _ptr(centroids), c4.shape[2], int(iters), _ptr(assign_out),
                           _ptr(workspace), workspace.numel(), _stream(stream)), "kv_kmeans")
    return centroids, assign_out


def decode_workspace(cache: KVCache, q_heads: int, n_tokens: int, device="cuda") -> torch.Tensor:
    n = lib().attn_int2_decode_workspace(ctypes.byref(cache.layout), q_heads, n_tokens)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def attn_int2_decode(cache: KVCache, n_tokens: int, q: torch.Tensor, scale: float,
                     out=None, out_dtype=torch.float32, lse=None, workspace=None,
                     stream=None) -> torch.Tensor:
    """q [B, Hq, D] (f32 or bf16) against the first n_tokens cached tokens."""
    out = _attention_io(cache, q, 3, (torch.float32, torch.bfloat16), out, out_dtype, lse,
                        q.shape[:2])
    qd = {torch.float32: F32, torch.bfloat16: BF16}[q.dtype]
    B, Hq, D = q.shape
    od = {torch.float32: F32, torch.bfloat16: BF16}[out.dtype]
    if workspace is None:
        workspace = decode_workspace(cache, Hq, n_tokens, q.device)
    _need_cuda(workspace, "workspace")
    cs = cache.struct()
    _check(lib().attn_int2_decode(ctypes.byref(cs), int(n_tokens), _ptr(q), qd, Hq, float(scale),
                                  _ptr(out), od, _ptr(lse), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)),
           "attn_int2_decode")
    return out


def attn_int2_decode_noalloc(cache: KVCache, n_tokens: int, q: torch.Tensor, scale: float,
                             out: torch.Tensor, lse=None, stream=None) -> torch.Tensor:
    """attn_int2_decode through the allocation-free entry point: the split
    partials live in the library's fixed per-device scratch buffer, so the
    call allocates nothing (out, and lse if wanted, are the caller's).
    Calls that overlap on one device race on that buffer."""
    out = _attention_io(cache, q, 3, (torch.float32, torch.bfloat16), out, None, lse, q.shape[:2])
    qd = {torch.float32: F32, torch.bfloat16: BF16}[q.dtype]
    od = {torch.float32: F32, torch.bfloat16: BF16}[out.dtype]
    cs = cache.struct()
    _check(lib().attn_int2_decode_noalloc(ctypes.byref(cs), int(n_tokens), _ptr(q), qd,
                                          q.shape[1], float(scale), _ptr(out), od, _ptr(lse),
                                          _stream(stream)), "attn_int2_decode_noalloc")
    return out


def chunk_workspace(cache: KVCache, q_len: int, q_heads: int, n_tokens: int,
                    device="cuda") -> torch.Tensor:
    n = lib().attn_int2_chunk_workspace(ctypes.byref(cache.layout), q_len, q_heads, n_tokens)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def attn_int2_top1(cache: KVCache, n_tokens: int, q: torch.Tensor, logits: bool = False,
                   stream=None):
    """Each query row's highest-logit cached token (q bf16 [B, Lq, Hq, D]):
    i32 [B, Hq, Lq], and with logits=True also the f32 logits."""
    L = cache.layout
    if q.dim() != 4 or q.shape[0] != L.batch or q.shape[3] != L.head_dim:
        raise ValueError(f"q must be [batch={L.batch}, Lq, Hq, head_dim={L.head_dim}], got {tuple(q.shape)}")
    _need_cuda(q, "q", torch.bfloat16)
    B, Lq, Hq, D = q.shape
    idx = torch.empty((B, Hq, Lq), dtype=torch.int32, device=q.device)
    lg = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device) if logits else None
    cs = cache.struct()
    _check(lib().attn_int2_top1(ctypes.byref(cs), int(n_tokens), _ptr(q), Lq, Hq, _ptr(idx),
                                _ptr(lg), _stream(stream)), "attn_int2_top1")
    return (idx, lg) if logits else idx


def attn_int2_chunk(cache: KVCache, n_tokens: int, q: torch.Tensor, scale: float,
                    out=None, out_dtype=torch.float32, lse=None, workspace=None,
                    stream=None) -> torch.Tensor:
    """q bf16 [B, Lq, Hq, D] against the first n_tokens cached tokens."""
    out = _attention_io(cache, q, 4, (torch.bfloat16,), out, out_dtype, lse,
                        (q.shape[0], q.shape[2], q.shape[1]))
    B, Lq, Hq, D = q.shape
    od = {torch.float32: F32, torch.bfloat16: BF16}[out.dtype]
    if workspace is None:
        workspace = chunk_workspace(cache, Lq, Hq, n_tokens, q.device)
    _need_cuda(workspace, "workspace")
    cs = cache.struct()
    _check(lib().attn_int2_chunk(ctypes.byref(cs), int(n_tokens), _ptr(q), Lq, Hq, float(scale),
                                 _ptr(out), od, _ptr(lse), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "attn_int2_chunk")
    return out


def mfma_peak_probe(blocks: int, iters: int, out: torch.Tensor = None, stream=None) -> float:
    """Enqueues the matrix-core rate probe (include/kvprobe.h) and returns
    the flops one launch performs; out: f32 device [blocks * 256]."""
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    _need_cuda(out, "out", torch.float32)
    if out.numel() < blocks * 256:
        raise ValueError(f"out must hold {blocks * 256} floats, got {out.numel()}")
    _check(lib().kvq_mfma_peak_probe(_ptr(out), int(blocks), int(iters), _stream(stream)),
           "kvq_mfma_peak_probe")
    return float(blocks) * 4 * iters * 8 * 16384
