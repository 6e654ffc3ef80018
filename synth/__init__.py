"""Seeded synthetic workloads for the INT2 KV-cache path.

Only input tensors are made here; none of the quantizer's or the attention's
arithmetic lives in this package.  The CPU oracle and the GPU library both
consume these buffers.  bf16 tensors are returned as numpy ``uint16`` bit
patterns; fp32/fp64 tensors as ordinary numpy floats.

Streams (counter-based SplitMix64, see ``synth.c``): 1 K noise, 2 V noise,
3 queries, 4 calibration queries, 5 k-means initial picks, 6 per-channel
key scales, 7 query principal subspace.  The workload seed is
``0x5EED0000 + workload number``.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

SEED_BASE = 0x5EED0000
S_K, S_V, S_Q, S_QCAL, S_KMEANS, S_SIGMA, S_SUBSPACE = 1, 2, 3, 4, 5, 6, 7

FRAME_ROWS, FRAME_COLS = 30, 52          # 1560-token latent frame
FRAME_TOKENS = FRAME_ROWS * FRAME_COLS


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, i32, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    vp = ctypes.c_void_p
    lib.synth_uniform.argtypes = [u64, u64, u64, i64, vp]
    lib.synth_gauss.argtypes = [u64, u64, u64, i64, vp]
    lib.synth_round_bf16.argtypes = [vp, i64, vp]
    lib.synth_llm.argtypes = [u64, u64, i32, i32, i32, i32, i64, vp, i32, dbl, vp]
    lib.synth_video.argtypes = [u64, u64, i32, i32, i32, i32, i64, dbl, vp]
    for f in (lib.synth_uniform, lib.synth_gauss, lib.synth_round_bf16,
              lib.synth_llm, lib.synth_video):
        f.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def seed_for(workload: int) -> int:
    return SEED_BASE + int(workload)


def uniform(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(int(n), np.float64)
    _load().synth_uniform(seed, stream, offset, int(n), _ptr(out))
    return out


def gauss(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(int(n), np.float64)
    _load().synth_gauss(seed, stream, offset, int(n), _ptr(out))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().synth_round_bf16(_ptr(x), x.size, _ptr(out))
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (plumbing for tests and reports)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def llm_sigma(seed: int, H: int, D: int, lo: float = 0.3, hi: float = 10.0) -> np.ndarray:
    """Per (kv head, channel) key scale, log-uniform on [lo, hi] (stream 6)."""
    u = uniform(seed, S_SIGMA, H * D)
    return np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))).reshape(H, D)


def llm(seed: int, stream: int, B: int, T: int, H: int, D: int, pos0: int,
        sigma: np.ndarray | None = None, rope: bool = False,
        theta: float = 1e4) -> np.ndarray:
    """bf16 bits [B][T][H][D] of N(0,1) draws at absolute positions
    pos0..pos0+T-1, optionally scaled per (head, channel) and rotated by
    RoPE (half-split pairs (c, c+D/2), angle pos * theta^(-2c/D))."""
    out = np.empty((B, T, H, D), np.uint16)
    sg = None
    if sigma is not None:
        sigma = np.ascontiguousarray(sigma, np.float64)
        assert sigma.shape == (H, D)
        sg = _ptr(sigma)
    _load().synth_llm(seed, stream, B, T, H, D, pos0, sg, 1 if rope else 0,
                      float(theta), _ptr(out))
    return out


def video(seed: int, stream: int, H: int, D: int, T: int, rho: float = 0.9,
          rows: int = FRAME_ROWS, cols: int = FRAME_COLS) -> np.ndarray:
    """bf16 bits [1][T][H][D]: AR(1) across frames (coefficient rho) of
    spatially smoothed unit-variance noise on rows x cols latent frames."""
    assert rows * cols <= 4096
    out = np.empty((T, H, D), np.uint16)
    _load().synth_video(seed, stream, H, D, rows, cols, T, float(rho), _ptr(out))
    return out.reshape(1, T, H, D)


def kmeans_init(seed: int, n: int, C: int, b: int = 0, h: int = 0, H: int = 1) -> np.ndarray:
    """C distinct token indices in [0, n): the first C slots of a partial
    Fisher-Yates shuffle driven by stream 5 (offset per (b, h))."""
    assert 1 <= C <= n
    u = uniform(seed, S_KMEANS, C, offset=((b * H + h) << 20))
    a = np.arange(n, dtype=np.int64)
    for i in range(C):
        j = i + int(math.floor(u[i] * (n - i)))
        a[i], a[j] = a[j], a[i]
    return a[:C].copy()


def lowrank_queries(seed: int, stream: int, n: int, H: int, D: int, rank: int = 8,
                    a: float = 11.05, noise_var: float = 0.3093) -> np.ndarray:
    """fp64 [n][H][D]: q = U0 (sqrt(a) z) + sqrt(noise_var) e with U0 a per-head
    random orthonormal D x rank basis (QR of a stream-7 Gaussian), z ~ N(0, I_rank)
    and e ~ N(0, I_D).  With the defaults E|q|^2 = D and ~71% of the energy
    lies in span(U0)."""
    q = np.empty((n, H, D), np.float64)
    per = rank + D
    g = gauss(seed, stream, n * H * per).reshape(n, H, per)
    for h in range(H):
        basis = gauss(seed, S_SUBSPACE, D * rank, offset=h * D * rank).reshape(D, rank)
        U0, _ = np.linalg.qr(basis)
        q[:, h, :] = (math.sqrt(a) * g[:, h, :rank]) @ U0.T + math.sqrt(noise_var) * g[:, h, rank:]
    return q


# ---------------------------------------------------------------------------
# The five workloads.  Each returns a dict of numpy arrays plus the sizes.
# ``scale`` dicts let tests shrink a workload while keeping its law.
# ---------------------------------------------------------------------------

def toy_single_head(T: int = 512, D: int = 64, C: int = 16, workload: int = 1):
    """head_dim 64, 512 tokens, K/V ~ N(0,1), 4 fixed K outlier channels x8,
    16 centroids, one fp32 query."""
    seed = seed_for(workload)
    sigma = np.ones((1, D))
    for c in (5, 21, 37, 53):
        if c < D:
            sigma[0, c] = 8.0
    K = llm(seed, S_K, 1, T, 1, D, 0, sigma=sigma)
    V = llm(seed, S_V, 1, T, 1, D, 0)
    q = gauss(seed, S_Q, D).astype(np.float32).reshape(1, 1, D)
    init = kmeans_init(seed, T, C)
    return dict(seed=seed, B=1, Hkv=1, Hq=1, D=D, T=T, C=C, K=K, V=V, q=q,
                kmeans_init=init[None, None, :])


def llm_decode(B: int = 16, Hkv: int = 8, Hq: int = 32, D: int = 128, T: int = 32768,
               workload: int = 2):
    """GQA decode: K = RoPE(sigma * z) with log-uniform per-channel sigma,
    V ~ N(0,1), one query token per sequence at position T (RoPE'd)."""
    seed = seed_for(workload)
    sigma = llm_sigma(seed, Hkv, D)
    K = llm(seed, S_K, B, T, Hkv, D, 0, sigma=sigma, rope=True)
    V = llm(seed, S_V, B, T, Hkv, D, 0)
    Q = llm(seed, S_Q, B, 1, Hq, D, T, rope=True).reshape(B, Hq, D)
    return dict(seed=seed, B=B, Hkv=Hkv, Hq=Hq, D=D, T=T, K=K, V=V, q=Q)


def video_chunk(H: int = 40, D: int = 128, T: int = 31200, Lq: int = 4680, C: int = 256,
                workload: int = 3):
    """Video world-model chunk: cached K/V of T tokens, the chunk's own Lq K/V
    tokens (next frames of the same processes) and Lq queries from an
    independent process."""
    seed = seed_for(workload)
    K = video(seed, S_K, H, D, T + Lq)
    V = video(seed, S_V, H, D, T + Lq)
    Q = video(seed, S_Q, H, D, Lq)
    init = np.stack([kmeans_init(seed, T, C, 0, h, H) for h in range(H)])[None]
    return dict(seed=seed, B=1, Hkv=H, Hq=H, D=D, T=T, Lq=Lq, C=C,
                K=np.ascontiguousarray(K[:, :T]), V=np.ascontiguousarray(V[:, :T]),
                K_new=np.ascontiguousarray(K[:, T:]), V_new=np.ascontiguousarray(V[:, T:]),
                q=Q, kmeans_init=init)


def long_history(H: int = 40, D: int = 128, T: int = 93600, Lq: int = 1560, workload: int = 4):
    """Long-history step: the LLM law with H heads at positions 0..T-1, plus a
    new frame of Lq tokens (K/V to append, queries) at positions T..T+Lq-1."""
    seed = seed_for(workload)
    sigma = llm_sigma(seed, H, D)
    K = llm(seed, S_K, 1, T, H, D, 0, sigma=sigma, rope=True)
    V = llm(seed, S_V, 1, T, H, D, 0)
    K_new = llm(seed, S_K, 1, Lq, H, D, T, sigma=sigma, rope=True)
    V_new = llm(seed, S_V, 1, Lq, H, D, T)
    Q = llm(seed, S_Q, 1, Lq, H, D, T, rope=True)
    return dict(seed=seed, B=1, Hkv=H, Hq=H, D=D, T=T, Lq=Lq, K=K, V=V,
                K_new=K_new, V_new=V_new, q=Q)


def sensitivity_aware(H: int = 40, D: int = 128, T: int = 65536, Lq: int = 1560, C: int = 256,
                      n_cal: int = 1024, rank: int = 8, workload: int = 5):
    """Video law truncated to T cached tokens; low-rank + noise queries
    (n_cal calibration queries on stream 4, Lq evaluation queries on stream 3)."""
    seed = seed_for(workload)
    K = video(seed, S_K, H, D, T)
    V = video(seed, S_V, H, D, T)
    q_cal = to_bf16_bits(lowrank_queries(seed, S_QCAL, n_cal, H, D, rank))
    Q = to_bf16_bits(lowrank_queries(seed, S_Q, Lq, H, D, rank)).reshape(1, Lq, H, D)
    init = np.stack([kmeans_init(seed, T, C, 0, h, H) for h in range(H)])[None]
    return dict(seed=seed, B=1, Hkv=H, Hq=H, D=D, T=T, Lq=Lq, C=C, K=K, V=V, q=Q,
                q_cal=q_cal, kmeans_init=init)
