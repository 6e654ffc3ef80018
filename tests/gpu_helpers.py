"""Shared plumbing for the GPU parity tests: host copies of the device
cache in the oracle's container, bit-exact comparison over the bytes the
cache contract specifies, and numpy <-> torch moves of bf16 bit patterns."""
import math

import numpy as np
import torch

import bit_kv_cache_int2_amd as kv
import oracle
import synth

TOL = 2e-3   # attention max |delta| vs the oracle's fp64 attention


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host(t: torch.Tensor, dtype) -> np.ndarray:
    return t.cpu().numpy().view(dtype)


def to_oracle(c: kv.KVCache) -> oracle.Cache:
    L = c.layout
    get = lambda name, dt: None if getattr(c, name) is None else np.ascontiguousarray(host(getattr(c, name), dt))
    int8 = c.k_psac8 is not None
    return oracle.Cache(L.batch, L.kv_heads, L.head_dim, L.capacity, L.key_mode, L.value_mode,
                        L.n_centroids, L.qsac_topk, L.psac_rank, L.qsac_score, L.psac_format,
                        k_codes=get("k_codes", np.uint8), k_params=get("k_params", np.uint32),
                        k_tail=get("k_tail", np.uint16), k_idx=get("k_idx", np.uint8),
                        centroids=get("centroids", np.float32), sens_w=get("sens_w", np.float32),
                        psac_basis=get("psac_basis", np.float32),
                        k_psac=None if int8 else get("k_psac", np.uint16),
                        k_psac8=get("k_psac8", np.int8) if int8 else None,
                        k_psac_sc=get("k_psac_sc", np.uint16) if int8 else None,
                        v_codes=get("v_codes", np.uint8), v_params=get("v_params", np.uint32),
                        M=L.n_modalities if L.value_mode == kv.VAL_HADAMARD_MODAL else 1,
                        v_signs=get("v_signs", np.uint32), v_modal=get("v_modality", np.uint8))


def oracle_like(c: kv.KVCache) -> oracle.Cache:
    """An empty oracle cache with the same layout and calibration inputs."""
    L = c.layout
    o = oracle.Cache(L.batch, L.kv_heads, L.head_dim, L.capacity, L.key_mode, L.value_mode,
                     L.n_centroids, L.qsac_topk, L.psac_rank, L.qsac_score, L.psac_format,
                     M=L.n_modalities if L.value_mode == kv.VAL_HADAMARD_MODAL else 1)
    if c.centroids is not None:
        o.centroids[:] = host(c.centroids, np.float32)
    if c.sens_w is not None:
        o.sens_w[:] = host(c.sens_w, np.float32)
    if c.psac_basis is not None:
        o.psac_basis[:] = host(c.psac_basis, np.float32)
    if c.v_signs is not None:
        o.v_signs[:] = host(c.v_signs, np.uint32)
        o.v_modal[:] = host(c.v_modality, np.uint8)
    return o


def assert_cache_equal(g: oracle.Cache, o: oracle.Cache, n: int, tag: str = "") -> None:
    """Bit-exact comparison of everything the cache contract defines after n
    tokens: rows [0, n) of value codes/params; for window keys, the rows and
    parameters of the finished windows and tail slots [0, n % 64); for
    centroid keys, rows [0, n) of indices, codes, params and PSAC words."""
    def eq(a, b, name):
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            raise AssertionError(f"{tag} {name}: {len(bad)} mismatches, first at {bad[:4].tolist()}")
    full_t, rem = n // 64, n % 64
    eq(g.v_codes[:, :, :full_t], o.v_codes[:, :, :full_t], "v_codes")
    if rem:     # partially filled value tile: only tokens < n % 64 are defined
        bits = np.zeros(128, np.uint8)
        bits[:2 * rem] = 1
        mask = np.packbits(bits.reshape(16, 8)[:, ::-1], axis=1).reshape(16)
        eq(g.v_codes[:, :, full_t] & mask, o.v_codes[:, :, full_t] & mask, "v_codes tail tile")
    eq(g.v_params[:, :, :n], o.v_params[:, :, :n], "v_params")
    if g.key_mode == oracle.KEY_WINDOW:
        full = (n // 64) * 64
        eq(g.k_codes[:, :, :full], o.k_codes[:, :, :full], "k_codes")
        eq(g.k_params[:, :, :n // 64], o.k_params[:, :, :n // 64], "k_params")
        eq(g.k_tail[:, :, :n % 64], o.k_tail[:, :, :n % 64], "k_tail")
    else:
        eq(g.k_idx[:, :, :n], o.k_idx[:, :, :n], "k_idx")
        eq(g.k_codes[:, :, :n], o.k_codes[:, :, :n], "k_codes")
        eq(g.k_params[:, :, :n], o.k_params[:, :, :n], "k_params")
        if g.R > 0 and g.psac_fmt == oracle.PSAC_INT8:
            eq(g.k_psac8[:, :, :n], o.k_psac8[:, :, :n], "k_psac8")
            eq(g.k_psac_sc[:, :, :n], o.k_psac_sc[:, :, :n], "k_psac_sc")
        elif g.R > 0:
            eq(g.k_psac[:, :, :n], o.k_psac[:, :, :n], "k_psac")


def calibrate(c: kv.KVCache, K_bits: np.ndarray, init: np.ndarray, iters: int,
              q_cal_bits: np.ndarray = None) -> None:
    """Fill the cache's calibration inputs with the oracle's calibration
    (k-means centroids, query weights, principal directions) -- the inputs
    both sides then share."""
    L = c.layout
    K = synth.bf16_bits_to_f32(K_bits)           # [B][T][H][D]
    cent = np.zeros((L.batch, L.kv_heads, L.n_centroids, L.head_dim), np.float32)
    for b in range(L.batch):
        for h in range(L.kv_heads):
            if iters == 0:      # the initial picks themselves
                cent[b, h] = K[b, init[b, h], h]
            else:
                cent[b, h] = oracle.kmeans(np.ascontiguousarray(K[b, :, h]), L.n_centroids,
                                           init[b, h], iters)[0]
    c.centroids.copy_(torch.from_numpy(cent))
    if q_cal_bits is not None:
        qc = synth.bf16_bits_to_f32(q_cal_bits).astype(np.float64)   # [N][H][D]
        w = np.zeros((L.batch, L.kv_heads, L.head_dim), np.float32)
        U = np.zeros((L.batch, L.kv_heads, L.head_dim, max(L.psac_rank, 1)), np.float32)
        for h in range(L.kv_heads):
            w[:, h] = oracle.sens_weights(np.ascontiguousarray(qc[:, h]))
            if L.psac_rank > 0:
                U[:, h] = oracle.pca(np.ascontiguousarray(qc[:, h]), L.psac_rank)[0]
        if c.sens_w is not None:
            c.sens_w.copy_(torch.from_numpy(w))
        if c.psac_basis is not None:
            c.psac_basis.copy_(torch.from_numpy(U))


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
