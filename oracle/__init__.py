"""CPU oracle for the INT2 KV-cache path -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and
the two share no code.  The arithmetic lives in ``oracle.c`` (plain C,
fp32 for discrete decisions, fp64 for continuous results); this module only
marshals numpy arrays.

Pages followed (cited by title and section):
  "QuantWM: Training-Free 2-bit KV Cache Quantization for Stable Video
   World Models", "QuantWM Framework" 1 (QSAC) and 2 (PSAC);
  "OmniKVQuant: KV Cache Quantization for Omni-LLMs", English abstract;
  "WUSH-KV Applies Data-Adaptive Transforms to KV Cache Quantization".
Parity pins for every function are in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

GROUP = 32
WINDOW = 64
KEY_WINDOW, KEY_CENTROID, KEY_CENTROID_QSAC = 0, 1, 2
VAL_GROUP, VAL_HADAMARD, VAL_HADAMARD_MODAL = 0, 1, 2


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.orc_bf16_to_f32.restype = ctypes.c_float
    L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
    L.orc_f16_to_f64.restype = dbl
    L.orc_f64_to_f16.argtypes = [dbl]
    L.orc_f64_to_f16.restype = ctypes.c_uint16
    L.orc_q2.argtypes = [vp, i32, i32, vp, vp, vp]
    L.orc_q2.restype = None
    L.orc_pack_row.argtypes = [vp, i32, vp]
    L.orc_pack_row.restype = None
    L.orc_wht_f32.argtypes = [vp, i32]
    L.orc_wht_f32.restype = None
    L.orc_wht_f64.argtypes = [vp, i32]
    L.orc_wht_f64.restype = None
    L.orc_rotate_modal_f32.argtypes = [vp, i32, vp]
    L.orc_rotate_modal_f32.restype = None
    L.orc_assign_plain.argtypes = [vp, vp, i32, i32]
    L.orc_assign_plain.restype = i32
    L.orc_assign_qsac.argtypes = [vp, vp, i32, i32, vp, i32, i32]
    L.orc_assign_qsac.restype = i32
    L.orc_quantize_append.argtypes = [i32] * 12 + [vp] * 14 + [vp, vp, i32, i32]
    L.orc_quantize_append.restype = i32
    L.orc_dequant_keys.argtypes = [i32] * 6 + [vp] * 5 + [i32, i32, i32, vp]
    L.orc_dequant_keys.restype = None
    L.orc_dequant_values.argtypes = [i32, i32, i32, vp, vp, i32, i32, i32, vp]
    L.orc_dequant_values.restype = None
    L.orc_attention.argtypes = ([i32] * 10 + [vp] * 13 + [i32, vp, i32, i32, dbl, vp, vp])
    L.orc_attention.restype = i32
    L.orc_top1.argtypes = [i32] * 8 + [vp] * 9 + [i32, vp, i32, i32, vp, vp]
    L.orc_top1.restype = i32
    L.orc_merge.argtypes = [i32, i32, vp, vp, vp, vp, vp]
    L.orc_merge.restype = None
    L.orc_kmeans.argtypes = [vp, i32, i32, i32, vp, i32, vp, vp]
    L.orc_kmeans.restype = None
    L.orc_sens_weights.argtypes = [vp, i32, i32, vp]
    L.orc_sens_weights.restype = None
    L.orc_pca.argtypes = [vp, i32, i32, i32, vp, vp]
    L.orc_pca.restype = i32
    L.orc_num_threads.argtypes = []
    L.orc_num_threads.restype = i32
    _lib = L
    return L


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "need C-contiguous numpy"
    return ctypes.c_void_p(a.ctypes.data)


def num_threads() -> int:
    return int(lib().orc_num_threads())


# ---------------------------------------------------------------- scalars
def f16_to_f64(bits: int) -> float:
    return lib().orc_f16_to_f64(int(bits))


def f64_to_f16(x: float) -> int:
    return int(lib().orc_f64_to_f16(float(x)))


def bf16_to_f32(bits: int) -> float:
    return float(lib().orc_bf16_to_f32(int(bits)))


def f16_array_to_f64(bits: np.ndarray) -> np.ndarray:
    f = np.vectorize(lambda b: lib().orc_f16_to_f64(int(b)), otypes=[np.float64])
    return f(bits) if bits.size else bits.astype(np.float64)


# ---------------------------------------------------------------- pieces
def q2(x: np.ndarray):
    """INT2 group quantizer of a 1-D fp32 group -> (codes u8, s_bits, z_bits)."""
    x = np.ascontiguousarray(x, np.float32)
    codes = np.empty(x.size, np.uint8)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    lib().orc_q2(_p(x), x.size, 1, _p(codes), _p(s), _p(z))
    return codes, int(s[0]), int(z[0])


def pack_row(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    out = np.empty(codes.size // 4, np.uint8)
    lib().orc_pack_row(_p(codes), codes.size, _p(out))
    return out


def wht_f32(x: np.ndarray) -> np.ndarray:
    y = np.array(x, np.float32, copy=True, order="C")
    lib().orc_wht_f32(_p(y), y.size)
    return y


def wht_f64(x: np.ndarray) -> np.ndarray:
    y = np.array(x, np.float64, copy=True, order="C")
    lib().orc_wht_f64(_p(y), y.size)
    return y


def rotate_modal_f32(x: np.ndarray, signs_row: np.ndarray) -> np.ndarray:
    """One modality's value rotation of an f32 row: the WHT, then the
    channels whose sign bit is set negated (signs_row u32 [D/32])."""
    y = np.array(x, np.float32, copy=True, order="C")
    sr = np.ascontiguousarray(signs_row, np.uint32)
    assert sr.size == y.size // 32
    lib().orc_rotate_modal_f32(_p(y), y.size, _p(sr))
    return y


def assign_plain(k: np.ndarray, cent: np.ndarray) -> int:
    k = np.ascontiguousarray(k, np.float32)
    cent = np.ascontiguousarray(cent, np.float32)
    return int(lib().orc_assign_plain(_p(k), _p(cent), cent.shape[0], k.size))


QSAC_EXACT, QSAC_RANGE = 0, 1     # QSAC perturbation estimate
PSAC_F16, PSAC_INT8 = 0, 1        # PSAC coefficient format


def assign_qsac(k: np.ndarray, cent: np.ndarray, w: np.ndarray, topk: int,
                score: int = QSAC_EXACT) -> int:
    k = np.ascontiguousarray(k, np.float32)
    cent = np.ascontiguousarray(cent, np.float32)
    w = np.ascontiguousarray(w, np.float32)
    return int(lib().orc_assign_qsac(_p(k), _p(cent), cent.shape[0], k.size, _p(w), int(topk),
                                     int(score)))


def merge(m: np.ndarray, l: np.ndarray, o: np.ndarray):
    m = np.ascontiguousarray(m, np.float64)
    l = np.ascontiguousarray(l, np.float64)
    o = np.ascontiguousarray(o, np.float64)
    S, D = o.shape
    out = np.empty(D, np.float64)
    lse = np.empty(1, np.float64)
    lib().orc_merge(S, D, _p(m), _p(l), _p(o), _p(out), _p(lse))
    return out, float(lse[0])


def kmeans(x: np.ndarray, C: int, init: np.ndarray, iters: int):
    """x f32 [n][D] -> (centroids f32 [C][D], assignment i32 [n])."""
    x = np.ascontiguousarray(x, np.float32)
    n, D = x.shape
    init = np.ascontiguousarray(init, np.int64)
    cent = np.empty((C, D), np.float32)
    asg = np.empty(n, np.int32)
    lib().orc_kmeans(_p(x), n, D, C, _p(init), int(iters), _p(cent), _p(asg))
    return cent, asg


def sens_weights(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, np.float64)
    N, D = q.shape
    w = np.empty(D, np.float32)
    lib().orc_sens_weights(_p(q), N, D, _p(w))
    return w


def pca(q: np.ndarray, R: int):
    """-> (U f32 [D][R], eigenvalues f64 [D] descending, sweeps)."""
    q = np.ascontiguousarray(q, np.float64)
    N, D = q.shape
    U = np.empty((D, R), np.float32)
    ev = np.empty(D, np.float64)
    sweeps = lib().orc_pca(_p(q), N, D, R, _p(U), _p(ev))
    return U, ev, sweeps


# ---------------------------------------------------------------- cache
@dataclass
class Cache:
    """Host copy of the packed cache, in the library's layout."""
    B: int
    H: int
    D: int
    Tcap: int
    key_mode: int = KEY_WINDOW
    value_mode: int = VAL_GROUP
    C: int = 0
    topk: int = 1
    R: int = 0
    qsac_score: int = 0        # QSAC_EXACT / QSAC_RANGE
    psac_fmt: int = 0          # PSAC_F16 / PSAC_INT8
    M: int = 1                 # modalities (VAL_HADAMARD_MODAL)
    k_codes: np.ndarray = field(default=None, repr=False)
    k_params: np.ndarray = field(default=None, repr=False)
    k_tail: np.ndarray = field(default=None, repr=False)
    k_idx: np.ndarray = field(default=None, repr=False)
    centroids: np.ndarray = field(default=None, repr=False)
    sens_w: np.ndarray = field(default=None, repr=False)
    psac_basis: np.ndarray = field(default=None, repr=False)
    k_psac: np.ndarray = field(default=None, repr=False)
    k_psac8: np.ndarray = field(default=None, repr=False)
    k_psac_sc: np.ndarray = field(default=None, repr=False)
    v_codes: np.ndarray = field(default=None, repr=False)
    v_params: np.ndarray = field(default=None, repr=False)
    v_signs: np.ndarray = field(default=None, repr=False)     # u32 [H][M][D/32] sign bits
    v_modal: np.ndarray = field(default=None, repr=False)     # u8 [B][Tcap] modality per token

    def __post_init__(self):
        B, H, D, T = self.B, self.H, self.D, self.Tcap
        assert T % WINDOW == 0 and D % GROUP == 0
        z = np.zeros
        if self.k_codes is None:
            self.k_codes = z((B, H, T, D // 4), np.uint8)
        if self.v_codes is None:      # per 64-token tile, channel-major
            self.v_codes = z((B, H, T // WINDOW, D, 16), np.uint8)
        if self.v_params is None:
            self.v_params = z((B, H, T, D // GROUP), np.uint32)
        if self.k_params is None:
            self.k_params = (z((B, H, T // WINDOW, D), np.uint32) if self.key_mode == KEY_WINDOW
                             else z((B, H, T, D // GROUP), np.uint32))
        if self.k_tail is None:
            self.k_tail = z((B, H, WINDOW, D), np.uint16)
        if self.k_idx is None:
            self.k_idx = z((B, H, T), np.uint8)
        if self.centroids is None:
            self.centroids = z((B, H, max(self.C, 1), D), np.float32)
        if self.sens_w is None:
            self.sens_w = np.ones((B, H, D), np.float32)
        if self.psac_basis is None:
            self.psac_basis = z((B, H, D, max(self.R, 1)), np.float32)
        if self.k_psac is None:
            self.k_psac = z((B, H, T, max(self.R, 1)), np.uint16)
        if self.k_psac8 is None:
            self.k_psac8 = z((B, H, T, max(self.R, 1)), np.int8)
        if self.k_psac_sc is None:
            self.k_psac_sc = z((B, H, T), np.uint16)
        if self.v_signs is None:
            self.v_signs = z((H, max(self.M, 1), D // 32), np.uint32)
        if self.v_modal is None:
            self.v_modal = z((B, T), np.uint8)

    def bufs(self):
        return [self.k_codes, self.k_params, self.k_tail, self.k_idx, self.centroids,
                self.sens_w, self.psac_basis, self.k_psac, self.k_psac8, self.k_psac_sc,
                self.v_codes, self.v_params]

    def append(self, k_bf16: np.ndarray, v_bf16: np.ndarray, cur_len: int) -> None:
        """Quantise tokens [cur_len, cur_len + n_new) of every sequence; inputs
        bf16 bits [B][n_new][H][D]."""
        k = np.ascontiguousarray(k_bf16, np.uint16)
        v = np.ascontiguousarray(v_bf16, np.uint16)
        B, n_new, H, D = k.shape
        assert (B, H, D) == (self.B, self.H, self.D) and v.shape == k.shape
        rc = lib().orc_quantize_append(
            self.B, self.H, self.D, self.Tcap, self.key_mode, self.value_mode,
            self.C, self.topk, self.R, self.qsac_score, self.psac_fmt, self.M,
            _p(self.v_signs), _p(self.v_modal), *[_p(b) for b in self.bufs()],
            _p(k), _p(v), int(cur_len), int(n_new))
        if rc != 0:
            raise ValueError(f"orc_quantize_append failed: {rc}")

    def keys(self, b: int, h: int, n: int) -> np.ndarray:
        out = np.empty((n, self.D), np.float64)
        lib().orc_dequant_keys(self.B, self.H, self.D, self.Tcap, self.key_mode, max(self.C, 1),
                               _p(self.k_codes), _p(self.k_params), _p(self.k_tail),
                               _p(self.k_idx), _p(self.centroids), b, h, n, _p(out))
        return out

    def values(self, b: int, h: int, n: int) -> np.ndarray:
        out = np.empty((n, self.D), np.float64)
        lib().orc_dequant_values(self.H, self.D, self.Tcap, _p(self.v_codes),
                                 _p(self.v_params), b, h, n, _p(out))
        return out

    def attention(self, q: np.ndarray, n: int, scale: float):
        """q f64 [B][Lq][Hq][D] -> (out f64 [B][Lq][Hq][D], lse f64 [B][Hq][Lq])."""
        q = np.ascontiguousarray(q, np.float64)
        B, Lq, Hq, D = q.shape
        out = np.empty_like(q)
        lse = np.empty((B, Hq, Lq), np.float64)
        rc = lib().orc_attention(
            self.B, self.H, self.D, self.Tcap, self.key_mode, self.value_mode,
            max(self.C, 1), self.R, self.psac_fmt, self.M, _p(self.v_signs), _p(self.v_modal),
            _p(self.k_codes), _p(self.k_params),
            _p(self.k_tail), _p(self.k_idx), _p(self.centroids), _p(self.psac_basis),
            _p(self.k_psac), _p(self.k_psac8), _p(self.k_psac_sc), _p(self.v_codes),
            _p(self.v_params), int(n), _p(q), Lq, Hq, float(scale), _p(out), _p(lse))
        if rc != 0:
            raise ValueError(f"orc_attention failed: {rc}")
        return out, lse

    def top1(self, q: np.ndarray, n: int):
        """q f64 [B][Lq][Hq][D] -> (idx i32 [B][Hq][Lq], logit f64 [B][Hq][Lq]): each
        row's largest-logit cached token (first on ties), logits before the scale."""
        q = np.ascontiguousarray(q, np.float64)
        B, Lq, Hq, D = q.shape
        idx = np.empty((B, Hq, Lq), np.int32)
        lg = np.empty((B, Hq, Lq), np.float64)
        rc = lib().orc_top1(
            self.B, self.H, self.D, self.Tcap, self.key_mode, max(self.C, 1), self.R, self.psac_fmt,
            _p(self.k_codes), _p(self.k_params), _p(self.k_tail), _p(self.k_idx),
            _p(self.centroids), _p(self.psac_basis), _p(self.k_psac), _p(self.k_psac8),
            _p(self.k_psac_sc), int(n), _p(q), Lq, Hq, _p(idx), _p(lg))
        if rc != 0:
            raise ValueError(f"orc_top1 failed: {rc}")
        return idx, lg

    def slice_bh(self, b: int, h: int) -> "Cache":
        """A one-sequence, one-head copy (for sampled checks at full size)."""
        sl = lambda a: np.ascontiguousarray(a[b:b + 1, h:h + 1])
        return Cache(1, 1, self.D, self.Tcap, self.key_mode, self.value_mode, self.C,
                     self.topk, self.R, self.qsac_score, self.psac_fmt, self.M,
                     *[sl(a) for a in self.bufs()],
                     v_signs=np.ascontiguousarray(self.v_signs[h:h + 1]),
                     v_modal=np.ascontiguousarray(self.v_modal[b:b + 1]))
