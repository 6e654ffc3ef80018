"""Pins for the oracle's number formats, INT2 group quantizer, packing and
Walsh-Hadamard rotation.  Every check here compares the oracle with
something other than itself: numpy's IEEE conversions, hand-derived
fixtures, brute force over the four levels, scipy's Sylvester Hadamard
matrix, or an algebraic identity."""
import math
import os

import numpy as np
import pytest
import scipy.linalg
from hypothesis import given, settings, strategies as st

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- formats
def test_f16_conversion_matches_numpy_ieee():
    rng = np.random.default_rng(1)
    xs = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 5, 4000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0, -2.5e-8]),
    ]).astype(np.float32)
    for x in xs:
        want = int(np.float32(x).astype(np.float16).view(np.uint16))
        assert oracle.f64_to_f16(float(x)) == want, x


def test_f16_widening_matches_numpy():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits[::7]])
    r = ref[::7]
    same = (got == r) | (np.isnan(got) & np.isnan(r))
    assert same.all()


# ----------------------------------------------------------------- quantizer
def _expand(tok):
    out = []
    for t in tok.split():
        if "*" in t and not t.startswith("*"):
            v, k = t.rsplit("*", 1)
            out += [v] * int(k)
        else:
            out.append(t)
    return out


def _golden_q2():
    rows = []
    with open(os.path.join(GOLDEN, "q2_groups.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, vals, s, z, codes = [p.strip() for p in line.split("|")]
            x = np.array([np.float32(float(v)) for v in _expand(vals)], np.float32)
            c = np.array([int(v) for v in _expand(codes)], np.uint8)
            rows.append((name, x, int(s, 16), int(z, 16), c))
    return rows


@pytest.mark.parametrize("case", _golden_q2(), ids=lambda c: c[0])
def test_q2_hand_derived_cases(case):
    name, x, s_bits, z_bits, codes = case
    assert x.size == 32 and codes.size == 32
    c, s, z = oracle.q2(x)
    assert (s, z) == (s_bits, z_bits)
    assert (c == codes).all()


def _levels(s_bits, z_bits):
    s = oracle.f16_to_f64(s_bits)
    z = oracle.f16_to_f64(z_bits)
    return s, z


def _check_group(x):
    c, sb, zb = oracle.q2(x)
    s, z = _levels(sb, zb)
    xs = x.astype(np.float64)
    mn, mx = xs.min(), xs.max()
    assert c.max() <= 3
    # scale and zero are the fp16 roundings of (max-min)/3 and min
    assert zb == int(np.float16(np.float32(mn + 0.0)).view(np.uint16))
    s32 = np.float32(np.float32(mx) - np.float32(mn)) / np.float32(3.0)
    assert sb == int(np.float16(s32).view(np.uint16))
    if s == 0.0:
        assert (c == 0).all()
        return
    # brute force: each code is the nearest stored level; where x sits within
    # an fp32 rounding of a midpoint either neighbour is accepted
    lv = np.arange(4) * s + z
    for xi, ci in zip(xs, c):
        d = np.abs(xi - lv)
        best = int(np.argmin(d))
        if best != ci:
            mid = (min(best, int(ci)) + 0.5) * s + z
            assert abs(xi - mid) <= 2 * np.spacing(np.float32(abs(mid) + abs(z) + s)), (xi, ci, best)
            assert abs(best - int(ci)) == 1
    # min element gets code 0 (its dequantisation is z) unless the first
    # threshold z + s/2 rounds onto it in fp32, which needs a step below the
    # fp32 resolution at z (impossible for distinct bf16 inputs)
    t0 = float(np.float32(0.5 * s + z))
    if t0 > mn:
        assert c[np.argmin(xs)] == 0
    # max element gets the top code unless s rounded up past it
    if 3 * s + z <= mx:
        assert c[np.argmax(xs)] == 3
    # per-element error bound: half a step plus the fp16 rounding of s and z
    xhat = c.astype(np.float64) * s + z
    bound = s / 2 + abs(z - mn) + 3 * abs(s - float(s32)) + 4 * np.spacing(np.float32(np.abs(xs).max()))
    assert np.all(np.abs(xs - xhat) <= bound)


@settings(max_examples=300, deadline=None)
@given(st.lists(st.floats(-300, 300, width=32, allow_subnormal=True), min_size=32, max_size=32))
def test_q2_properties_random_groups(vals):
    _check_group(np.array(vals, np.float32))


def test_q2_properties_adversarial():
    rng = np.random.default_rng(7)
    cases = [np.zeros(32), np.full(32, -2.5), np.r_[np.zeros(31), 1e-30],
             np.r_[np.full(16, 1.0), np.full(16, 1.0 + 2 ** -23)],
             rng.standard_normal(32) * 1e-6, rng.standard_normal(32) * 60.0,
             np.linspace(-1, 2, 32), np.r_[np.full(31, 0.0), 3.0 * 2 ** -24]]
    for x in cases:
        _check_group(np.asarray(x, np.float32))
    # bf16 inputs (the cache's input type): min is fp16-exact, so the
    # dequantised minimum equals the input minimum bit for bit
    for _ in range(200):
        x = (rng.standard_normal(32) * rng.uniform(0.01, 20)).astype(np.float32)
        x = ((x.view(np.uint32) + 0x8000) & 0xFFFF0000).view(np.float32)
        c, sb, zb = oracle.q2(x)
        s, z = _levels(sb, zb)
        assert z == float(x.min())
        assert c[np.argmin(x)] == 0


def test_q2_exact_at_max_when_step_is_representable():
    # max - min = 3 * s with s an fp16 value: the top level hits the max exactly
    rng = np.random.default_rng(3)
    for _ in range(100):
        s = float(np.float16(rng.uniform(0.01, 4)))
        mn = float(np.float16(rng.uniform(-8, 8)))
        x = np.float32(mn) + np.float32(3 * s) * rng.random(32).astype(np.float32)
        x[0], x[1] = mn, mn + 3 * s
        x = x.astype(np.float32)
        if float(x[1]) != mn + 3 * s:
            continue
        c, sb, zb = oracle.q2(x)
        sd, zd = _levels(sb, zb)
        assert c[1] == 3 and 3 * sd + zd == float(x[1])


# ----------------------------------------------------------------- packing
def test_pack_order_and_roundtrip():
    assert list(oracle.pack_row(np.array([0, 1, 2, 3], np.uint8))) == [0xE4]
    assert list(oracle.pack_row(np.array([3, 0, 0, 0, 0, 0, 0, 3], np.uint8))) == [0x03, 0xC0]
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 4, 128).astype(np.uint8)
    row = oracle.pack_row(codes)
    back = np.array([(row[c // 4] >> (2 * (c % 4))) & 3 for c in range(128)], np.uint8)
    assert (back == codes).all()


# ----------------------------------------------------------------- WHT
@pytest.mark.parametrize("D", [64, 128])
def test_wht_is_sylvester_hadamard(D):
    H = scipy.linalg.hadamard(D).astype(np.float64)
    assert (H @ H.T == D * np.eye(D)).all()
    rng = np.random.default_rng(D)
    for _ in range(5):
        x = rng.standard_normal(D)
        ref = H @ x / math.sqrt(D)
        assert np.allclose(oracle.wht_f64(x), ref, rtol=0, atol=1e-12)
        xf = x.astype(np.float32)
        got = oracle.wht_f32(xf).astype(np.float64)
        ref32 = H @ xf.astype(np.float64) / math.sqrt(D)
        assert np.max(np.abs(got - ref32)) <= 1e-6 * np.abs(ref32).max() * math.log2(D)
    # involution and Parseval
    x = rng.standard_normal(D)
    y = oracle.wht_f64(x)
    assert np.allclose(oracle.wht_f64(y), x, atol=1e-12)
    assert abs(np.dot(y, y) - np.dot(x, x)) < 1e-10 * np.dot(x, x)


def test_wht_unit_vector_and_constant():
    e0 = np.zeros(128, np.float32)
    e0[0] = 1.0
    y = oracle.wht_f32(e0)
    assert (y.view(np.uint32) == 0x3DB504F3).all()       # f32(1/sqrt(128))
    ones = np.ones(64, np.float32)
    y = oracle.wht_f32(ones)                              # all energy in bin 0
    assert y[0] == np.float32(8.0) and (y[1:] == 0).all()
