"""Pins of the oracle's FP8 (OCP E4M3) KV-cache functions, on the CPU.

None of these retypes the encoder: values come from the format's definition
(sign, 4-bit exponent with bias 7, 3-bit mantissa, subnormals m/8 * 2^-6,
0x7F/0xFF NaN, largest finite 448), from an exhaustive nearest-value search
over the 254 finite codes, and from closed forms of attention.
"""

import math

import numpy as np
import pytest

import oracle
from oracle.fp8 import E4M3_MAX


def code_value(c):
    """Value of one code by the definition, in plain Python."""
    s = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 0xF, c & 7
    if e == 0xF and m == 7:
        return math.nan
    if e == 0:
        return s * math.ldexp(m, -9)
    return s * math.ldexp(8 + m, e - 10)


def test_decode_named_codes():
    d = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        want = code_value(c)
        assert (math.isnan(want) and math.isnan(d[c])) or d[c] == want, c
    assert d[0x38] == 1.0 and d[0xB8] == -1.0
    assert d[0x01] == 2.0 ** -9 and d[0x08] == 2.0 ** -6 and d[0x07] == 7 * 2.0 ** -9
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0 == -E4M3_MAX
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.isfinite(d).sum() == 254


def nearest_code(y):
    """Exhaustive search: the finite code nearest to y, ties to the even
    mantissa (code bit 0 clear); y is first clamped to +-448."""
    y = max(-448.0, min(448.0, y))
    best = None
    for c in range(256):
        v = code_value(c)
        if math.isnan(v):
            continue
        if v == 0.0 and c == 0x80 and not math.copysign(1.0, y) < 0:
            continue  # +0 for non-negative inputs
        if v == 0.0 and c == 0x00 and math.copysign(1.0, y) < 0:
            continue  # -0 for negative inputs
        dist = abs(v - y)
        key = (dist, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_encode_matches_exhaustive_nearest_search():
    rng = np.random.default_rng(8)
    ys = np.concatenate([
        rng.normal(0, 1, 400), rng.normal(0, 100, 200), rng.uniform(-600, 600, 100),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 200),           # subnormal range
        np.array([d for d in oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
                  if np.isfinite(d)]),                     # every code value
    ])
    # midpoints between neighbouring positive codes: ties
    vals = sorted({abs(code_value(c)) for c in range(0x7F) if not math.isnan(code_value(c))})
    mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]
    ys = np.concatenate([ys, mids, -np.array(mids)])
    got = oracle.e4m3_encode(ys)
    for y, g in zip(ys, got):
        assert g == nearest_code(float(y)), (y, g, nearest_code(float(y)))


def test_encode_special_values():
    e = oracle.e4m3_encode
    assert list(e([1e9, -1e9, 448.0, 464.0, 500.0])) == [0x7E, 0xFE, 0x7E, 0x7E, 0x7E]
    # every NaN -- either sign bit, any payload -- is the one code 0x7F
    nans = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF], dtype=np.uint32)
    assert list(e(nans.view(np.float32).astype(np.float64))) == [0x7F] * 4
    assert list(e([np.inf, -np.inf])) == [0x7E, 0xFE]
    assert e([0.0])[0] == 0x00 and e([-0.0])[0] == 0x80
    # ties to even: 1.0625 -> 1.0 (mantissa 0), 1.1875 -> 1.25 (mantissa 2)
    assert list(e([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10])) == [0x38, 0x3A, 0x00, 0x02]


def test_quantize_uses_per_head_scales():
    # x = scale * code value exactly -> the code comes back
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7F, size=(5, 2, 8)).astype(np.uint8)
    codes[codes == 0x7F] = 0x7E
    scales = np.array([0.5, 4.0], dtype=np.float32)
    x = oracle.e4m3_decode(codes) * scales[None, :, None]
    x32 = x.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x)     # exact in float32
    assert np.array_equal(oracle.quantize(x32, "f32", scales), codes)
    # swapping the heads' scales changes the codes (a per-head mistake shows)
    assert not np.array_equal(oracle.quantize(x32, "f32", scales[::-1]), codes)


def test_kv_write_fp8_brute_force():
    rng = np.random.default_rng(11)
    nt, hkv, d, nb = 5, 2, 4, 3
    key = rng.normal(0, 3, (nt, hkv, d)).astype(np.float32)
    value = rng.normal(0, 3, (nt, hkv, d)).astype(np.float32)
    kc = rng.integers(0, 256, (nb, hkv, 16, d)).astype(np.uint8)
    vc = rng.integers(0, 256, (nb, hkv, d, 16)).astype(np.uint8)
    slots = np.array([17, 3, -1, 40, 16])
    ks = np.array([0.25, 2.0], dtype=np.float32)
    vs = np.array([1.0, 0.125], dtype=np.float32)
    kp, vp = oracle.kv_write_fp8(key, value, kc, vc, slots, ks, vs, "f32")
    ek, ev = kc.copy(), vc.copy()
    for t in range(nt):
        if slots[t] < 0:
            continue
        b, o = divmod(int(slots[t]), 16)
        for h in range(hkv):
            for j in range(d):
                ek[b, h, o, j] = nearest_code(float(np.float32(key[t, h, j]) / ks[h]))
                ev[b, h, j, o] = nearest_code(float(np.float32(value[t, h, j]) / vs[h]))
    assert np.array_equal(kp, ek) and np.array_equal(vp, ev)


def test_attention_fp8_closed_forms():
    # one key: the output is that key's dequantised V row; lse = scale * q.k
    rng = np.random.default_rng(5)
    hq, hkv, d, nb = 4, 2, 8, 2
    kc = rng.integers(0, 0x70, (nb, hkv, 16, d)).astype(np.uint8)
    vc = rng.integers(0, 0x70, (nb, hkv, d, 16)).astype(np.uint8)
    ks = np.array([0.5, 3.0], dtype=np.float32)
    vs = np.array([2.0, 0.25], dtype=np.float32)
    q = rng.normal(size=(1, hq, d)).astype(np.float32)
    out, lse = oracle.attention_fp8(q, kc, vc, ks, vs, [0, 1], [1], np.array([[1]]), 0.3, hkv,
                                    query_dtype="f32")
    for h in range(hq):
        g = h // (hq // hkv)
        vrow = [code_value(int(vc[1, g, j, 0])) * float(vs[g]) for j in range(d)]
        krow = [code_value(int(kc[1, g, 0, j])) * float(ks[g]) for j in range(d)]
        assert np.allclose(out[0, h], vrow, rtol=0, atol=1e-12)
        s = 0.3 * sum(float(q[0, h, j]) * krow[j] for j in range(d))
        assert abs(lse[0, h] - s) < 1e-9
