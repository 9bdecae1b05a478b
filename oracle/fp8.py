"""fp64 reference for an FP8 (E4M3) KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name an FP8 KV cache as a way to halve the cache's bytes ("Anatomy
of a serving engine", section on KV-cache capacity; "Model execution",
section "Attention backends") without fixing its format.  Reading taken: the
OCP 8-bit floating-point E4M3 format -- 1 sign bit, 4 exponent bits with bias
7, 3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; no
infinities; the all-ones exponent and mantissa (0x7F, 0xFF) are NaN, so the
largest finite magnitude is 1.75 * 2^8 = 448.  One float32 scale per KV head
for K and one for V: a cached value stands for code * scale.

Quantisation (the KV write): y = float32(x) / scale[h] in float32 (IEEE
division, as the kernel computes it, since the float decides the code), then
y is clamped to [-448, 448] and rounded to the nearest E4M3 value, ties to the
even mantissa.  Every NaN, whatever its sign bit, encodes as 0x7F (the pages
fix no NaN code; one canonical code keeps the write deterministic).
"""

from __future__ import annotations

import numpy as np

from .paged_attention import BLOCK_SIZE, attention, to_f64

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6      # 2^-6 = smallest normal
_MANT_BITS = 3


def e4m3_decode(codes) -> np.ndarray:
    """Value of every code (float64; NaN for 0x7F and 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** _MIN_NORMAL_EXP,
                   (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_encode(y) -> np.ndarray:
    """Code of each value: clamp to +-448, round to nearest, ties to even."""
    y = np.asarray(y, dtype=np.float64)
    nan = np.isnan(y)
    sign = np.signbit(y)
    a = np.minimum(np.abs(np.where(nan, 0.0, y)), E4M3_MAX)
    # quantum of the binade that holds a (subnormal range shares 2^-9)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, _MIN_NORMAL_EXP)
    q = np.exp2(e - _MANT_BITS)
    r = np.round(a / q) * q              # a / q is exact (power-of-two q); round = ties to even
    # r may have stepped into the next binade (e.g. 1.96875 -> 2.0): re-derive
    with np.errstate(divide="ignore"):
        e2 = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    normal = r >= 2.0 ** _MIN_NORMAL_EXP
    e2 = np.where(normal, e2, _MIN_NORMAL_EXP - 1)         # field 0 for subnormals / zero
    field = (e2 + 7).astype(np.int64)
    frac = np.where(normal, r / np.exp2(e2) - 1.0, r / 2.0 ** _MIN_NORMAL_EXP)
    mant = np.round(frac * 8.0).astype(np.int64)
    code = (np.where(sign, 0x80, 0) | (field << 3) | mant).astype(np.int64)
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)


def quantize(x, dtype: str, scale_h) -> np.ndarray:
    """Codes of x [..., Hkv, d] with one scale per KV head (axis -2)."""
    xf = to_f64(x, dtype).astype(np.float32)            # exact: bf16/f32 -> f32
    s = np.asarray(scale_h, dtype=np.float32)[:, None]
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        y = xf / s                                      # float32 IEEE division
    return e4m3_encode(y.astype(np.float64))


def kv_write_fp8(key, value, k_codes, v_codes, slot_mapping, k_scale, v_scale, dtype: str,
                 block_size: int = BLOCK_SIZE):
    """Quantising KV write: the codes of the step's new K/V at their slots."""
    kq = quantize(key, dtype, k_scale)                   # [Nt, Hkv, d]
    vq = quantize(value, dtype, v_scale)
    kp = np.array(k_codes, dtype=np.uint8, copy=True)
    vp = np.array(v_codes, dtype=np.uint8, copy=True)
    for t, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s < 0:
            continue
        blk, off = divmod(int(s), block_size)
        kp[blk, :, off, :] = kq[t]
        vp[blk, :, :, off] = vq[t]
    return kp, vp


def dequantize_pool(codes, scale_h, kv_head_axis: int = 1) -> np.ndarray:
    """code * scale of every pool entry, float64 (exact)."""
    vals = e4m3_decode(codes)
    shape = [1] * vals.ndim
    shape[kv_head_axis] = -1
    return vals * np.asarray(scale_h, dtype=np.float32).astype(np.float64).reshape(shape)


def attention_fp8(query, k_codes, v_codes, k_scale, v_scale, query_start_loc, seq_lens,
                  block_tables, scale, num_kv_heads, query_dtype: str = "bf16", rows=None):
    """Attention over the dequantised pools (the textbook form on code * scale)."""
    q = to_f64(query, query_dtype)
    kd = dequantize_pool(k_codes, k_scale)
    vd = dequantize_pool(v_codes, v_scale)
    return attention(q, kd, vd, query_start_loc, seq_lens, block_tables, scale, num_kv_heads,
                     "f64", rows=rows)
