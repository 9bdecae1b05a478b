"""Pins of the oracle's rotary embedding + KV write, on the CPU.

Checked against what rotation fixes without retyping the oracle: position 0
is the identity, every (i, i + d/2) pair keeps its norm, scores depend only
on the distance between positions, a single pair at unit frequency traces
(cos p, sin p), the pairing is half-split (a planted interleaved pairing
fails), the bf16 rounding agrees with torch's conversion, and a plain-Python
write reproduces the pools.
"""

import math

import numpy as np
import torch

import oracle
from workloads import rope_table


def test_position_zero_is_identity():
    tab = rope_table(4, 8)
    x = np.random.default_rng(0).normal(size=(3, 2, 8)).astype(np.float32)
    assert np.array_equal(oracle.rope(x, [0, 0, 0], tab, "f32"), x.astype(np.float64))


def test_pair_norms_are_kept():
    rng = np.random.default_rng(1)
    tab = rope_table(5000, 64)
    x = rng.normal(size=(20, 3, 64)).astype(np.float32)
    pos = rng.integers(0, 5000, 20)
    y = oracle.rope(x, pos, tab, "f32")
    n0 = x[..., :32].astype(np.float64) ** 2 + x[..., 32:].astype(np.float64) ** 2
    n1 = y[..., :32] ** 2 + y[..., 32:] ** 2
    assert np.allclose(n0, n1, rtol=1e-6, atol=0)


def test_scores_depend_on_distance_only():
    rng = np.random.default_rng(2)
    tab = rope_table(3000, 32)
    q = rng.normal(size=(1, 1, 32)).astype(np.float32)
    k = rng.normal(size=(1, 1, 32)).astype(np.float32)
    s = [float(np.sum(oracle.rope(q, [m + t], tab, "f32") * oracle.rope(k, [n + t], tab, "f32")))
         for m, n, t in ((50, 20, 0), (50, 20, 1000), (50, 20, 2500))]
    assert abs(s[0] - s[1]) < 1e-4 and abs(s[0] - s[2]) < 1e-4


def test_unit_frequency_pair_traces_the_circle():
    tab = rope_table(100, 2)          # one pair, angle p * 1
    x = np.array([[[1.0, 0.0]]], dtype=np.float32)
    for p in (1, 7, 99):
        y = oracle.rope(x, [p], tab, "f32")[0, 0]
        assert abs(y[0] - math.cos(p)) < 1e-7 and abs(y[1] - math.sin(p)) < 1e-7


def test_pairing_is_half_split():
    tab = rope_table(10, 4)
    e1 = np.array([[[0.0, 1.0, 0.0, 0.0]]], dtype=np.float32)
    y = oracle.rope(e1, [3], tab, "f32")[0, 0]
    # dim 1 pairs with dim 3 (half split), never with dim 0 (interleaved)
    assert y[0] == 0.0 and y[2] == 0.0 and y[3] != 0.0


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = rng.normal(size=4096) * np.exp2(rng.integers(-20, 20, 4096))
    # exact ties of bf16 (a float32 with only bit 15 set below the bf16 mantissa)
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32).astype(np.float64)
    x = np.concatenate([x, ties, -ties])
    want = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(oracle.round_to(x, "bf16"), want.view(np.uint16))


def test_rope_kv_write_brute_force():
    rng = np.random.default_rng(4)
    nt, hq, hkv, d, nb = 6, 4, 2, 8, 3
    tab = rope_table(40, d)
    bits = lambda a: torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q = bits(rng.normal(size=(nt, hq, d)).astype(np.float32))
    k = bits(rng.normal(size=(nt, hkv, d)).astype(np.float32))
    v = bits(rng.normal(size=(nt, hkv, d)).astype(np.float32))
    kp = rng.integers(0, 1 << 16, (nb, hkv, 16, d)).astype(np.uint16)
    vp = rng.integers(0, 1 << 16, (nb, hkv, d, 16)).astype(np.uint16)
    slots = np.array([3, 17, -1, 40, 9, 33])
    pos = np.array([0, 5, 6, 39, 40, 12])            # 40 is past the table
    qr, kq, vq = oracle.rope_kv_write(q, k, v, kp, vp, slots, pos, tab, "bf16")
    widen = lambda u: float((np.uint32(u) << np.uint32(16)).view(np.float32))
    ek, ev = kp.copy(), vp.copy()
    for t in range(nt):
        p = int(pos[t])
        ok = 0 <= p < 40
        for h in range(hkv):
            for i in range(d):
                j = (i + d // 2) % d
                c, s = float(tab[p % 40, i % (d // 2)]), float(tab[p % 40, d // 2 + i % (d // 2)])
                a, b = widen(k[t, h, i]), widen(k[t, h, j])
                val = a * c - b * s if i < d // 2 else a * c + b * s
                if ok and slots[t] >= 0:
                    blk, off = divmod(int(slots[t]), 16)
                    ek[blk, h, off, i] = torch.tensor([val], dtype=torch.float64).to(
                        torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)[0]
                    ev[blk, h, i, off] = v[t, h, i]
        if not ok:
            assert np.array_equal(qr[t], oracle.to_f64(q[t], "bf16"))
    assert np.array_equal(kq, ek) and np.array_equal(vq, ev)


def test_rope_table_frequencies():
    # the input table's angles p * 10000^(-2i/d): at d = 128 pair 16 turns by
    # 10000^(-1/4) = 1/10 per position and pair 32 by 10000^(-1/2) = 1/100,
    # pair 0 by 1; the last pair by 10000^(-63/64)
    tab = rope_table(2000, 128).astype(np.float64)
    p = np.arange(2000)
    for i, w in ((0, 1.0), (16, 0.1), (32, 0.01), (63, 10000.0 ** (-63 / 64))):
        assert np.abs(tab[:, i] - np.cos(w * p)).max() < 1e-6, i
        assert np.abs(tab[:, 64 + i] - np.sin(w * p)).max() < 1e-6, i
