"""Random small batches (hypothesis, derandomized): the oracle against the
pure-Python brute force of the definition, and its own invariants (block
placement, split into key ranges), on shapes drawn over the edge cases --
requests with no new tokens, contexts ending on block boundaries, group sizes
1-3, both dtypes, zero and large scales."""

import numpy as np
from hypothesis import HealthCheck, assume, given, settings
from hypothesis import strategies as hst

import oracle
from test_oracle_pins import brute_force, run_oracle, tiny_step

SETTINGS = dict(max_examples=40, deadline=None, derandomize=True,
                suppress_health_check=[HealthCheck.too_slow])


@hst.composite
def small_batch(draw):
    B = draw(hst.integers(1, 3))
    shapes = []
    for _ in range(B):
        n = draw(hst.integers(0, 6))
        prior = draw(hst.sampled_from([0, 1, 15, 16, 17, 31, 32, 40]))
        if prior + n == 0:
            n = 1
        shapes.append((prior, n))
    hkv = draw(hst.sampled_from([1, 2]))
    g = draw(hst.sampled_from([1, 2, 3]))
    dtype = draw(hst.sampled_from(["f32", "bf16"]))
    scale = draw(hst.sampled_from([0.0, 0.37, 1.5]))
    seed = draw(hst.integers(0, 2 ** 31 - 1))
    return shapes, hkv * g, hkv, dtype, scale, seed


@settings(**SETTINGS)
@given(small_batch())
def test_random_batches_match_brute_force(case):
    shapes, hq, hkv, dtype, scale, seed = case
    assume(sum(n for _, n in shapes) > 0)
    st = tiny_step(np.random.default_rng(seed), shapes, hq, hkv, 4, dtype)
    out, lse = run_oracle(st, scale)
    bf = brute_force(st, scale)
    assert len(bf) == out.shape[0] * hq
    for (t, h), (o, l) in bf.items():
        np.testing.assert_allclose(out[t, h], o, rtol=0, atol=1e-12)
        assert abs(lse[t, h] - l) <= 1e-12


@settings(**SETTINGS)
@given(small_batch(), hst.integers(1, 5))
def test_random_batches_split_equals_unsplit(case, splits):
    shapes, hq, hkv, dtype, scale, seed = case
    assume(sum(n for _, n in shapes) > 0)
    st = tiny_step(np.random.default_rng(seed), shapes, hq, hkv, 4, dtype)
    out, lse = run_oracle(st, scale)
    po, pl = run_oracle(st, scale, fn=oracle.attention_split_partials, num_splits=splits)
    so, sl = oracle.combine_partials(po, pl)
    np.testing.assert_allclose(so, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(sl, lse, rtol=0, atol=1e-12)


@settings(**SETTINGS)
@given(small_batch())
def test_random_batches_online_equals_full(case):
    shapes, hq, hkv, dtype, scale, seed = case
    assume(sum(n for _, n in shapes) > 0)
    rng = np.random.default_rng(seed)
    st = tiny_step(rng, shapes, hq, hkv, 4, dtype)
    out, lse = run_oracle(st, scale)
    tiles = [int(x) for x in rng.integers(1, 20, size=8)]
    oo, ol = run_oracle(st, scale, fn=oracle.attention_online, tile_sizes=tiles)
    np.testing.assert_allclose(oo, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ol, lse, rtol=0, atol=1e-12)
