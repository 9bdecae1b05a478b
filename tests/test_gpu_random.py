"""GPU parity on random small batches (hypothesis, derandomized, bounded
examples) and the decode and prefill kernels on the same rows.

Each example draws a flat step (also over an E4M3 cache) -- 1 to 5 requests, each with 0 to 40 new
tokens on 0 to 200 tokens of prior context (so rows go to the decode or the
matrix-core kernel, splits or not, blocks end anywhere), block placement a
seeded permutation of a NaN-poisoned pool, group sizes 1 to 8, head dims 64
and 128, bf16 and fp32 -- and compares the library, called through its C ABI,
with the fp64 oracle at the bars of test_gpu_parity.
"""

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as hst

from test_gpu_parity import TOL_OUT, check, run_gpu, run_oracle, to64
from workloads import Request, build_step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    import paged_attention_flat_amd as pa  # noqa: F401  (fails loudly without libpa.so)


def random_step(shapes, hq, hkv, d, dtype, seed):
    rng = np.random.default_rng(seed)
    need = [-(-(p + n) // 16) for p, n in shapes]
    pool = sum(need) + 5
    perm = rng.permutation(pool)
    reqs, k = [], 0
    for (p, n), nb in zip(shapes, need):
        reqs.append(Request(p, n, list(perm[k:k + nb])))
        k += nb
    return build_step("random", reqs, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                      head_dim=d, num_blocks=pool, seed=seed)


@hst.composite
def flat_step(draw):
    B = draw(hst.integers(1, 5))
    shapes = []
    for _ in range(B):
        n = draw(hst.sampled_from([0, 1, 1, 2, 3, 4, 5, 9, 16, 17, 40]))
        prior = draw(hst.integers(0, 200))
        if prior + n == 0:
            n = 1
        shapes.append((prior, n))
    if sum(n for _, n in shapes) == 0:
        shapes[0] = (shapes[0][0], 1)
    hkv = draw(hst.sampled_from([1, 2]))
    g = draw(hst.sampled_from([1, 2, 4, 8]))
    d = draw(hst.sampled_from([64, 128]))
    dtype = draw(hst.sampled_from(["bf16", "f32"]))
    splits = draw(hst.sampled_from([0, 1, 3]))
    seed = draw(hst.integers(0, 2 ** 31 - 1))
    return shapes, hkv * g, hkv, d, dtype, splits, seed


@settings(max_examples=60, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(flat_step())
def test_random_flat_steps_match_oracle(case):
    shapes, hq, hkv, d, dtype, splits, seed = case
    step = random_step(shapes, hq, hkv, d, dtype, seed)
    print(f"case shapes={shapes} hq={hq} hkv={hkv} d={d} {dtype} splits={splits} seed={seed}",
          flush=True)
    out, lse, _ = run_gpu(step, num_splits=splits)
    (ro, rl), _ = run_oracle(step)
    check(step, out, lse, ro, rl, what=f"random {shapes} hq={hq} hkv={hkv} d={d} {dtype}")


@pytest.mark.parametrize("dtype,d,hq,hkv,n", [("bf16", 128, 32, 8, 5), ("bf16", 64, 8, 8, 17),
                                              ("f32", 64, 4, 2, 9)])
def test_decode_and_prefill_kernels_agree_on_the_same_row(dtype, d, hq, hkv, n):
    # the last row of a request with n new tokens (more than the decode kernel
    # packs for this group size: the matrix-core kernel) is the same row as a
    # one-token decode of that token over the same cache (the decode kernel)
    import paged_attention_flat_amd as pa
    prior = 150
    step = random_step([(prior, n)], hq, hkv, d, dtype, seed=n)
    out_a, lse_a, g = run_gpu(step)
    qsl = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    sl = torch.tensor([prior + n], dtype=torch.int32, device="cuda")
    q1 = g["query"][-1:].contiguous()
    out_b, lse_b = pa.attention(q1, g["k_pool"], g["v_pool"], qsl, sl, g["tables"], 1,
                                prior + n, step.scale, want_lse=True)
    torch.cuda.synchronize()
    (ro, rl), _ = run_oracle(step)
    a, b = to64(out_a)[-1], to64(out_b)[0]
    assert np.abs(a - ro[-1]).max() <= TOL_OUT[dtype]
    assert np.abs(b - ro[-1]).max() <= TOL_OUT[dtype]
    assert np.abs(a - b).max() <= TOL_OUT[dtype]
    la, lb = lse_a[-1].cpu().double().numpy(), lse_b[0].cpu().double().numpy()
    assert np.abs(la - rl[-1]).max() <= 1e-3 and np.abs(lb - rl[-1]).max() <= 1e-3


@settings(max_examples=30, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(flat_step())
def test_random_flat_steps_fp8_cache_match_oracle(case):
    # the same random steps over an E4M3 cache (bf16 query): quantised write
    # bit-exact, attention against the oracle over the dequantised pools
    from test_gpu_fp8 import check as check8, oracle_attn, oracle_write, run_gpu as run_gpu8
    from test_gpu_fp8 import same_codes
    from workloads import fp8_cache
    shapes, hq, hkv, d, _, splits, seed = case
    step = fp8_cache(random_step(shapes, hq, hkv, d, "bf16", seed), seed % 1000)
    print(f"fp8 case shapes={shapes} hq={hq} hkv={hkv} d={d} splits={splits} seed={seed}",
          flush=True)
    out, lse, g = run_gpu8(step, num_splits=splits)
    kp, vp = oracle_write(step)
    assert same_codes(g["k_pool"], kp) and same_codes(g["v_pool"], vp)
    ro, rl = oracle_attn(step, kp, vp)
    check8(step, out, lse, ro, rl, what=f"fp8 random {shapes} hq={hq} hkv={hkv} d={d}")

