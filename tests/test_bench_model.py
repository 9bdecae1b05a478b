"""The algorithmic bytes and FLOPs that bench.py divides by its times, pinned
to closed forms of the workload definitions (a wrong count would mis-state
every roofline fraction).  CPU only: the steps are built without values."""

import importlib.util
import os

import numpy as np

from workloads import Request, build_step, config_step

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench():
    spec = importlib.util.spec_from_file_location("bench_model", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_long_decode_bytes_and_flops():
    b = bench()
    step = config_step(2, with_values=False)
    w = b.work_model(step)
    hq, hkv, d, ctx = 32, 8, 128, 32768
    kv = ctx * 2 * hkv * d * 2                       # every cached token, K and V, bf16
    q_o = 2 * hq * d * 2 + hq * 4                    # Q read, output and lse written
    meta = (ctx // 16) * 4 + 3 * 4                   # table entries, qsl (2) and seq_lens (1)
    write = 2 * hkv * d * 2 * 2 + 8                  # new K and V read and written, one slot
    assert w["kv_bytes"] == kv == 134217728
    assert w["bytes"] == kv + q_o + meta + write == 134250644
    assert w["flops"] == 4 * d * hq * ctx            # one row against 32768 keys
    # the decode kernel alone: K/V, Q, table entries
    kb, toks = b.decode_kernel_bytes(step)
    assert (kb, toks) == (kv + hq * d * 2 + (ctx // 16) * 4, ctx)


def test_long_prefill_flops():
    b = bench()
    step = config_step(4, with_values=False)
    w = b.work_model(step)
    pairs = 4 * (8192 * 8193 // 2)                   # causal pairs of 4 fresh requests
    assert w["pairs"] == pairs
    assert w["flops"] == w["prefill_flops"] == 4 * 128 * 32 * pairs == 2199291691008
    assert w["kv_bytes"] == 4 * 8192 * 4096


def test_mixed_step_prefill_flops():
    b = bench()
    step = config_step(5, with_values=False)
    w = b.work_model(step)
    q = step.q_lens
    pre = np.nonzero(q > 4)[0]
    pairs = sum(int(q[i]) * int(step.seq_lens[i] - q[i]) + int(q[i]) * (int(q[i]) + 1) // 2
                for i in pre)
    # chunks of 2048 after 4096 and 16384 cached tokens
    assert pairs == 2048 * 4096 + 2048 * 2049 // 2 + 2048 * 16384 + 2048 * 2049 // 2
    assert w["prefill_flops"] == 4 * 128 * 32 * pairs


def test_large_batch_counts_every_context_token():
    b = bench()
    step = config_step(3, with_values=False)
    w = b.work_model(step)
    assert w["ctx_tokens"] == int(step.seq_lens.sum())     # no block is shared
    assert w["kv_bytes"] == int(step.seq_lens.sum()) * 4096


def test_shared_blocks_count_once():
    b = bench()
    prefix = [0, 1, 2, 3]
    reqs = [Request(64 + 5, 1, prefix + [4 + i]) for i in range(3)]
    step = build_step("share", reqs, dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                      num_blocks=8, seed=1, with_values=False)
    w = b.work_model(step)
    assert w["ctx_tokens"] == 64 + 3 * 6             # the prefix once, each tail block
