"""GPU parity of steps that hold both prefill rows and decode rows, which the
library runs as one persistent launch (prefill units and decode units taken
from two device counters), against the fp64 oracle.

Each step has a few prefill requests (with and without prior context) and
enough decode requests (1 .. 16 / G new tokens each) that the host knows
decode rows are present.  Checked through the one-call step (the prefill
rows' tokens written over the work list, the decode rows' tokens inside the
launch) and through the plain attention entry point, for every group size,
both head dims, forced splits and an E4M3 cache.  Bars as in
test_gpu_parity: pools bit-exact, output 2e-2 (and relative 2e-2), lse 1e-3.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import Request, build_step, fp8_cache, raw_numpy

pytestmark = pytest.mark.gpu


def mixed_step(hq, hkv, d, seed, n_dec=None, dtype="bf16"):
    rng = np.random.default_rng(seed)
    dq = 16 // (hq // hkv)
    shapes = [(0, 70), (35, 150), (300, dq + 1)]            # prefill rows
    # decode requests average (dq + 1) / 2 tokens: this many make them certain
    n_dec = n_dec or 2 * (-(-(220 + dq + 1) // (dq + 1))) + 16
    for _ in range(n_dec):
        shapes.append((int(rng.integers(0, 700)), int(rng.integers(1, dq + 1))))
    shapes.append((40, 0))                                    # an empty request
    order = rng.permutation(len(shapes))
    need = [max(1, -(-(p + n) // 16)) for p, n in shapes]
    nb = sum(need) + 8
    perm = [int(x) for x in rng.permutation(nb)]
    tables, k = [], 0
    for n in need:
        tables.append(perm[k:k + n])
        k += n
    reqs = [Request(p, n, t) for (p, n), t in zip(shapes, tables)]
    step = build_step(f"mixed{hq}x{hkv}d{d}", reqs, dtype=dtype, num_q_heads=hq,
                      num_kv_heads=hkv, head_dim=d, num_blocks=nb, seed=seed, pad_tokens=2,
                      order=list(order))
    assert step.num_seqs > step.num_tokens // (dq + 1), "decode rows must be certain"
    assert step.max_query_len > dq
    return step


def upload(step):
    names = ["query", "key", "value", "k_pool", "v_pool"]
    if step.kv_cache == "fp8":
        names += ["k_scale", "v_scale"]
    g = {n: getattr(step, n).to("cuda").contiguous() for n in names}
    g["qsl"] = torch.as_tensor(step.query_start_loc).to("cuda")
    g["sl"] = torch.as_tensor(step.seq_lens).to("cuda")
    g["bt"] = torch.as_tensor(step.block_tables).to("cuda")
    g["sm"] = torch.as_tensor(step.slot_mapping).to("cuda")
    return g


def check(step, out, lse, ro, rl, what):
    n = int(step.query_start_loc[-1])
    o = out.float().cpu().double().numpy()[:n]
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = float(np.abs(o - ro[:n]).max())
    assert err <= 2e-2, f"{what}: max |out - oracle| = {err}"
    rel = float(np.linalg.norm(o - ro[:n]) / np.linalg.norm(ro[:n]))
    assert rel <= 2e-2, f"{what}: relative error {rel}"
    le = float(np.abs(lse.cpu().double().numpy()[:n] - rl[:n]).max())
    assert le <= 1e-3, f"{what}: max |lse - oracle| = {le}"
    # padded rows are never written
    assert torch.isnan(out[n:]).all()


def same(t, ref):
    return np.array_equal(np.ascontiguousarray(raw_numpy(t)).view(np.uint8),
                          np.ascontiguousarray(ref).view(np.uint8))


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 8, 64), (16, 1, 128), (16, 2, 64),
                                      (16, 8, 128), (16, 16, 64)])
@pytest.mark.parametrize("splits", [1, 3])
def test_mixed_step_one_call(hq, hkv, d, splits):
    import paged_attention_flat_amd as pa
    step = mixed_step(hq, hkv, d, seed=hq * 7 + hkv + d + splits)
    g = upload(step)
    out = torch.full_like(g["query"], float("nan"))
    out, lse = pa.decode_step(g["key"], g["value"], g["k_pool"], g["v_pool"], g["sm"],
                              g["query"], g["qsl"], g["sl"], g["bt"], step.max_query_len,
                              step.max_seq_len, step.scale, num_splits=splits, out=out)
    torch.cuda.synchronize()
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value),
                             raw_numpy(step.k_pool), raw_numpy(step.v_pool), step.slot_mapping)
    assert same(g["k_pool"], kp) and same(g["v_pool"], vp), "pools differ from the oracle's write"
    ro, rl = oracle.attention(raw_numpy(step.query), kp, vp, step.query_start_loc,
                              step.seq_lens, step.block_tables, step.scale, step.num_kv_heads,
                              step.dtype)
    check(step, out, lse, ro, rl, f"one call G={hq // hkv} d={d} S={splits}")


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (8, 4, 64)])
def test_mixed_step_attention_entry(hq, hkv, d):
    # the plain entry point over a cache the separate write filled
    import paged_attention_flat_amd as pa
    step = mixed_step(hq, hkv, d, seed=91 + d)
    g = upload(step)
    pa.kv_write(g["key"], g["value"], g["k_pool"], g["v_pool"], g["sm"])
    out = torch.full_like(g["query"], float("nan"))
    out, lse = pa.attention(g["query"], g["k_pool"], g["v_pool"], g["qsl"], g["sl"], g["bt"],
                            step.max_query_len, step.max_seq_len, step.scale, out=out)
    torch.cuda.synchronize()
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value),
                             raw_numpy(step.k_pool), raw_numpy(step.v_pool), step.slot_mapping)
    ro, rl = oracle.attention(raw_numpy(step.query), kp, vp, step.query_start_loc,
                              step.seq_lens, step.block_tables, step.scale, step.num_kv_heads,
                              step.dtype)
    check(step, out, lse, ro, rl, f"attention entry G={hq // hkv} d={d}")
    # the same step twice gives the same bytes (the work counters restart)
    out2 = torch.full_like(g["query"], float("nan"))
    out2, lse2 = pa.attention(g["query"], g["k_pool"], g["v_pool"], g["qsl"], g["sl"], g["bt"],
                              step.max_query_len, step.max_seq_len, step.scale, out=out2)
    torch.cuda.synchronize()
    n = int(step.query_start_loc[-1])         # (padded rows' lse is never written)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse[:n].view(torch.int32), lse2[:n].view(torch.int32))


@pytest.mark.parametrize("d", [64, 128])
def test_mixed_step_fp8_cache(d):
    import paged_attention_flat_amd as pa
    step = fp8_cache(mixed_step(32, 8, d, seed=55 + d), 55 + d)
    g = upload(step)
    out = torch.full_like(g["query"], float("nan"))
    out, lse = pa.decode_step_fp8(g["key"], g["value"], g["k_pool"], g["v_pool"], g["sm"],
                                  g["k_scale"], g["v_scale"], g["query"], g["qsl"], g["sl"],
                                  g["bt"], step.max_query_len, step.max_seq_len, step.scale,
                                  out=out)
    torch.cuda.synchronize()
    kp, vp = oracle.kv_write_fp8(raw_numpy(step.key), raw_numpy(step.value),
                                 raw_numpy(step.k_pool), raw_numpy(step.v_pool),
                                 step.slot_mapping, step.k_scale.numpy(), step.v_scale.numpy(),
                                 step.dtype)
    assert np.array_equal(g["k_pool"].cpu().numpy(), kp)
    assert np.array_equal(g["v_pool"].cpu().numpy(), vp)
    ro, rl = oracle.attention_fp8(raw_numpy(step.query), kp, vp, step.k_scale.numpy(),
                                  step.v_scale.numpy(), step.query_start_loc, step.seq_lens,
                                  step.block_tables, step.scale, step.num_kv_heads,
                                  query_dtype=step.dtype)
    check(step, out, lse, ro, rl, f"fp8 mixed d={d}")
