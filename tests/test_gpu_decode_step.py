"""GPU parity of the one-call decode step (KV write + attention, fused into
the decode kernel for bf16 decode steps) against the fp64 oracle: pools
bit-exact after the step, outputs within the usual bars (max-abs 2e-2 /
relative 2e-2 bf16, 1e-4 fp32; lse 1e-3)."""

import numpy as np
import pytest
import torch

import oracle
from workloads import Request, build_step, config_step, raw_numpy

pytestmark = pytest.mark.gpu

SMALL = {
    2: {"context": 1000, "pool_blocks": 200},
    3: {"batch": 12, "lo": 40, "hi": 700},
    5: {"chunk": 90, "priors": (70, 300), "decodes": 40, "lo": 20, "hi": 900,
        "prefix": 64, "sharers": 10, "stride": 64},
}


def run_step(step, num_splits=0):
    import paged_attention_flat_amd as pa
    dev = "cuda"
    g = {n: getattr(step, n).to(dev).contiguous()
         for n in ("query", "key", "value", "k_pool", "v_pool")}
    out = torch.full_like(g["query"], float("nan"))
    out, lse = pa.decode_step(g["key"], g["value"], g["k_pool"], g["v_pool"],
                              torch.as_tensor(step.slot_mapping).to(dev), g["query"],
                              torch.as_tensor(step.query_start_loc).to(dev),
                              torch.as_tensor(step.seq_lens).to(dev),
                              torch.as_tensor(step.block_tables).to(dev), step.max_query_len,
                              step.max_seq_len, step.scale, num_splits=num_splits, out=out)
    torch.cuda.synchronize()
    return out, lse, g


def check_all(step, out, lse, g, what):
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value), raw_numpy(step.k_pool),
                             raw_numpy(step.v_pool), step.slot_mapping)
    for got, ref in ((g["k_pool"], kp), (g["v_pool"], vp)):
        gb = np.ascontiguousarray(raw_numpy(got)).view(np.uint8)
        assert np.array_equal(gb, np.ascontiguousarray(ref).view(np.uint8)), f"{what}: pool"
    ro, rl = oracle.attention(raw_numpy(step.query), kp, vp, step.query_start_loc,
                              step.seq_lens, step.block_tables, step.scale, step.num_kv_heads,
                              step.dtype)
    rows = np.arange(int(step.query_start_loc[-1]))
    o = out.float().cpu().double().numpy()[rows]
    tol = 2e-2 if step.dtype == "bf16" else 1e-4
    assert np.isfinite(o).all(), f"{what}: non-finite"
    assert float(np.abs(o - ro[rows]).max()) <= tol, what
    assert float(np.linalg.norm(o - ro[rows]) / np.linalg.norm(ro[rows])) <= tol, what
    assert float(np.abs(lse.cpu().double().numpy()[rows] - rl[rows]).max()) <= 1e-3, what


@pytest.mark.parametrize("cfg,splits", [(2, 0), (2, 1), (2, 7), (3, 0), (3, 4)])
def test_decode_step_fused_small_configs(cfg, splits):
    step = config_step(cfg, scale_down=SMALL[cfg])
    out, lse, g = run_step(step, splits)
    check_all(step, out, lse, g, f"config{cfg} S={splits}")


def test_decode_step_tokens_across_blocks_and_splits():
    # up to 4 new tokens (G = 4) straddling block and split boundaries, plus
    # trailing tokens after the last request: one written, two padded
    rng = np.random.default_rng(5)
    shapes = [(30, 4), (14, 3), (1000, 2), (47, 1), (0, 4)]
    need = [-(-(p + n) // 16) for p, n in shapes]
    nb = sum(need) + 6
    perm = [int(x) for x in rng.permutation(nb)]
    tables, k = [], 0
    for n in need:
        tables.append(perm[k:k + n])
        k += n
    step = build_step("straddle", [Request(p, n, t) for (p, n), t in zip(shapes, tables)],
                      dtype="bf16", num_q_heads=16, num_kv_heads=4, head_dim=128,
                      num_blocks=nb, seed=77, pad_tokens=3)
    sm = step.slot_mapping.copy()
    sm[-2] = perm[k] * 16 + 5          # a trailing token written to a free block
    step.slot_mapping = sm
    for splits in (0, 32, 63, 256):
        out, lse, g = run_step(step, splits)
        check_all(step, out, lse, g, f"straddle S={splits}")


@pytest.mark.parametrize("group,head_dim", [(1, 128), (2, 64), (8, 128), (16, 128), (16, 64)])
def test_decode_step_group_sizes(group, head_dim):
    # every group size the decode kernel packs (16 / G new tokens per
    # request), new tokens in a wave's first pair, in two pairs owned by
    # different waves, and across split boundaries; both launch shapes
    dq = 16 // group
    rng = np.random.default_rng(11 + group)
    shapes = [(0, dq), (30, dq), (17, max(1, dq // 2)), (600, 1), (63, dq), (5, 0)]
    need = [max(1, -(-(p + n) // 16)) for p, n in shapes]
    nb = sum(need) + 4
    perm = [int(x) for x in rng.permutation(nb)]
    tables, k = [], 0
    for n in need:
        tables.append(perm[k:k + n])
        k += n
    step = build_step(f"groups{group}", [Request(p, n, t) for (p, n), t in zip(shapes, tables)],
                      dtype="bf16", num_q_heads=2 * group, num_kv_heads=2, head_dim=head_dim,
                      num_blocks=nb, seed=90 + group, pad_tokens=2)
    for splits in (0, 3, 40):
        out, lse, g = run_step(step, splits)
        check_all(step, out, lse, g, f"G={group} d={head_dim} S={splits}")


def test_decode_step_falls_back_for_prefill_rows_and_fp32():
    step = config_step(5, scale_down=SMALL[5])
    out, lse, g = run_step(step)
    check_all(step, out, lse, g, "mixed step (two calls)")
    step1 = config_step(1)
    out, lse, g = run_step(step1)
    check_all(step1, out, lse, g, "fp32 step (two calls)")
