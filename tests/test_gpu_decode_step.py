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


def check_all(step, out, lse, g, what, before=None):
    # `before`: host copies of the pools taken before the call (needed when
    # the step lives on the GPU, where the call writes the step's own pools)
    kb, vb = before if before is not None else (raw_numpy(step.k_pool), raw_numpy(step.v_pool))
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value), kb, vb,
                             step.slot_mapping)
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


@pytest.mark.parametrize("splits", [0, 1])
def test_full_config2_decode_step(splits):
    # the headline workload in the launch the benchmark times: one call, the
    # new token written inside the decode launch, 32768 keys, the heuristic
    # split count (0) and no split (1).  Whole pools byte-compared, the row
    # against the oracle.
    step = config_step(2, device="cuda")
    before = (raw_numpy(step.k_pool), raw_numpy(step.v_pool))
    out, lse, g = run_step(step, splits)
    assert g["k_pool"].data_ptr() == step.k_pool.data_ptr()   # written in place
    check_all(step, out, lse, g, f"full config2 decode step S={splits}", before)


def test_full_config5_decode_step_pools():
    # the mixed step (prefill chunks + 4096 decodes, 65 GB of pools) through
    # the one call the benchmark times: every block holding a new token is
    # compared with the oracle's write of that block, and every other block
    # of both pools must keep its bytes (compared on the device against a
    # copy taken before the call)
    step = config_step(5, device="cuda")
    sm = step.slot_mapping
    blocks = np.unique(sm[sm >= 0] // 16)
    bidx = torch.as_tensor(blocks).to("cuda")
    k_before = {n: getattr(step, n).view(torch.int16).clone() for n in ("k_pool", "v_pool")}
    k_sel = {n: raw_numpy(getattr(step, n)[bidx]) for n in ("k_pool", "v_pool")}
    out, lse, g = run_step(step, 0)
    # the written blocks: the oracle's write applied to their old contents
    remap = {int(b): i for i, b in enumerate(blocks)}
    local = np.array([remap[int(s) // 16] * 16 + int(s) % 16 if s >= 0 else -1 for s in sm])
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value), k_sel["k_pool"],
                             k_sel["v_pool"], local)
    for name, ref in (("k_pool", kp), ("v_pool", vp)):
        got = raw_numpy(g[name][bidx])
        assert np.array_equal(np.ascontiguousarray(got).view(np.uint8),
                              np.ascontiguousarray(ref).view(np.uint8)), name
        keep = torch.ones(g[name].shape[0], dtype=torch.bool, device="cuda")
        keep[bidx] = False
        after = g[name].view(torch.int16)
        assert torch.equal(after[keep], k_before[name][keep]), f"{name}: other blocks changed"
    del k_before


def check_sampled_rows(step, out, lse, pick, what, sub=None, seed=0):
    # rows of the requests `pick` (or `sub` of them) against the oracle on a
    # compact copy of those requests; the step's pools were written in place,
    # which the oracle's own write repeats bit for bit
    from workloads import extract_requests
    small, rows = extract_requests(step, pick)
    idx = np.arange(len(rows)) if sub is None else np.asarray(sub)
    kp, vp = oracle.kv_write(raw_numpy(small.key), raw_numpy(small.value),
                             raw_numpy(small.k_pool), raw_numpy(small.v_pool), small.slot_mapping)
    ro, rl = oracle.attention(raw_numpy(small.query), kp, vp, small.query_start_loc,
                              small.seq_lens, small.block_tables, small.scale,
                              small.num_kv_heads, small.dtype, rows=idx)
    o = out.float().cpu().double().numpy()[rows[idx]]
    assert np.isfinite(o).all(), what
    assert float(np.abs(o - ro[idx]).max()) <= 2e-2, what
    assert float(np.linalg.norm(o - ro[idx]) / np.linalg.norm(ro[idx])) <= 2e-2, what
    assert float(np.abs(lse.cpu().double().numpy()[rows[idx]] - rl[idx]).max()) <= 1e-3, what


def test_full_config3_decode_step():
    # the large-batch decode in the launch the benchmark times: one call (the
    # new tokens written inside the decode launch), no split, the automatic V
    # read policy (every request's first block is its own).  Every written
    # block byte-compared with the oracle's write, nine requests' rows (the
    # shortest, the longest and three seeded ones) against the oracle.
    step = config_step(3, device="cuda")
    sm = step.slot_mapping
    blocks = np.unique(sm[sm >= 0] // 16)
    bidx = torch.as_tensor(blocks).to("cuda")
    k_sel = {n: raw_numpy(getattr(step, n)[bidx]) for n in ("k_pool", "v_pool")}
    out, lse, g = run_step(step, 0)
    remap = {int(b): i for i, b in enumerate(blocks)}
    local = np.array([remap[int(s) // 16] * 16 + int(s) % 16 if s >= 0 else -1 for s in sm])
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value), k_sel["k_pool"],
                             k_sel["v_pool"], local)
    for name, ref in (("k_pool", kp), ("v_pool", vp)):
        got = raw_numpy(g[name][bidx])
        assert np.array_equal(np.ascontiguousarray(got).view(np.uint8),
                              np.ascontiguousarray(ref).view(np.uint8)), name
    order = np.argsort(step.seq_lens)
    rng = np.random.default_rng(33)
    pick = sorted(set(order[:3].tolist() + order[-3:].tolist() +
                      rng.choice(step.num_seqs, 3, replace=False).tolist()))
    check_sampled_rows(step, out, lse, pick, "full config3 decode step")


def test_full_config5_decode_step_rows():
    # the mixed step through the one call the benchmark times (persistent
    # launch, automatic V read policy: sharers of the prefix cached, the
    # others streamed): sampled decode rows of sharers and non-sharers and
    # seeded rows of both chunks against the oracle
    step = config_step(5, device="cuda")
    out, lse, g = run_step(step, 0)
    ql = np.diff(step.query_start_loc)
    shared = set(step.info["shared_blocks"])
    dec = np.nonzero(ql == 1)[0]
    sharers = [int(b) for b in dec if int(step.block_tables[b, 0]) in shared]
    non = [int(b) for b in dec if int(step.block_tables[b, 0]) not in shared]
    rng = np.random.default_rng(55)
    pick = sorted(rng.choice(sharers, 4, replace=False).tolist() +
                  rng.choice(non, 4, replace=False).tolist())
    check_sampled_rows(step, out, lse, pick, "full config5 decode step (decode rows)")
    for c in np.nonzero(ql > 1)[0]:
        sub = sorted(int(x) for x in rng.choice(int(ql[c]), 24, replace=False))
        check_sampled_rows(step, out, lse, [int(c)], f"full config5 decode step (chunk {c})",
                           sub=sub)


def check_pools(step, g, before, what):
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value), before[0], before[1],
                             step.slot_mapping)
    for got, ref, name in ((g["k_pool"], kp, "K"), (g["v_pool"], vp, "V")):
        gb = np.ascontiguousarray(raw_numpy(got)).view(np.uint8)
        assert np.array_equal(gb, np.ascontiguousarray(ref).view(np.uint8)), f"{what}: {name} pool"
    return kp, vp


def test_full_config4_step():
    # the long prefill step (4 x 8192 new tokens) through the one call the
    # benchmark times: both 128 MB pools byte-compared with the oracle's
    # write, then a seeded sample of rows (first, last and 40 random rows of
    # each request) against the oracle's attention over its own pools
    step = config_step(4, device="cuda")
    before = (raw_numpy(step.k_pool), raw_numpy(step.v_pool))
    out, lse, g = run_step(step, 0)
    kp, vp = check_pools(step, g, before, "full config4")
    rng = np.random.default_rng(404)
    qsl = step.query_start_loc
    rows = []
    for b in range(step.num_seqs):
        lo, hi = int(qsl[b]), int(qsl[b + 1])
        rows += [lo, hi - 1] + rng.integers(lo, hi, 40).tolist()
    rows = sorted(set(rows))
    ro, rl = oracle.attention(raw_numpy(step.query), kp, vp, step.query_start_loc,
                              step.seq_lens, step.block_tables, step.scale, step.num_kv_heads,
                              step.dtype, rows=rows)
    o = out.float().cpu().double().numpy()[rows]
    assert np.isfinite(o).all()
    assert float(np.abs(o - ro[rows]).max()) <= 2e-2
    assert float(np.linalg.norm(o - ro[rows]) / np.linalg.norm(ro[rows])) <= 2e-2
    assert float(np.abs(lse.cpu().double().numpy()[rows] - rl[rows]).max()) <= 1e-3
