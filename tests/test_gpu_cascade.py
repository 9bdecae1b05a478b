"""GPU parity of shared-prefix (cascade) attention against the fp64 oracle.

The cascade path reads the shared blocks once for all sharers' decode rows
and merges that partial into each sharer's own splits; the result must be
plain attention (oracle.attention), within the usual bars: output max-abs
2e-2 and relative Frobenius 2e-2, lse 1e-3.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import Request, build_step, config_step, extract_requests, raw_numpy

pytestmark = pytest.mark.gpu

SMALL5 = {"chunk": 90, "priors": (70, 300), "decodes": 40, "lo": 20, "hi": 900,
          "prefix": 64, "sharers": 10, "stride": 64}


def sharers_of(step, prefix):
    P = len(prefix)
    return [b for b in range(step.num_seqs)
            if step.block_tables.shape[1] >= P and
            list(step.block_tables[b, :P]) == list(prefix)]


def run_cascade(step, sharers, prefix, num_splits=0):
    import paged_attention_flat_amd as pa
    dev = "cuda"
    g = {n: getattr(step, n).to(dev) for n in ("query", "key", "value", "k_pool", "v_pool")}
    qsl = torch.as_tensor(step.query_start_loc).to(dev)
    sl = torch.as_tensor(step.seq_lens).to(dev)
    bt = torch.as_tensor(step.block_tables).to(dev)
    pa.kv_write(g["key"], g["value"], g["k_pool"], g["v_pool"],
                torch.as_tensor(step.slot_mapping).to(dev))
    out = torch.full_like(g["query"], float("nan"))
    out, lse = pa.attention_cascade(g["query"], g["k_pool"], g["v_pool"], qsl, sl, bt,
                                    step.max_query_len, step.max_seq_len, step.scale,
                                    torch.as_tensor(np.asarray(sharers, dtype=np.int32)).to(dev),
                                    torch.as_tensor(np.asarray(prefix, dtype=np.int32)).to(dev),
                                    num_splits=num_splits, out=out)
    torch.cuda.synchronize()
    return out, lse


def oracle_plain(step, rows=None):
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value),
                             raw_numpy(step.k_pool), raw_numpy(step.v_pool), step.slot_mapping)
    return oracle.attention(raw_numpy(step.query), kp, vp, step.query_start_loc, step.seq_lens,
                            step.block_tables, step.scale, step.num_kv_heads, step.dtype,
                            rows=rows)


def check(out, lse, ro, rl, rows, what):
    o = out.float().cpu().double().numpy()[rows]
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = float(np.abs(o - ro[rows]).max())
    assert err <= 2e-2, f"{what}: max |out - oracle| = {err}"
    rel = float(np.linalg.norm(o - ro[rows]) / np.linalg.norm(ro[rows]))
    assert rel <= 2e-2, f"{what}: relative error {rel}"
    le = float(np.abs(lse.cpu().double().numpy()[rows] - rl[rows]).max())
    assert le <= 1e-3, f"{what}: max |lse - oracle| = {le}"


@pytest.mark.parametrize("splits", [1, 4])
def test_cascade_mixed_step_small(splits):
    step = config_step(5, scale_down=SMALL5)
    prefix = list(step.info["shared_blocks"])
    sharers = sharers_of(step, prefix)
    assert len(sharers) >= 5
    out, lse = run_cascade(step, sharers, prefix, num_splits=splits)
    ro, rl = oracle_plain(step)
    rows = np.arange(int(step.query_start_loc[-1]))
    check(out, lse, ro, rl, rows, f"cascade small config5 S={splits}")


@pytest.mark.parametrize("splits", [1, 3])
def test_cascade_persistent_mixed_step(splits):
    # enough decode requests that the host knows decode rows are present: the
    # prefix stage runs, then the prefill and decode units share one
    # persistent launch whose sharers' decode units merge the stage's partials
    import paged_attention_flat_amd as pa
    step = config_step(5, scale_down=dict(SMALL5, decodes=80, sharers=20))
    assert step.num_seqs > step.num_tokens // 5 and step.max_query_len > 4
    prefix = list(step.info["shared_blocks"])
    sharers = sharers_of(step, prefix)
    assert len(sharers) >= 10
    pa.trace_begin()
    out, lse = run_cascade(step, sharers, prefix, num_splits=splits)
    names = [n for n, _ in pa.trace_read()]
    pa.trace_end()
    assert "cascade_prefix" in names and "mixed_prefill_decode" in names, names
    assert names.index("cascade_prefix") < names.index("mixed_prefill_decode"), names
    ro, rl = oracle_plain(step)
    rows = np.arange(int(step.query_start_loc[-1]))
    check(out, lse, ro, rl, rows, f"cascade persistent config5 S={splits}")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (32, 4), (16, 2)])
def test_cascade_edge_cases(hq, hkv):
    # sharers: decodes with 1 and 2 new tokens, one whose context ends inside
    # the prefix, a prefill-row sharer (computed as usual); plus non-sharers
    rng = np.random.default_rng(hq + 7 * hkv)
    P = 3
    nb = 64
    perm = list(rng.permutation(nb))
    prefix = perm[:P]
    k = P
    shapes = [(100, 1, True), (60, 2, True), (20, 1, True), (70, 40, True), (50, 1, False),
              (0, 9, False), (130, 1, True)]
    reqs, sharers = [], []
    for i, (prior, n, share) in enumerate(shapes):
        need = -(-(prior + n) // 16)
        own = need - P if share else need
        own = max(own, 0)
        table = (prefix[:min(P, need)] if share else []) + perm[k:k + own]
        if share and need < P:
            table = prefix[:need]
        k += own
        reqs.append(Request(prior, n, table))
        if share:
            sharers.append(i)
    step = build_step("casc", reqs, dtype="bf16", num_q_heads=hq, num_kv_heads=hkv,
                      head_dim=128, num_blocks=nb, seed=int(rng.integers(1 << 30)), pad_tokens=2)
    for splits in (1, 3):
        out, lse = run_cascade(step, sharers, prefix, num_splits=splits)
        ro, rl = oracle_plain(step)
        rows = np.arange(int(step.query_start_loc[-1]))
        check(out, lse, ro, rl, rows, f"cascade G={hq // hkv} S={splits}")
        assert torch.isnan(out[-2:]).all()


def test_cascade_full_mixed_step_sampled():
    step = config_step(5, device="cuda")
    prefix = list(step.info["shared_blocks"])
    sharers = sharers_of(step, prefix)
    assert len(sharers) == step.info["num_sharers"]
    out, lse = run_cascade(step, sharers, prefix)
    rng = np.random.default_rng(3)
    non = [b for b in range(step.num_seqs) if b not in set(sharers)
           and int(step.query_start_loc[b + 1] - step.query_start_loc[b]) == 1]
    pick = list(rng.choice(sharers, 6, replace=False)) + list(rng.choice(non, 2, replace=False))
    small, rows = extract_requests(step, pick)
    ro, rl = oracle_plain(small)
    o_rows = np.arange(len(rows))
    o = out.float().cpu().double().numpy()[rows]
    ref = ro[o_rows]
    assert float(np.abs(o - ref).max()) <= 2e-2
    assert float(np.linalg.norm(o - ref) / np.linalg.norm(ref)) <= 2e-2
    assert float(np.abs(lse.cpu().double().numpy()[rows] - rl[o_rows]).max()) <= 1e-3


@pytest.mark.parametrize("splits", [0, 1, 5])
def test_cascade_long_shared_prefix(splits):
    # 16 decodes sharing a 2048-token prefix, private suffixes of 10..300 tokens
    from workloads import shared_prefix_step
    step = shared_prefix_step(16, 2048, 10, 300, 7, num_q_heads=16, num_kv_heads=4)
    prefix = list(step.info["shared_blocks"])
    out, lse = run_cascade(step, list(range(16)), prefix, num_splits=splits)
    ro, rl = oracle_plain(step)
    check(out, lse, ro, rl, np.arange(16), f"long shared prefix S={splits}")


def test_cascade_key_ranges_with_short_sharers():
    # a 2048-token prefix cut into many key ranges; two sharers end early
    # inside it (100 and 700 tokens), so they see no key in most ranges
    rng = np.random.default_rng(12)
    P = 128
    nb = 400
    perm = [int(x) for x in rng.permutation(nb)]
    prefix = perm[:P]
    k = P
    reqs = []
    for prior in (2048 + 40, 2048 + 333, 100, 700, 2048 + 7, 2048 + 250):
        need = -(-(prior + 1) // 16)
        if need <= P:
            table = prefix[:need]
        else:
            table = prefix + perm[k:k + need - P]
            k += need - P
        reqs.append(Request(prior, 1, table))
    step = build_step("short-sharers", reqs, dtype="bf16", num_q_heads=16, num_kv_heads=4,
                      head_dim=128, num_blocks=nb, seed=12)
    for splits in (1, 4):
        out, lse = run_cascade(step, list(range(6)), prefix, num_splits=splits)
        ro, rl = oracle_plain(step)
        check(out, lse, ro, rl, np.arange(6), f"short sharers S={splits}")
