"""The seeded input generator: metadata consistency (checked by the oracle's
validator), determinism, and the shapes the five workloads promise."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import Request, build_step, config_step, extract_requests, raw_numpy


def _validate(step):
    oracle.validate_step(step.query_start_loc, step.seq_lens, step.block_tables,
                         step.slot_mapping, step.num_tokens, step.num_blocks)


def test_page_schedule_metadata_matches_oracle_flatten():
    sched = [(0, 5, [7]), (37, 1, [2, 9, 4]), (32, 3, [11, 12, 3])]
    st = build_step("page", [Request(p, n, t) for p, n, t in sched], dtype="f32",
                    num_q_heads=2, num_kv_heads=1, head_dim=8, num_blocks=16, seed=0)
    ref = oracle.flatten_schedule(sched)
    assert st.query_start_loc.tolist() == ref["query_start_loc"]
    assert st.seq_lens.tolist() == ref["seq_lens"]
    assert st.slot_mapping.tolist() == ref["slot_mapping"]
    _validate(st)


def test_config1_shape():
    st = config_step(1)
    assert st.dtype == "f32" and st.num_q_heads == 4 and st.num_kv_heads == 2
    assert st.head_dim == 64 and st.num_blocks == 32 and st.scale == 0.125
    assert st.query_start_loc.tolist() == [0, 37, 38, 39, 40]
    assert st.seq_lens.tolist() == [37, 5, 17, 64]
    used = np.concatenate([st.block_tables[b, :n] for b, n in enumerate([3, 1, 2, 4])])
    assert sorted(used.tolist()) == sorted(np.unique(used).tolist()) and used.size == 10
    _validate(st)
    alt = config_step(1, variant="alt")
    assert alt.seq_lens.tolist() == [37, 6, 18, 65]
    _validate(alt)


def test_config1_poison_and_determinism():
    a = config_step(1)
    b = config_step(1)
    for x, y in [(a.query, b.query), (a.k_pool, b.k_pool), (a.v_pool, b.v_pool)]:
        assert torch.equal(torch.nan_to_num(x, 7.0), torch.nan_to_num(y, 7.0))
    # slots of new tokens are poisoned before the write
    s = int(a.slot_mapping[0])
    assert torch.isnan(a.k_pool[s // 16, :, s % 16, :]).all()
    assert torch.isnan(a.v_pool[s // 16, :, :, s % 16]).all()
    # a prior-context slot of request 3 holds a finite value
    blk = int(a.block_tables[3, 0])
    assert torch.isfinite(a.k_pool[blk, :, 0, :]).all()


@pytest.mark.parametrize("cfg,sd", [
    (2, {"context": 1000, "pool_blocks": 128}),
    (3, {"batch": 6, "lo": 20, "hi": 90}),
    (4, {"batch": 2, "new": 70, "pool_blocks": 20}),
    (5, {"chunk": 40, "priors": (33, 70), "decodes": 24, "lo": 10, "hi": 200,
         "prefix": 32, "sharers": 6, "stride": 20}),
])
def test_scaled_down_configs_validate(cfg, sd):
    st = config_step(cfg, scale_down=sd)
    _validate(st)
    assert st.dtype == "bf16" and st.num_q_heads == 32 and st.num_kv_heads == 8
    assert st.head_dim == 128


def test_config5_structure_full_metadata():
    st = config_step(5, with_values=False)
    q = st.q_lens
    assert st.num_seqs == 4098 and st.num_tokens == 8192
    assert sorted(q.tolist())[-2:] == [2048, 2048] and (q == 1).sum() == 4096
    assert st.block_tables.shape[1] == 1152
    shared = set(st.info["shared_blocks"])
    rows_with_shared = sum(1 for b in range(st.num_seqs)
                           if int(st.block_tables[b, 0]) in shared)
    assert rows_with_shared == st.info["num_sharers"] == 1024
    assert workloads.unique_block_count(st) == st.info["unique_blocks"]
    assert st.max_seq_len == 18432


def test_config3_and_2_full_metadata():
    st = config_step(3, with_values=False)
    assert st.num_seqs == 256 and st.num_tokens == 256
    assert st.seq_lens.min() >= 512 and st.seq_lens.max() <= 8192
    st2 = config_step(2, with_values=False)
    assert st2.seq_lens.tolist() == [32768] and st2.num_blocks == 4096
    assert len(set(st2.block_tables[0].tolist())) == 2048


@pytest.mark.parametrize("cfg", [2, 3])
def test_tensor_parallel_shard_keeps_requests_and_placement(cfg):
    # one GPU's share at 8-way tensor parallelism: the heads change, nothing else
    full = config_step(cfg, with_values=False)
    shard = config_step(cfg, with_values=False, scale_down={"q_heads": 4, "kv_heads": 1})
    assert (shard.num_q_heads, shard.num_kv_heads) == (4, 1)
    assert shard.seq_lens.tolist() == full.seq_lens.tolist()
    assert (shard.block_tables == full.block_tables).all()
    assert list(shard.slot_mapping) == list(full.slot_mapping)
    assert shard.num_blocks == full.num_blocks


def test_extract_requests_preserves_rows():
    st = config_step(5, scale_down={"chunk": 40, "priors": (33, 70), "decodes": 24,
                                    "lo": 10, "hi": 200, "prefix": 32, "sharers": 6,
                                    "stride": 20})
    ids = [0, 3, 7]
    small, rows = extract_requests(st, ids)
    _validate(small)
    assert torch.equal(torch.nan_to_num(small.query), torch.nan_to_num(st.query[rows]))
    # the oracle gives the same rows either way
    kp, vp = oracle.kv_write(raw_numpy(st.key), raw_numpy(st.value), raw_numpy(st.k_pool),
                             raw_numpy(st.v_pool), st.slot_mapping)
    full, _ = oracle.attention(raw_numpy(st.query), kp, vp, st.query_start_loc,
                               st.seq_lens, st.block_tables, st.scale, 8, "bf16",
                               rows=rows.tolist())
    kp2, vp2 = oracle.kv_write(raw_numpy(small.key), raw_numpy(small.value),
                               raw_numpy(small.k_pool), raw_numpy(small.v_pool),
                               small.slot_mapping)
    part, _ = oracle.attention(raw_numpy(small.query), kp2, vp2, small.query_start_loc,
                               small.seq_lens, small.block_tables, small.scale, 8, "bf16")
    np.testing.assert_array_equal(part, full[rows])
