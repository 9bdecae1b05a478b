"""GPU parity of the fused rotary embedding + KV write against the oracle.

Bars, from the arithmetic (fp32 evaluation of x c - y s, one rounding to the
storage type): every rotated element within 2^-7 |ref| (two bf16 ulps; fp32:
2^-22 |ref|) plus 2^-20 (fp32: 2^-21) of its pair's norm, which covers the
fp32 error when the two products nearly cancel.  V and every byte not written
are bit-exact.  Attention after the fused write matches the oracle's
attention over its own rotated inputs within the usual bars.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import Request, build_step, config_step, raw_numpy, rope_table, token_positions

pytestmark = pytest.mark.gpu

SMALL = {
    2: {"context": 1000, "pool_blocks": 200},
    5: {"chunk": 90, "priors": (70, 300), "decodes": 40, "lo": 20, "hi": 900,
        "prefix": 64, "sharers": 10, "stride": 64},
}


def positions_of(step):
    pos = np.full(step.num_tokens, -1, dtype=np.int64)
    qsl = step.query_start_loc
    for b in range(step.num_seqs):
        n = int(qsl[b + 1] - qsl[b])
        ctx = int(step.seq_lens[b]) - n
        pos[int(qsl[b]): int(qsl[b + 1])] = ctx + np.arange(n)
    return pos


def widen(x, dtype):
    return oracle.to_f64(x, dtype)


def check_rotated(got, ref, dtype, what):
    g = widen(got, dtype)
    d = ref.shape[-1]
    pn = np.sqrt(ref[..., : d // 2] ** 2 + ref[..., d // 2:] ** 2)
    pn = np.concatenate([pn, pn], axis=-1)
    rel, slack = (2.0 ** -7, 2.0 ** -20) if dtype == "bf16" else (2.0 ** -22, 2.0 ** -21)
    bad = np.abs(g - ref) > rel * np.abs(ref) + slack * pn
    assert not bad.any(), f"{what}: {int(bad.sum())} elements off (first {np.argwhere(bad)[:3]})"


def run(step, max_pos, table_np):
    import paged_attention_flat_amd as pa
    dev = "cuda"
    q = step.query.to(dev).clone()
    k, v = step.key.to(dev), step.value.to(dev)
    kc, vc = step.k_pool.to(dev).clone(), step.v_pool.to(dev).clone()
    sm = torch.as_tensor(step.slot_mapping).to(dev)
    pos = torch.as_tensor(step.info["positions"]).to(dev)
    tab = torch.as_tensor(table_np).to(dev)
    pa.rope_kv_write(q, k, v, kc, vc, sm, pos, tab)
    torch.cuda.synchronize()
    return q, kc, vc


def rotated_positions_case(step, positions, max_pos):
    step.info["positions"] = positions
    table = rope_table(max_pos, step.head_dim)
    q, kc, vc = run(step, max_pos, table)
    qr, kp, vp = oracle.rope_kv_write(raw_numpy(step.query), raw_numpy(step.key),
                                      raw_numpy(step.value), raw_numpy(step.k_pool),
                                      raw_numpy(step.v_pool), step.slot_mapping, positions,
                                      table, step.dtype)
    return q, kc, vc, qr, kp, vp, table


@pytest.mark.parametrize("cfg", [2, 5])
def test_rope_kv_write_matches_oracle(cfg):
    step = config_step(cfg, scale_down=SMALL[cfg])
    pos = positions_of(step)
    q, kc, vc, qr, kp, vp, table = rotated_positions_case(step, pos, int(pos.max()) + 1)
    check_rotated(raw_numpy(q), qr, step.dtype, f"config{cfg} query")
    # rotated keys at their slots; everything else in the pools bit-exact
    written = np.zeros(kp.shape[0] * 16, dtype=bool)
    written[step.slot_mapping[step.slot_mapping >= 0]] = True
    w = written.reshape(kp.shape[0], 16)
    kg, kr = raw_numpy(kc), kp
    mask_k = np.broadcast_to(w[:, None, :, None], kg.shape)
    assert np.array_equal(kg[~mask_k], kr[~mask_k])
    kref = widen(kr, step.dtype)  # oracle's rounded keys; compare against its fp64 rotation
    krot = oracle.rope(raw_numpy(step.key), pos, table, step.dtype)
    for t, s in enumerate(step.slot_mapping):
        if s < 0:
            continue
        b, o = divmod(int(s), 16)
        check_rotated(kg[b, :, o, :], krot[t], step.dtype, f"config{cfg} key row {t}")
    assert np.array_equal(raw_numpy(vc).view(np.uint8), np.ascontiguousarray(vp).view(np.uint8))
    assert kref.shape == kg.shape


def test_rope_then_attention_end_to_end():
    import paged_attention_flat_amd as pa
    step = config_step(5, scale_down=SMALL[5])
    pos = positions_of(step)
    q, kc, vc, qr, kp, vp, table = rotated_positions_case(step, pos, int(pos.max()) + 1)
    dev = "cuda"
    out, lse = pa.attention(q, kc, vc, torch.as_tensor(step.query_start_loc).to(dev),
                            torch.as_tensor(step.seq_lens).to(dev),
                            torch.as_tensor(step.block_tables).to(dev), step.max_query_len,
                            step.max_seq_len, step.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(oracle.round_to(qr, "bf16"), kp, vp, step.query_start_loc,
                              step.seq_lens, step.block_tables, step.scale, step.num_kv_heads,
                              "bf16")
    rows = np.arange(int(step.query_start_loc[-1]))
    o = out.float().cpu().double().numpy()[rows]
    assert float(np.abs(o - ro[rows]).max()) <= 2e-2
    assert float(np.linalg.norm(o - ro[rows]) / np.linalg.norm(ro[rows])) <= 2e-2
    assert float(np.abs(lse.cpu().double().numpy()[rows] - rl[rows]).max()) <= 1e-3


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("f32", 128)])
def test_rope_dtypes_and_out_of_table_positions(dtype, d):
    reqs = [Request(3, 20, [5, 1]), Request(30, 2, [2, 0, 4])]
    step = build_step("rope", reqs, dtype=dtype, num_q_heads=8, num_kv_heads=2, head_dim=d,
                      num_blocks=8, seed=31, pad_tokens=2)
    pos = positions_of(step)
    pos[1] = 10 ** 6        # past the table: this token is left alone
    pos[-1] = -5            # padded token with a negative position
    q, kc, vc, qr, kp, vp, table = rotated_positions_case(step, pos, 64)
    check_rotated(raw_numpy(q)[:-2], qr[:-2], dtype, f"{dtype} d={d} query")
    assert np.array_equal(np.ascontiguousarray(raw_numpy(q)[1]).view(np.uint8),
                          np.ascontiguousarray(raw_numpy(step.query)[1]).view(np.uint8))
    assert np.array_equal(raw_numpy(vc).view(np.uint8), np.ascontiguousarray(vp).view(np.uint8))
    kg = raw_numpy(kc)
    krot = oracle.rope(raw_numpy(step.key), pos, table, dtype)
    for t, s in enumerate(step.slot_mapping):
        if s < 0:
            continue
        b, o = divmod(int(s), 16)
        if 0 <= pos[t] < 64:
            check_rotated(kg[b, :, o, :], krot[t], dtype, f"{dtype} key row {t}")
        else:
            # not written: the pool keeps its old bytes
            old = raw_numpy(step.k_pool)[b, :, o, :]
            assert np.array_equal(np.ascontiguousarray(kg[b, :, o, :]).view(np.uint8),
                                  np.ascontiguousarray(old).view(np.uint8))


def test_rope_kv_write_full_long_prefill_step():
    # the workload the benchmark times: all 4 x 8192 new tokens of the long
    # prefill step rotated and written in one launch.  Every rotated key and
    # a seeded sample of 2048 query tokens against the oracle; V and every
    # byte the write must not touch bit-exact over the whole pools.
    import paged_attention_flat_amd as pa
    step = config_step(4, device="cuda")
    pos = token_positions(step)
    maxp = int(pos.max()) + 1
    table = rope_table(maxp, step.head_dim)
    dev = "cuda"
    q = step.query.clone()
    kc, vc = step.k_pool.clone(), step.v_pool.clone()
    pa.rope_kv_write(q, step.key, step.value, kc, vc, torch.as_tensor(step.slot_mapping).to(dev),
                     torch.as_tensor(pos).to(dev), torch.as_tensor(table).to(dev))
    torch.cuda.synchronize()
    key = raw_numpy(step.key)
    krot = oracle.rope(key, pos, table, step.dtype)            # [Nt, Hkv, d] float64
    kg = raw_numpy(kc)
    sm = step.slot_mapping
    live = sm >= 0
    blk, off = sm[live] // 16, sm[live] % 16
    check_rotated(kg[blk, :, off, :], krot[live], step.dtype, "full long prefill keys")
    # everything but the written key rows keeps the old bytes
    written = np.zeros((kg.shape[0], 16), dtype=bool)
    written[blk, off] = True
    kold = raw_numpy(step.k_pool)
    keep = ~np.broadcast_to(written[:, None, :, None], kg.shape)
    assert np.array_equal(kg[keep], kold[keep])
    # V: the plain write, whole pool
    _, vp = oracle.kv_write(key, raw_numpy(step.value), kold, raw_numpy(step.v_pool), sm)
    assert np.array_equal(np.ascontiguousarray(raw_numpy(vc)).view(np.uint8),
                          np.ascontiguousarray(vp).view(np.uint8))
    rng = np.random.default_rng(44)
    pick = np.unique(np.concatenate([[0, step.num_tokens - 1],
                                     rng.integers(0, step.num_tokens, 2048)]))
    qg = raw_numpy(q[torch.as_tensor(pick).to(dev)])
    qr = oracle.rope(raw_numpy(step.query[torch.as_tensor(pick).to(dev)]), pos[pick], table,
                     step.dtype)
    check_rotated(qg, qr, step.dtype, "full long prefill queries (sampled)")
