"""GPU parity of the one-call shared-prefix decode step (pa_decode_step_cascade).

The step writes every new token in the launch of the shared-prefix setup and
then runs the prefix stage and the rest of the step; its pools, out and lse
must equal those of pa_kv_write followed by pa_attention_fwd_cascade bit for
bit, the pools must equal the oracle's write byte for byte, and the rows must
equal plain attention (oracle.attention) within the usual bars (output
max-abs 2e-2 and relative Frobenius 2e-2, lse 1e-3).
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import Request, build_step, config_step, raw_numpy, shared_prefix_step

pytestmark = pytest.mark.gpu

SMALL5 = {"chunk": 90, "priors": (70, 300), "decodes": 40, "lo": 20, "hi": 900,
          "prefix": 64, "sharers": 10, "stride": 64}


def _sharers_of(step, prefix):
    P = len(prefix)
    return [b for b in range(step.num_seqs)
            if step.block_tables.shape[1] >= P and
            list(step.block_tables[b, :P]) == list(prefix)]


def _inputs(step, sharers, prefix):
    dev = "cuda"
    g = {n: getattr(step, n).to(dev) for n in ("query", "key", "value", "k_pool", "v_pool")}
    g["qsl"] = torch.as_tensor(step.query_start_loc).to(dev)
    g["sl"] = torch.as_tensor(step.seq_lens).to(dev)
    g["bt"] = torch.as_tensor(step.block_tables).to(dev)
    g["slots"] = torch.as_tensor(step.slot_mapping).to(dev)
    g["sh"] = torch.as_tensor(np.asarray(sharers, dtype=np.int32)).to(dev)
    g["pb"] = torch.as_tensor(np.asarray(prefix, dtype=np.int32)).to(dev)
    g["out"] = torch.full_like(g["query"], float("nan"))
    g["lse"] = torch.full((g["query"].shape[0], g["query"].shape[1]), float("nan"),
                          dtype=torch.float32, device=dev)
    return g


def run_one_call(step, sharers, prefix, splits):
    import paged_attention_flat_amd as pa
    g = _inputs(step, sharers, prefix)
    pa.decode_step_cascade(g["key"], g["value"], g["k_pool"], g["v_pool"], g["slots"],
                           g["query"], g["qsl"], g["sl"], g["bt"], step.max_query_len,
                           step.max_seq_len, step.scale, g["sh"], g["pb"], num_splits=splits,
                           out=g["out"], lse=g["lse"])
    torch.cuda.synchronize()
    return g


def run_two_calls(step, sharers, prefix, splits):
    import paged_attention_flat_amd as pa
    g = _inputs(step, sharers, prefix)
    pa.kv_write(g["key"], g["value"], g["k_pool"], g["v_pool"], g["slots"])
    pa.attention_cascade(g["query"], g["k_pool"], g["v_pool"], g["qsl"], g["sl"], g["bt"],
                         step.max_query_len, step.max_seq_len, step.scale, g["sh"], g["pb"],
                         num_splits=splits, out=g["out"], lse=g["lse"])
    torch.cuda.synchronize()
    return g


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu()


def check_step(step, sharers, prefix, splits, what):
    a = run_one_call(step, sharers, prefix, splits)
    b = run_two_calls(step, sharers, prefix, splits)
    for n in ("k_pool", "v_pool", "out", "lse"):
        assert torch.equal(_bits(a[n]), _bits(b[n])), f"{what}: {n} differs from the two calls"
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value), raw_numpy(step.k_pool),
                             raw_numpy(step.v_pool), step.slot_mapping)
    assert np.array_equal(raw_numpy(a["k_pool"]).view(np.uint8),
                          np.ascontiguousarray(kp).view(np.uint8)), f"{what}: K pool"
    assert np.array_equal(raw_numpy(a["v_pool"]).view(np.uint8),
                          np.ascontiguousarray(vp).view(np.uint8)), f"{what}: V pool"
    ro, rl = oracle.attention(raw_numpy(step.query), kp, vp, step.query_start_loc,
                              step.seq_lens, step.block_tables, step.scale, step.num_kv_heads,
                              step.dtype)
    rows = np.arange(int(step.query_start_loc[-1]))
    o = a["out"].float().cpu().double().numpy()[rows]
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    assert float(np.abs(o - ro[rows]).max()) <= 2e-2, what
    assert float(np.linalg.norm(o - ro[rows]) / np.linalg.norm(ro[rows])) <= 2e-2, what
    assert float(np.abs(a["lse"].cpu().double().numpy()[rows] - rl[rows]).max()) <= 1e-3, what
    # rows past the last request are not written
    assert torch.isnan(a["out"][int(step.query_start_loc[-1]):]).all(), what
    return a


@pytest.mark.parametrize("splits", [1, 4])
def test_step_cascade_mixed_small(splits):
    step = config_step(5, scale_down=SMALL5)
    prefix = list(step.info["shared_blocks"])
    sharers = _sharers_of(step, prefix)
    assert len(sharers) >= 5
    check_step(step, sharers, prefix, splits, f"one-call cascade small config5 S={splits}")


def test_step_cascade_many_tokens():
    # a larger write beside the setup: 2 x 1100 chunk tokens + 40 decodes
    # (140 groups of 16 tokens x 8 KV heads)
    step = config_step(5, scale_down=dict(SMALL5, chunk=1100, stride=128))
    assert step.num_tokens >= 2200
    prefix = list(step.info["shared_blocks"])
    sharers = _sharers_of(step, prefix)
    check_step(step, sharers, prefix, 0, "one-call cascade, 2240 tokens")


def test_step_cascade_persistent_mixed():
    # decode rows certain: the stage, then one persistent launch; the trace
    # shows the write beside the setup and no other write kernel
    import paged_attention_flat_amd as pa
    step = config_step(5, scale_down=dict(SMALL5, decodes=80, sharers=20))
    assert step.num_seqs > step.num_tokens // 5 and step.max_query_len > 4
    prefix = list(step.info["shared_blocks"])
    sharers = _sharers_of(step, prefix)
    pa.trace_begin()
    run_one_call(step, sharers, prefix, 0)
    names = [n for n, _ in pa.trace_read()]
    pa.trace_end()
    assert names[0] == "cascade_write_setup", names
    assert "kv_write" not in names and "cascade_setup" not in names, names
    assert names.index("cascade_prefix") < names.index("mixed_prefill_decode"), names
    check_step(step, sharers, prefix, 0, "one-call cascade persistent config5")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (32, 4), (16, 2), (16, 16)])
def test_step_cascade_edge_cases(hq, hkv):
    # sharers with 1 and 2 new tokens, one whose context ends inside the
    # prefix (its token is written into a prefix block, before the stage
    # reads it), a prefill-row sharer; non-sharers; two padded tokens (one
    # with a slot in the pool, written as pa_kv_write does); KV-head counts
    # that are not a multiple of four
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
        own = max(need - P if share else need, 0)
        table = (prefix[:min(P, need)] if share else []) + perm[k:k + own]
        if share and need < P:
            table = prefix[:need]
        k += own
        reqs.append(Request(prior, n, table))
        if share:
            sharers.append(i)
    step = build_step("casc-step", reqs, dtype="bf16", num_q_heads=hq, num_kv_heads=hkv,
                      head_dim=128, num_blocks=nb, seed=int(rng.integers(1 << 30)), pad_tokens=2)
    # one padded token goes to a free slot of the pool
    step.slot_mapping[-1] = int(perm[k]) * 16 + 3
    for splits in (1, 3):
        check_step(step, sharers, prefix, splits, f"one-call cascade G={hq // hkv} S={splits}")


@pytest.mark.parametrize("splits", [0, 5])
def test_step_cascade_long_prefix(splits):
    # 16 decodes sharing a 2048-token prefix, private suffixes of 10..300 tokens
    step = shared_prefix_step(16, 2048, 10, 300, 7, num_q_heads=16, num_kv_heads=4)
    prefix = list(step.info["shared_blocks"])
    check_step(step, list(range(16)), prefix, splits, f"one-call long prefix S={splits}")


def test_step_cascade_without_sharers_is_decode_step():
    import paged_attention_flat_amd as pa
    step = shared_prefix_step(8, 512, 10, 100, 5, num_q_heads=16, num_kv_heads=4)
    a = run_one_call(step, [], [], 0)
    g = _inputs(step, [], [])
    pa.decode_step(g["key"], g["value"], g["k_pool"], g["v_pool"], g["slots"], g["query"],
                   g["qsl"], g["sl"], g["bt"], step.max_query_len, step.max_seq_len, step.scale,
                   out=g["out"], lse=g["lse"])
    torch.cuda.synchronize()
    for n in ("k_pool", "v_pool", "out", "lse"):
        assert torch.equal(_bits(a[n]), _bits(g[n])), n


def _check_sampled(step, out, lse, kc, vc, pick, what, sub=None):
    """Rows of the requests `pick` (or the rows `sub` of them) against the
    oracle on a compact copy of those requests, and their new tokens' cache
    entries against the inputs (the write is a bit copy)."""
    from workloads import extract_requests
    small, rows = extract_requests(step, pick)
    rows = np.asarray(rows)
    kp, vp = oracle.kv_write(raw_numpy(small.key), raw_numpy(small.value),
                             raw_numpy(small.k_pool), raw_numpy(small.v_pool), small.slot_mapping)
    idx = np.arange(len(rows)) if sub is None else np.asarray(sub)
    ro, rl = oracle.attention(raw_numpy(small.query), kp, vp, small.query_start_loc,
                              small.seq_lens, small.block_tables, small.scale,
                              small.num_kv_heads, small.dtype, rows=idx)
    ro, rl = ro[idx], rl[idx]
    o = out.float().cpu().double().numpy()[rows[idx]]
    assert np.isfinite(o).all(), what
    assert float(np.abs(o - ro).max()) <= 2e-2, what
    assert float(np.linalg.norm(o - ro) / np.linalg.norm(ro)) <= 2e-2, what
    assert float(np.abs(lse.cpu().double().numpy()[rows[idx]] - rl).max()) <= 1e-3, what
    kin = raw_numpy(step.key).view(np.uint16)
    vin = raw_numpy(step.value).view(np.uint16)
    for t in rows:
        s = int(step.slot_mapping[t])
        blk, off = s // 16, s % 16
        kk = kc[blk, :, off, :].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        vv = vc[blk, :, :, off].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(kk, kin[t]), f"{what}: K entry of token {t}"
        assert np.array_equal(vv, vin[t]), f"{what}: V entry of token {t}"


def test_step_cascade_full_mixed_step_sampled():
    # the full mixed chunked-prefill step (4096 decodes, 1024 sharers of a
    # 64-block prefix, two 2048-token chunks) through the one call, as timed
    # (drawn on the device; the pools are written in place)
    step = config_step(5, device="cuda")
    prefix = list(step.info["shared_blocks"])
    sharers = _sharers_of(step, prefix)
    assert len(sharers) == step.info["num_sharers"]
    g = run_one_call(step, sharers, prefix, 0)
    rng = np.random.default_rng(5)
    ql = np.diff(step.query_start_loc)
    non = [b for b in range(step.num_seqs) if b not in set(sharers) and ql[b] == 1]
    chunks = [b for b in range(step.num_seqs) if ql[b] > 1]
    pick = list(rng.choice(sharers, 4, replace=False)) + list(rng.choice(non, 2, replace=False))
    _check_sampled(step, g["out"], g["lse"], g["k_pool"], g["v_pool"], pick,
                   "one-call cascade, full mixed step (decode rows)")
    # 24 seeded rows of each prefill chunk (2048 rows over a 4096- and a
    # 16384-token prior context); every chunk token's cache entries
    for c in chunks:
        sub = sorted(int(x) for x in rng.choice(int(ql[c]), 24, replace=False))
        _check_sampled(step, g["out"], g["lse"], g["k_pool"], g["v_pool"], [c],
                       f"one-call cascade, full mixed step (chunk {c})", sub=sub)


def test_step_cascade_full_shared_prefix_sampled():
    # 256 decodes sharing a 16384-token prefix, 0..512 private tokens, as timed
    step = shared_prefix_step(256, 16384, 0, 512, 11, fill="nan")
    prefix = list(step.info["shared_blocks"])
    g = run_one_call(step, list(range(step.num_seqs)), prefix, 0)
    rng = np.random.default_rng(11)
    pick = [int(x) for x in rng.choice(step.num_seqs, 5, replace=False)]
    _check_sampled(step, g["out"], g["lse"], g["k_pool"], g["v_pool"], pick,
                   "one-call cascade, 256 x 16384 shared prefix")
