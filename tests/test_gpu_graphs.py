"""GPU: decode steps replayed from HIP graphs at the capture ladder's padded
sizes ("Model execution", section "Code"), against the fp64 oracle.

Every step is checked element by element (bars as in test_gpu_parity: bf16
output 2e-2, lse 1e-3) and the pool bit for bit after the write: padded tokens
(slot -1) must write nothing.  Graphs are replayed several times with new data
and with eager work in between, and every replay is checked.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import Request, build_step, raw_numpy

pytestmark = pytest.mark.gpu

TOL_OUT = 2e-2
TOL_LSE = 1e-3
HQ, HKV, D = 8, 2, 128
STRIDE = 24          # table capacity: 384 tokens
NB = 6400            # shared pool size of every step


def make_step(n, seed):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(NB)
    reqs, k = [], 0
    for _ in range(n):
        prior = int(rng.integers(0, STRIDE * 16 - 1))
        need = -(-(prior + 1) // 16)
        reqs.append(Request(prior, 1, list(perm[k:k + need])))
        k += need
    assert k <= NB
    return build_step(f"decode{n}", reqs, dtype="bf16", num_q_heads=HQ, num_kv_heads=HKV,
                      head_dim=D, num_blocks=NB, seed=seed, stride=STRIDE)


def check_step(step, out, lse, kc, vc, what):
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value),
                             raw_numpy(step.k_pool), raw_numpy(step.v_pool), step.slot_mapping)
    ro, rl = oracle.attention(raw_numpy(step.query), kp, vp, step.query_start_loc,
                              step.seq_lens, step.block_tables, step.scale, HKV, "bf16")
    o = out.float().cpu().double().numpy()
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = float(np.abs(o - ro).max())
    assert err <= TOL_OUT, f"{what}: max |out - oracle| = {err}"
    le = float(np.abs(lse.cpu().double().numpy() - rl).max())
    assert le <= TOL_LSE, f"{what}: max |lse - oracle| = {le}"
    # the pool after the write: bit-exact, nothing written for padded tokens
    for got, ref in ((kc, kp), (vc, vp)):
        g = np.ascontiguousarray(got.view(torch.int16).cpu().numpy()).view(np.uint8)
        r = np.ascontiguousarray(ref).view(np.uint8)
        assert g.shape == r.shape and np.array_equal(g, r), \
            f"{what}: pool differs from the oracle's write"


def test_decode_graphs_padded_replays():
    import paged_attention_flat_amd as pa
    from paged_attention_flat_amd.graphs import DecodeGraphs
    dev = torch.device("cuda:0")
    kc = torch.empty(NB, HKV, 16, D, dtype=torch.bfloat16, device=dev)
    vc = torch.empty(NB, HKV, D, 16, dtype=torch.bfloat16, device=dev)
    dg = DecodeGraphs(kc, vc, HQ, STRIDE, 1.0 / D ** 0.5, max_size=512)
    # sizes from the printed padding table, one repeated size with new data,
    # and one past the top size (runs without a graph)
    plan = [(1, 1), (3, 2), (5, 3), (13, 4), (16, 5), (13, 6), (100, 7), (257, 8)]
    for n, seed in plan:
        step = make_step(n, 1000 + seed)
        kc.copy_(step.k_pool.to(dev))
        vc.copy_(step.v_pool.to(dev))
        g = [t.to(dev) for t in (step.query, step.key, step.value)]
        sm = torch.as_tensor(step.slot_mapping).to(dev)
        sl = torch.as_tensor(step.seq_lens).to(dev)
        bt = torch.as_tensor(step.block_tables).to(dev)
        # eager work between replays on the same stream
        scratch = torch.randn(1 << 20, device=dev)
        scratch.mul_(2.0).sum().item()
        out, lse = dg.step(g[0], g[1], g[2], sm, sl, bt)
        torch.cuda.synchronize()
        print(f"step n={n} padded to {pa.capture_size(n)}", flush=True)
        check_step(step, out, lse, kc, vc, f"n={n} (graph size {pa.capture_size(n)})")
    # 4, 8, 16, 104, 272 (and 1) were captured once each
    assert sorted(dg.graphs) == [1, 4, 8, 16, 104, 272]


def test_decode_graphs_past_the_top_size_run_eagerly():
    from paged_attention_flat_amd.graphs import DecodeGraphs
    dev = torch.device("cuda:0")
    kc = torch.empty(NB, HKV, 16, D, dtype=torch.bfloat16, device=dev)
    vc = torch.empty(NB, HKV, D, 16, dtype=torch.bfloat16, device=dev)
    dg = DecodeGraphs(kc, vc, HQ, STRIDE, 1.0 / D ** 0.5, max_size=16)
    step = make_step(20, 77)
    kc.copy_(step.k_pool.to(dev))
    vc.copy_(step.v_pool.to(dev))
    out, lse = dg.step(step.query.to(dev), step.key.to(dev), step.value.to(dev),
                       torch.as_tensor(step.slot_mapping).to(dev),
                       torch.as_tensor(step.seq_lens).to(dev),
                       torch.as_tensor(step.block_tables).to(dev))
    torch.cuda.synchronize()
    check_step(step, out, lse, kc, vc, "n=20 eager")
    assert dg.graphs == {}


def test_mixed_step_graph_replays_match_eager():
    # a mixed step (prefill chunks + decodes) in one call: the work-list
    # write, the plan and order kernels and the attention launch (persistent
    # prefill + decode units when decode rows are certain, else the separate
    # kernels), with work counters reset inside the step.  Captured once,
    # replayed three times with the pools reset by eager copies in between;
    # every replay must give the eager call's bytes (pools, out, lse), and
    # the eager call the oracle's.
    import paged_attention_flat_amd as pa
    from workloads import config_step
    step = config_step(5, scale_down={"chunk": 90, "priors": (70, 300), "decodes": 80,
                                      "lo": 20, "hi": 900, "prefix": 64, "sharers": 10,
                                      "stride": 64})
    assert step.num_seqs > step.num_tokens // 5       # the persistent launch is taken
    dev = torch.device("cuda:0")
    g = {n: getattr(step, n).to(dev).contiguous() for n in ("query", "key", "value")}
    k0, v0 = step.k_pool.to(dev), step.v_pool.to(dev)
    kc, vc = k0.clone(), v0.clone()
    meta = [torch.as_tensor(x).to(dev) for x in (step.slot_mapping, step.query_start_loc,
                                                   step.seq_lens, step.block_tables)]
    out = torch.empty_like(g["query"])
    lse = torch.empty(step.num_tokens, step.num_q_heads, dtype=torch.float32, device=dev)
    ws = pa.workspace(step.num_seqs, step.num_tokens, step.num_q_heads, step.head_dim, 1,
                      device=dev)

    def call():
        pa.decode_step(g["key"], g["value"], kc, vc, meta[0], g["query"], meta[1], meta[2],
                       meta[3], step.max_query_len, step.max_seq_len, step.scale,
                       num_splits=1, out=out, lse=lse, workspace=ws)

    call()
    torch.cuda.synchronize()
    n = int(step.query_start_loc[-1])
    ref = [t.clone() for t in (out[:n], lse[:n], kc, vc)]
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value), raw_numpy(step.k_pool),
                             raw_numpy(step.v_pool), step.slot_mapping)
    for got, r in ((kc, kp), (vc, vp)):
        assert np.array_equal(np.ascontiguousarray(got.view(torch.int16).cpu().numpy()).view(np.uint8),
                              np.ascontiguousarray(r).view(np.uint8))
    ro, rl = oracle.attention(raw_numpy(step.query), kp, vp, step.query_start_loc,
                              step.seq_lens, step.block_tables, step.scale, step.num_kv_heads,
                              "bf16")
    assert float(np.abs(out[:n].float().cpu().double().numpy() - ro[:n]).max()) <= TOL_OUT
    assert float(np.abs(lse[:n].cpu().double().numpy() - rl[:n]).max()) <= TOL_LSE
    kc.copy_(k0)
    vc.copy_(v0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(3):
        kc.copy_(k0)
        vc.copy_(v0)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.randn(1 << 20, device=dev).mul_(2.0).sum().item()   # eager work between
        graph.replay()
        torch.cuda.synchronize()
        for a, b, what in zip((out[:n], lse[:n], kc, vc), ref, ("out", "lse", "K", "V")):
            ab = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
            bb = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
            assert torch.equal(ab, bb), f"replay {rep}: {what} differs from the eager call"
