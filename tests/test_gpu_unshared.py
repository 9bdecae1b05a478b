"""The decode rows' cache-read policy (pa_set_unshared_blocks: -1 every
request shared, 0 automatic from the requests' first blocks, 1 every request
unshared) changes only how V is loaded: every output, lse and pool byte must
be the same under the three modes, on the many-work-group decode shape (bf16
and E4M3 caches), on a mixed step whose sharers of a prefix and private
requests take different policies in one persistent launch, and through the
one-call step; and the results must match the fp64 oracle at the usual bars
(output 2e-2, lse 1e-3)."""

import numpy as np
import pytest
import torch

import oracle
from workloads import config_step, raw_numpy

pytestmark = pytest.mark.gpu


MODES = (-1, 0, 1)


def same(a, b):
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)


def run_step(step, hint, fused):
    import paged_attention_flat_amd as pa
    dev = "cuda"
    g = {n: getattr(step, n).to(dev).contiguous() for n in ("query", "key", "value",
                                                              "k_pool", "v_pool")}
    qsl = torch.as_tensor(step.query_start_loc).to(dev)
    sl = torch.as_tensor(step.seq_lens).to(dev)
    bt = torch.as_tensor(step.block_tables).to(dev)
    sm = torch.as_tensor(step.slot_mapping).to(dev)
    prev = pa.set_unshared_blocks(hint)
    try:
        if fused:
            out, lse = pa.decode_step(g["key"], g["value"], g["k_pool"], g["v_pool"], sm,
                                      g["query"], qsl, sl, bt, step.max_query_len,
                                      step.max_seq_len, step.scale)
        else:
            pa.kv_write(g["key"], g["value"], g["k_pool"], g["v_pool"], sm)
            out, lse = pa.attention(g["query"], g["k_pool"], g["v_pool"], qsl, sl, bt,
                                    step.max_query_len, step.max_seq_len, step.scale)
        torch.cuda.synchronize()
    finally:
        pa.set_unshared_blocks(prev)
    n = int(step.query_start_loc[-1])
    return out[:n].cpu(), lse[:n].cpu(), g["k_pool"].cpu(), g["v_pool"].cpu()


def check_oracle(step, out, lse):
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value), raw_numpy(step.k_pool),
                             raw_numpy(step.v_pool), step.slot_mapping)
    ro, rl = oracle.attention(raw_numpy(step.query), kp, vp, step.query_start_loc,
                              step.seq_lens, step.block_tables, step.scale, step.num_kv_heads,
                              step.dtype)
    n = out.shape[0]
    o = out.float().double().numpy()
    assert np.isfinite(o).all()
    assert float(np.abs(o - ro[:n]).max()) <= 2e-2
    assert float(np.linalg.norm(o - ro[:n]) / np.linalg.norm(ro[:n])) <= 2e-2
    assert float(np.abs(lse.double().numpy() - rl[:n]).max()) <= 1e-3


@pytest.mark.parametrize("fused", [False, True])
def test_many_unit_decode_same_under_every_mode(fused):
    # 96 decodes x 8 KV heads = 768 work units: the many-work-group shape
    step = config_step(3, scale_down={"batch": 96, "lo": 200, "hi": 1200})
    runs = [run_step(step, m, fused) for m in MODES]
    for r in runs[1:]:
        same(runs[0], r)
    check_oracle(step, runs[1][0], runs[1][1])


@pytest.mark.parametrize("fused", [False, True])
def test_mixed_step_same_under_every_mode(fused):
    # two prefill chunks and 120 decodes: the persistent mixed launch
    step = config_step(5, scale_down={"chunk": 90, "priors": (70, 300), "decodes": 120,
                                      "lo": 20, "hi": 900, "prefix": 64, "sharers": 30,
                                      "stride": 64})
    assert step.num_seqs > step.num_tokens // 5
    runs = [run_step(step, m, fused) for m in MODES]
    for r in runs[1:]:
        same(runs[0], r)
    check_oracle(step, runs[1][0], runs[1][1])


def run_step_fp8(step, hint):
    import paged_attention_flat_amd as pa
    dev = "cuda"
    g = {n: getattr(step, n).to(dev).contiguous()
         for n in ("query", "key", "value", "k_pool", "v_pool", "k_scale", "v_scale")}
    qsl = torch.as_tensor(step.query_start_loc).to(dev)
    sl = torch.as_tensor(step.seq_lens).to(dev)
    bt = torch.as_tensor(step.block_tables).to(dev)
    sm = torch.as_tensor(step.slot_mapping).to(dev)
    prev = pa.set_unshared_blocks(hint)
    try:
        out, lse = pa.decode_step_fp8(g["key"], g["value"], g["k_pool"], g["v_pool"], sm,
                                      g["k_scale"], g["v_scale"], g["query"], qsl, sl, bt,
                                      step.max_query_len, step.max_seq_len, step.scale)
        torch.cuda.synchronize()
    finally:
        pa.set_unshared_blocks(prev)
    n = int(step.query_start_loc[-1])
    return out[:n].cpu(), lse[:n].cpu(), g["k_pool"].cpu(), g["v_pool"].cpu()


def test_many_unit_decode_fp8_same_under_every_mode():
    # E4M3 cache: the V codes streamed non-temporally give the same bytes
    from workloads import fp8_cache
    step = fp8_cache(config_step(3, scale_down={"batch": 96, "lo": 200, "hi": 1200}), 3)
    runs = [run_step_fp8(step, m) for m in MODES]
    for r in runs[1:]:
        same(runs[0], r)
    b = runs[1]
    kp, vp = oracle.kv_write_fp8(raw_numpy(step.key), raw_numpy(step.value),
                                 raw_numpy(step.k_pool), raw_numpy(step.v_pool),
                                 step.slot_mapping, step.k_scale.cpu().numpy(),
                                 step.v_scale.cpu().numpy(), step.dtype)
    ro, rl = oracle.attention_fp8(raw_numpy(step.query), kp, vp, step.k_scale.cpu().numpy(),
                                  step.v_scale.cpu().numpy(), step.query_start_loc,
                                  step.seq_lens, step.block_tables, step.scale,
                                  step.num_kv_heads, query_dtype=step.dtype)
    n = b[0].shape[0]
    o = b[0].float().double().numpy()
    assert float(np.abs(o - ro[:n]).max()) <= 2e-2
    assert float(np.abs(b[1].double().numpy() - rl[:n]).max()) <= 1e-3
