"""GPU check of pa_decode_step_noalloc (the step with the library's own
per-GPU workspace) against pa_decode_step with a caller workspace, on the
same inputs, through the C ABI: pools byte-identical, out and lse
bit-identical (same kernels, same split count; the library is deterministic),
and both within the oracle bars (2e-2 / 1e-3).  Several calls in a row share
the one device array, each smaller than the one before, so a call that relied
on what an earlier one left behind (other than the zeroed arrival counters)
would show here.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import config_step, raw_numpy

pytestmark = pytest.mark.gpu

SMALL = {
    2: {"context": 8000, "pool_blocks": 1200},
    3: {"batch": 12, "lo": 40, "hi": 700},
    5: {"chunk": 90, "priors": (70, 300), "decodes": 40, "lo": 20, "hi": 900,
        "prefix": 64, "sharers": 10, "stride": 64},
}


def upload(step):
    g = {n: getattr(step, n).to("cuda").contiguous()
         for n in ("query", "key", "value", "k_pool", "v_pool")}
    g["qsl"] = torch.as_tensor(step.query_start_loc).to("cuda")
    g["sl"] = torch.as_tensor(step.seq_lens).to("cuda")
    g["bt"] = torch.as_tensor(step.block_tables).to("cuda")
    g["sm"] = torch.as_tensor(step.slot_mapping).to("cuda")
    return g


def both(step, splits=0):
    import paged_attention_flat_amd as pa
    res = []
    for fn in ("decode_step", "decode_step_noalloc"):
        g = upload(step)
        out = torch.full_like(g["query"], float("nan"))
        lse = torch.full((step.num_tokens, step.num_q_heads), float("nan"),
                         dtype=torch.float32, device="cuda")
        args = (g["key"], g["value"], g["k_pool"], g["v_pool"], g["sm"], g["query"], g["qsl"],
                g["sl"], g["bt"], step.max_query_len, step.max_seq_len, step.scale)
        if fn == "decode_step":
            pa.decode_step(*args, num_splits=splits, out=out, lse=lse)
        else:
            pa.decode_step_noalloc(*args, out=out, lse=lse, num_splits=splits)
        torch.cuda.synchronize()
        res.append((out, lse, g))
    return res


def bytes_of(t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.numpy().view(np.uint8)


def check(step, res, what):
    (o0, l0, g0), (o1, l1, g1) = res
    for name in ("k_pool", "v_pool"):
        assert np.array_equal(bytes_of(g0[name]), bytes_of(g1[name])), f"{what}: {name}"
    n = int(step.query_start_loc[-1])
    assert np.array_equal(bytes_of(o0[:n]), bytes_of(o1[:n])), f"{what}: out"
    assert np.array_equal(bytes_of(l0[:n]), bytes_of(l1[:n])), f"{what}: lse"
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value), raw_numpy(step.k_pool),
                             raw_numpy(step.v_pool), step.slot_mapping)
    assert np.array_equal(bytes_of(g1["k_pool"]), np.ascontiguousarray(kp).view(np.uint8))
    assert np.array_equal(bytes_of(g1["v_pool"]), np.ascontiguousarray(vp).view(np.uint8))
    ro, rl = oracle.attention(raw_numpy(step.query), kp, vp, step.query_start_loc,
                              step.seq_lens, step.block_tables, step.scale, step.num_kv_heads,
                              step.dtype)
    o = o1.float().cpu().double().numpy()[:n]
    assert np.isfinite(o).all(), what
    assert float(np.abs(o - ro[:n]).max()) <= 2e-2, what
    assert float(np.abs(l1.cpu().double().numpy()[:n] - rl[:n]).max()) <= 1e-3, what


def test_noalloc_matches_decode_step_on_successive_smaller_steps():
    # a mixed step (prefill rows: write + matrix-core kernel + decode), then a
    # 12-request decode (3 splits), then a single long decode (32 splits) and
    # a single shorter one: each call smaller than the one before it
    steps = [(config_step(5, scale_down=SMALL[5]), 0),
             (config_step(3, scale_down=SMALL[3]), 0),
             (config_step(2, scale_down=SMALL[2]), 0),
             (config_step(2, scale_down={"context": 3000, "pool_blocks": 400}), 7)]
    sizes = [st.num_tokens for st, _ in steps]
    assert sizes == sorted(sizes, reverse=True)
    for i, (st, splits) in enumerate(steps):
        check(st, both(st, splits), f"call {i} ({st.name}, S={splits})")


def test_noalloc_rejects_a_step_beyond_its_array():
    import paged_attention_flat_amd as pa
    from paged_attention_flat_amd import _lib
    st = config_step(2, scale_down=SMALL[2])
    # 256 forced splits x 4 tokens x 32 heads x 128 dims of fp32 partials
    # exceed the array: refused before anything is enqueued
    need = _lib.LIB.pa_attention_workspace_size(1, 4, 32, 128, 256)
    assert need > _lib.PA_NOALLOC_SCRATCH_BYTES
    g = upload(st)
    q4 = g["query"].repeat(4, 1, 1)
    k4, v4 = g["key"].repeat(4, 1, 1), g["value"].repeat(4, 1, 1)
    sm4 = torch.full((4,), -1, dtype=torch.int64, device="cuda")
    out = torch.empty_like(q4)
    with pytest.raises(pa.PaError) as e:
        pa.decode_step_noalloc(k4, v4, g["k_pool"], g["v_pool"], sm4, q4, g["qsl"], g["sl"],
                               g["bt"], st.max_query_len, st.max_seq_len, st.scale, out=out,
                               num_splits=256)
    assert e.value.status == _lib.PA_ERR_WORKSPACE
