"""Host-side metadata validator of the package (pa.validate_step): valid
steps of every workload pass, and each planted mistake is reported.  Where
the oracle's own validator checks the same rule, both must agree."""

import numpy as np
import pytest

import oracle
import paged_attention_flat_amd as pa
from workloads import Request, build_step, config_step, shared_prefix_step

SMALL = {
    2: {"context": 1000, "pool_blocks": 200},
    3: {"batch": 12, "lo": 40, "hi": 700},
    4: {"batch": 2, "new": 300, "pool_blocks": 48},
    5: {"chunk": 90, "priors": (70, 300), "decodes": 40, "lo": 20, "hi": 900,
        "prefix": 64, "sharers": 10, "stride": 64},
}


def meta(step):
    return dict(query_start_loc=step.query_start_loc.copy(), seq_lens=step.seq_lens.copy(),
                block_tables=step.block_tables.copy(), slot_mapping=step.slot_mapping.copy(),
                num_blocks=step.num_blocks)


def oracle_ok(m):
    try:
        oracle.validate_step(m["query_start_loc"], m["seq_lens"], m["block_tables"],
                             m["slot_mapping"], m["slot_mapping"].shape[0], m["num_blocks"])
        return True
    except AssertionError:
        return False


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_valid_workloads_pass(cfg):
    step = config_step(cfg, scale_down=SMALL.get(cfg), with_values=False)
    m = meta(step)
    assert pa.step_problems(**m, max_query_len=step.max_query_len,
                            max_seq_len=step.max_seq_len) == []
    pa.validate_step(**m)
    assert oracle_ok(m)


def test_valid_shared_prefix_and_padding_pass():
    step = shared_prefix_step(6, 64, 0, 20, 3, with_values=False)
    assert pa.step_problems(**meta(step)) == []
    # requests without new tokens and padded tokens (slot -1) after the last row
    shapes = [(40, 1), (17, 0), (3, 2)]
    need = [-(-(p + n) // 16) for p, n in shapes]
    tables, k = [], 0
    for n in need:
        tables.append(list(range(k, k + n)))
        k += n
    step = build_step("pad", [Request(p, n, t) for (p, n), t in zip(shapes, tables)],
                      dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=64, num_blocks=k + 2,
                      seed=1, pad_tokens=3, with_values=False)
    assert pa.step_problems(**meta(step)) == []


def test_torch_tensors_accepted():
    torch = pytest.importorskip("torch")
    step = config_step(2, scale_down=SMALL[2], with_values=False)
    m = meta(step)
    for k in ("query_start_loc", "seq_lens", "block_tables", "slot_mapping"):
        m[k] = torch.as_tensor(m[k])
    assert pa.step_problems(**m) == []


def mutate(name):
    """A valid mixed step with one planted mistake; returns (metadata, what
    the report must mention, whether the oracle's validator checks it)."""
    step = config_step(5, scale_down=SMALL[5], with_values=False)
    m = meta(step)
    qsl, sl, bt, sm = m["query_start_loc"], m["seq_lens"], m["block_tables"], m["slot_mapping"]
    q_len = np.diff(qsl)
    d = int(np.nonzero(q_len == 1)[0][0])    # a decode request
    p = int(np.nonzero(q_len > 1)[0][0])     # a prefill chunk
    if name == "qsl0":
        qsl[0] = 1
        return m, "query_start_loc[0]", True
    if name == "qsl_down":
        qsl[p + 1] = qsl[p] - 1
        return m, "decreases", True
    if name == "qsl_end":
        m["slot_mapping"] = sm[: int(qsl[-1]) - 1]
        return m, "exceeds", True
    if name == "seq_short":
        sl[p] = q_len[p] - 1
        return m, "seq_len", True
    if name == "table_narrow":
        m["block_tables"] = bt[:, : max(1, int(-(-sl.max() // 16)) - 1)]
        return m, "columns", True
    if name == "block_range":
        bt[d, 0] = m["num_blocks"]
        return m, "outside [0,", True
    if name == "slot_rule":
        t = int(qsl[p]) + 3
        sm[t] = sm[t] + 1 if (sm[t] + 1) % 16 else sm[t] - 1
        return m, "the block table gives", True
    if name == "slot_dup":
        m["slot_mapping"] = np.concatenate([sm, sm[int(qsl[d]):int(qsl[d]) + 1]])
        return m, "more than one token", True
    if name == "written_shared":
        # another request's table reads the block of the decode token's slot
        e = int(np.nonzero((q_len == 1) & (np.arange(len(q_len)) != d))[0][0])
        bt[e, 0] = sm[int(qsl[d])] // 16
        return m, "also read by request", False
    raise ValueError(name)


@pytest.mark.parametrize("name", ["qsl0", "qsl_down", "qsl_end", "seq_short", "table_narrow",
                                  "block_range", "slot_rule", "slot_dup", "written_shared"])
def test_planted_mistakes_reported(name):
    m, needle, oracle_checks = mutate(name)
    probs = pa.step_problems(**m)
    assert probs and any(needle in x for x in probs), probs
    with pytest.raises(ValueError):
        pa.validate_step(**m)
    if oracle_checks:
        assert not oracle_ok(m)


def test_host_bounds():
    step = config_step(4, scale_down=SMALL[4], with_values=False)
    m = meta(step)
    assert any("max_query_len" in x
               for x in pa.step_problems(**m, max_query_len=step.max_query_len - 1))
    assert any("max_seq_len" in x
               for x in pa.step_problems(**m, max_seq_len=step.max_seq_len - 1))
