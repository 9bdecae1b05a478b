"""GPU parity: the HIP library, called through its C ABI, against the fp64
CPU oracle on identical seeded inputs.

Bars (written here, used by every comparison):
* KV write: bit-exact pools (every byte, poisoned slots included);
* attention output: max |gpu - oracle| <= 2e-2 (bf16) or 1e-4 (fp32), and
  the relative Frobenius error of the rows checked <= 2e-2 (bf16) or 1e-4;
* log-sum-exp: max |gpu - oracle| <= 1e-3.
Every pool is NaN-poisoned outside the prior context (tail slots, unreferenced
blocks, and the new tokens' slots before the write), so a value that must
not be read shows up as a NaN in the output.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from workloads import Request, build_step, config_step, extract_requests, raw_numpy

pytestmark = pytest.mark.gpu

TOL_OUT = {"bf16": 2e-2, "f32": 1e-4}
TOL_LSE = 1e-3
# supplementary: relative Frobenius error of the output rows.  bf16 rounding
# of P and of the output gives ~1e-3 (fp32: ~1e-6); a zeroed or mis-scaled
# output, which can pass the absolute bar when a long context averages the
# output toward 0, gives ~1.
TOL_REL = {"bf16": 2e-2, "f32": 1e-4}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    import paged_attention_flat_amd as pa  # noqa: F401  (fails loudly without libpa.so)
    return torch.device("cuda:0")


def pa_mod():
    import paged_attention_flat_amd as pa
    return pa


def upload(step, dev="cuda"):
    g = {}
    for name in ("query", "key", "value", "k_pool", "v_pool"):
        g[name] = getattr(step, name).to(dev).contiguous()
    g["qsl"] = torch.as_tensor(step.query_start_loc).to(dev)
    g["seq_lens"] = torch.as_tensor(step.seq_lens).to(dev)
    g["tables"] = torch.as_tensor(step.block_tables).to(dev)
    g["slots"] = torch.as_tensor(step.slot_mapping).to(dev)
    return g


def run_gpu(step, num_splits=0, g=None, lse=True):
    pa = pa_mod()
    g = g or upload(step)
    pa.kv_write(g["key"], g["value"], g["k_pool"], g["v_pool"], g["slots"])
    out = torch.full_like(g["query"], float("nan"))
    out, l = pa.attention(g["query"], g["k_pool"], g["v_pool"], g["qsl"], g["seq_lens"],
                          g["tables"], step.max_query_len, step.max_seq_len, step.scale,
                          num_splits=num_splits, out=out, want_lse=lse)
    torch.cuda.synchronize()
    return out, l, g


def run_oracle(step, rows=None):
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value),
                             raw_numpy(step.k_pool), raw_numpy(step.v_pool), step.slot_mapping)
    return oracle.attention(raw_numpy(step.query), kp, vp, step.query_start_loc,
                            step.seq_lens, step.block_tables, step.scale, step.num_kv_heads,
                            step.dtype, rows=rows), (kp, vp)


def to64(t):
    return t.detach().float().cpu().double().numpy()


def check(step, out, lse, ref_out, ref_lse, rows=None, what=""):
    o = to64(out)
    rows = np.arange(int(step.query_start_loc[-1])) if rows is None else np.asarray(rows)
    diff = np.abs(o[rows] - ref_out[rows])
    assert np.isfinite(o[rows]).all(), f"{what}: non-finite output"
    err = float(diff.max()) if diff.size else 0.0
    assert err <= TOL_OUT[step.dtype], f"{what}: max |out - oracle| = {err}"
    if diff.size:
        ref_norm = np.linalg.norm(ref_out[rows])
        rel = float(np.linalg.norm(o[rows] - ref_out[rows]) / max(ref_norm, 1e-30))
        assert rel <= TOL_REL[step.dtype], f"{what}: |out - oracle| / |oracle| = {rel}"
    if lse is not None:
        le = float(np.abs(lse.cpu().double().numpy()[rows] - ref_lse[rows]).max())
        assert le <= TOL_LSE, f"{what}: max |lse - oracle| = {le}"
    return err


def _bytes(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().contiguous()
        if x.dtype == torch.bfloat16:
            x = x.view(torch.int16)
        x = x.numpy()
    return np.ascontiguousarray(x).view(np.uint8)


def same_bits(a, b) -> bool:
    """Byte-for-byte equality (NaN payloads included)."""
    return np.shape(a) == np.shape(b) and np.array_equal(_bytes(a), _bytes(b))


# ----------------------------------------------------------------------------
# KV write
# ----------------------------------------------------------------------------

SMALL = {
    2: {"context": 1000, "pool_blocks": 200},
    3: {"batch": 12, "lo": 40, "hi": 700},
    4: {"batch": 2, "new": 300, "pool_blocks": 48},
    5: {"chunk": 90, "priors": (70, 300), "decodes": 40, "lo": 20, "hi": 900,
        "prefix": 64, "sharers": 10, "stride": 64},
}


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_kv_write_bit_exact(cfg):
    step = config_step(cfg, scale_down=SMALL.get(cfg))
    pa = pa_mod()
    g = upload(step)
    pa.kv_write(g["key"], g["value"], g["k_pool"], g["v_pool"], g["slots"])
    torch.cuda.synchronize()
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value), raw_numpy(step.k_pool),
                             raw_numpy(step.v_pool), step.slot_mapping)
    assert same_bits(g["k_pool"], kp)
    assert same_bits(g["v_pool"], vp)


def test_kv_write_skips_padded_tokens():
    reqs = [Request(3, 20, [5, 1]), Request(0, 1, [2])]
    step = build_step("pad", reqs, dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128,
                      num_blocks=8, seed=41, pad_tokens=5)
    assert (step.slot_mapping[-5:] < 0).all()
    pa = pa_mod()
    g = upload(step)
    pa.kv_write(g["key"], g["value"], g["k_pool"], g["v_pool"], g["slots"])
    torch.cuda.synchronize()
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value), raw_numpy(step.k_pool),
                             raw_numpy(step.v_pool), step.slot_mapping)
    assert same_bits(g["k_pool"], kp)
    assert same_bits(g["v_pool"], vp)


def test_kv_write_drops_slots_past_the_pool():
    # a slot at or past num_blocks * 16 is dropped like a padded token
    reqs = [Request(3, 20, [5, 1]), Request(0, 1, [2])]
    step = build_step("oob", reqs, dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128,
                      num_blocks=8, seed=43, pad_tokens=4)
    bad = step.slot_mapping.copy()
    bad[-4:] = [8 * 16, 8 * 16 + 5, 1 << 40, 8 * 16 + 15]
    pa = pa_mod()
    g = upload(step)
    g["slots"] = torch.as_tensor(bad).to("cuda")
    pa.kv_write(g["key"], g["value"], g["k_pool"], g["v_pool"], g["slots"])
    torch.cuda.synchronize()
    kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value), raw_numpy(step.k_pool),
                             raw_numpy(step.v_pool), step.slot_mapping)
    assert same_bits(g["k_pool"], kp)
    assert same_bits(g["v_pool"], vp)


def test_kv_write_f32_head_dim_128_and_bf16_64():
    for dtype, d in (("f32", 128), ("bf16", 64)):
        reqs = [Request(0, 37, [3, 0, 6]), Request(9, 2, [1])]
        step = build_step("kvw", reqs, dtype=dtype, num_q_heads=4, num_kv_heads=4, head_dim=d,
                          num_blocks=8, seed=42)
        pa = pa_mod()
        g = upload(step)
        pa.kv_write(g["key"], g["value"], g["k_pool"], g["v_pool"], g["slots"])
        torch.cuda.synchronize()
        kp, vp = oracle.kv_write(raw_numpy(step.key), raw_numpy(step.value),
                                 raw_numpy(step.k_pool), raw_numpy(step.v_pool),
                                 step.slot_mapping)
        assert same_bits(g["k_pool"], kp)
        assert same_bits(g["v_pool"], vp)


# ----------------------------------------------------------------------------
# attention parity on the five workloads (small sizes: every row checked)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("variant", [None, "alt"])
@pytest.mark.parametrize("splits", [1, 3])
def test_config1_fp32(variant, splits):
    step = config_step(1, variant=variant)
    out, lse, g = run_gpu(step, num_splits=splits)
    (ro, rl), _ = run_oracle(step)
    check(step, out, lse, ro, rl, what=f"config1 {variant} S={splits}")


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_small_configs_bf16(cfg):
    step = config_step(cfg, scale_down=SMALL[cfg])
    out, lse, _ = run_gpu(step)
    (ro, rl), _ = run_oracle(step)
    check(step, out, lse, ro, rl, what=f"config{cfg} small")


@pytest.mark.parametrize("splits", [1, 2, 7, 64, 128, 256])
def test_split_sweep_small_decode(splits):
    step = config_step(2, scale_down=SMALL[2])
    out, lse, _ = run_gpu(step, num_splits=splits)
    (ro, rl), _ = run_oracle(step)
    check(step, out, lse, ro, rl, what=f"config2 small S={splits}")


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (16, 4), (32, 4), (16, 1), (4, 1)])
def test_head_dims_and_groups(dtype, d, hq, hkv):
    # a prefill chunk with prior context, a decode, a 2-token and a 3-token
    # request, a fresh prefill, and an empty request
    rng = np.random.default_rng(hq * 100 + d + (dtype == "f32"))
    shapes = [(45, 70), (130, 1), (17, 2), (60, 3), (0, 33), (12, 0)]
    need = [-(-(p + n) // 16) for p, n in shapes]
    nb = sum(need) + 5
    perm = rng.permutation(nb)
    tables, k = [], 0
    for n in need:
        tables.append(list(perm[k:k + n]))
        k += n
    step = build_step("mix", [Request(p, n, t) for (p, n), t in zip(shapes, tables)],
                      dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                      num_blocks=nb, seed=int(rng.integers(1 << 30)), pad_tokens=3)
    for splits in (1, 4):
        out, lse, _ = run_gpu(step, num_splits=splits)
        (ro, rl), _ = run_oracle(step)
        check(step, out, lse, ro, rl, what=f"{dtype} d={d} G={hq // hkv} S={splits}")
        # padded rows past the scheduled tokens are not written
        assert torch.isnan(out[-3:]).all()


# ----------------------------------------------------------------------------
# exactness properties on the GPU: bitwise at a fixed split count
# ----------------------------------------------------------------------------

def test_deterministic_repeat():
    step = config_step(5, scale_down=SMALL[5])
    a, la, _ = run_gpu(step, num_splits=1)
    b, lb, _ = run_gpu(step, num_splits=1)
    assert same_bits(a, b) and same_bits(la, lb)


@pytest.mark.parametrize("splits", [1, 8])
def test_block_permutation_is_bitwise_invariant(splits):
    step = config_step(3, scale_down=SMALL[3])
    out, lse, _ = run_gpu(step, num_splits=splits)
    perm = np.random.default_rng(77).permutation(step.num_blocks)
    inv = torch.as_tensor(np.argsort(perm))
    bt = step.block_tables.copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    sm = step.slot_mapping
    step2 = config_step(3, scale_down=SMALL[3])
    step2.block_tables = bt.astype(np.int32)
    step2.slot_mapping = (perm[sm // 16] * 16 + sm % 16).astype(np.int64)
    step2.k_pool = step.k_pool[inv]
    step2.v_pool = step.v_pool[inv]
    out2, lse2, _ = run_gpu(step2, num_splits=splits)
    assert same_bits(out, out2) and same_bits(lse, lse2)


def test_shared_prefix_is_bitwise_equal_to_private_copies():
    step = config_step(5, scale_down=SMALL[5])
    shared = set(step.info["shared_blocks"])
    out_s, lse_s, _ = run_gpu(step, num_splits=1)
    # give every sharer private copies of the shared blocks
    bt = step.block_tables.copy()
    kp, vp = step.k_pool, step.v_pool
    extra_k, extra_v = [], []
    nb = step.num_blocks
    for b in range(step.num_seqs):
        for j in range(bt.shape[1]):
            if int(bt[b, j]) in shared:
                extra_k.append(kp[int(bt[b, j])])
                extra_v.append(vp[int(bt[b, j])])
                bt[b, j] = nb
                nb += 1
    priv = config_step(5, scale_down=SMALL[5])
    priv.block_tables = bt
    priv.k_pool = torch.cat([kp, torch.stack(extra_k)])
    priv.v_pool = torch.cat([vp, torch.stack(extra_v)])
    priv.num_blocks = nb
    out_p, lse_p, _ = run_gpu(priv, num_splits=1)
    assert same_bits(out_s, out_p) and same_bits(lse_s, lse_p)


def test_split_merge_deterministic_and_workspace_reusable():
    # the last split to finish merges; which one that is varies between runs,
    # the merge order does not.  One workspace serves every call: the arrival
    # counters at its head must be back to zero after each.
    pa = pa_mod()
    step = config_step(5, scale_down=SMALL[5])
    g = upload(step)
    (ro, rl), _ = run_oracle(step)
    hq = step.query.shape[1]
    ws = pa.workspace(step.num_seqs, step.num_tokens, hq, step.query.shape[2], 64)
    first = {}
    for rep in range(3):
        for splits in (8, 64, 3):
            pa.kv_write(g["key"], g["value"], g["k_pool"], g["v_pool"], g["slots"])
            out, lse = pa.attention(g["query"], g["k_pool"], g["v_pool"], g["qsl"],
                                    g["seq_lens"], g["tables"], step.max_query_len,
                                    step.max_seq_len, step.scale, num_splits=splits,
                                    workspace=ws)
            torch.cuda.synchronize()
            sem = ws[:4 * step.num_seqs * hq].view(torch.int32)
            assert int(sem.abs().sum()) == 0, f"counters not reset (S={splits})"
            if rep == 0:
                check(step, out, lse, ro, rl, what=f"shared workspace S={splits}")
                first[splits] = (out.clone(), lse.clone())
            else:
                assert same_bits(out, first[splits][0]) and same_bits(lse, first[splits][1])


def test_split_results_agree_with_each_other():
    step = config_step(2, scale_down=SMALL[2])
    outs = [run_gpu(step, num_splits=s)[0] for s in (1, 2, 16, 64)]
    for o in outs[1:]:
        assert float((o.float() - outs[0].float()).abs().max()) <= 2e-2


# ----------------------------------------------------------------------------
# split combine as its own entry point
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_split_combine_entry_point(dtype, d):
    pa = pa_mod()
    rng = np.random.default_rng(5)
    S, nt, hq = 37, 6, 8
    po = rng.standard_normal((S, nt, hq, d)).astype(np.float32)
    pl = (rng.standard_normal((S, nt, hq)) * 3).astype(np.float32)
    pl[rng.random((S, nt, hq)) < 0.3] = -np.inf
    pl[:, 2, 3] = -np.inf            # an entry with no key at all
    po[np.isneginf(pl)] = np.nan     # ignored entries may hold anything
    out, lse = pa.split_combine(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(),
                                dtype=dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.combine_partials(po.astype(np.float64), pl.astype(np.float64))
    o = to64(out)
    lg = lse.cpu().numpy().astype(np.float64)
    tol = 2e-2 if dtype == torch.bfloat16 else 1e-5
    # every entry, the one with no key included (oracle: out NaN, lse -inf)
    assert np.array_equal(np.isnan(o), np.isnan(ro))
    assert np.array_equal(np.isneginf(lg), np.isneginf(rl))
    fin = ~np.isnan(ro)
    assert np.abs(o[fin] - ro[fin]).max() <= tol
    fl = np.isfinite(rl)
    assert np.abs(lg[fl] - rl[fl]).max() <= 1e-4
    assert np.isnan(ro[2, 3]).all() and np.isneginf(rl[2, 3])


# ----------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times:
# sampled rows, each recomputed by the oracle from the requests it belongs to
# ----------------------------------------------------------------------------

def sampled_parity(step, req_ids, num_splits=0, rows_per_req=None, seed=0):
    out, lse, g = run_gpu(step, num_splits=num_splits)
    small, rows = extract_requests(step, req_ids)
    pick = None
    if rows_per_req is not None:
        rng = np.random.default_rng(seed)
        qsl = small.query_start_loc
        pick = []
        for i in range(small.num_seqs):
            lo, hi = int(qsl[i]), int(qsl[i + 1])
            n = hi - lo
            cand = sorted(set([lo, hi - 1] + rng.integers(lo, hi, size=min(n, rows_per_req)).tolist()))
            pick.extend(cand)
    (ro, rl), _ = run_oracle(small, rows=pick)
    sel = np.arange(len(rows)) if pick is None else np.asarray(pick)
    o = to64(out)[rows[sel]]
    assert np.isfinite(o).all()
    err = float(np.abs(o - ro[sel]).max())
    assert err <= TOL_OUT[step.dtype], f"{step.name}: max |out - oracle| = {err}"
    le = float(np.abs(lse.cpu().double().numpy()[rows[sel]] - rl[sel]).max())
    assert le <= TOL_LSE, f"{step.name}: max |lse - oracle| = {le}"
    return out, lse


@pytest.mark.parametrize("splits", [0, 1, 16, 128])
def test_full_config2(splits):
    step = config_step(2, device="cuda")
    sampled_parity(step, [0], num_splits=splits)


def test_full_config3():
    step = config_step(3, device="cuda")
    order = np.argsort(step.seq_lens)
    ids = sorted(set(order[:3].tolist() + order[-3:].tolist() + [7, 100, 200]))
    sampled_parity(step, ids)


@pytest.mark.parametrize("cfg", [2, 3])
def test_full_tensor_parallel_shard(cfg):
    # one GPU's share under 8-way tensor parallelism by KV head: Hq 4 / Hkv 1
    # at the full contexts (config 2: 32768 keys, split by the heuristic)
    step = config_step(cfg, device="cuda", scale_down={"q_heads": 4, "kv_heads": 1})
    assert step.num_q_heads == 4 and step.num_kv_heads == 1
    if cfg == 2:
        sampled_parity(step, [0])
    else:
        order = np.argsort(step.seq_lens)
        sampled_parity(step, sorted(set(order[:2].tolist() + order[-2:].tolist() + [50])))


def test_full_config4():
    step = config_step(4, device="cuda")
    sampled_parity(step, [0, 3], rows_per_req=24, seed=4)


def test_full_config5():
    step = config_step(5, device="cuda")
    q = step.q_lens
    prefill = np.nonzero(q > 1)[0].tolist()
    dec = np.nonzero(q == 1)[0]
    sl = step.seq_lens[dec]
    shared = set(step.info["shared_blocks"])
    sharer = [int(b) for b in dec if int(step.block_tables[b, 0]) in shared][:3]
    ids = sorted(set(prefill + dec[np.argsort(sl)[-3:]].tolist() + dec[:6].tolist() + sharer))
    sampled_parity(step, ids, rows_per_req=12, seed=5)


def test_bf16_rounding_matches_torch_rne():
    # a single split passes o_0 through unchanged (weight 1), so the bf16
    # output is exactly the kernel's fp32 -> bf16 rounding of o_0
    pa = pa_mod()
    rng = np.random.default_rng(17)
    po = (rng.standard_normal((1, 64, 8, 128)) * 7).astype(np.float32)
    # values that sit exactly on rounding ties and next to them
    # (the sum over splits starts from +0, so a -0 input or a subnormal would
    # test the accumulation, not the rounding: none are used)
    po[0, 0, 0, :8] = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -120,
                                65504.5, 3.4e38, 1 + 5 * 2 ** -9, 1 + 2 ** -9], dtype=np.float32)
    pl = np.zeros((1, 64, 8), dtype=np.float32)
    out, lse = pa.split_combine(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(),
                                dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = torch.from_numpy(po[0]).to(torch.bfloat16)
    got = out.cpu().view(torch.int16).numpy()
    want = ref.view(torch.int16).numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, [(tuple(i), float(po[0][tuple(i)]), hex(got[tuple(i)] & 0xffff),
                            hex(want[tuple(i)] & 0xffff)) for i in bad[:8]]
    assert np.all(lse.cpu().numpy() == 0.0)
