"""Pins for the fp64 oracle: it is checked against what the pages and the
mathematics fix, never against itself or the HIP path.

* printed worked example of the flat metadata ("Model execution", section
  "Code", output of flatten_batch.py) and the page's slot explanation;
* the "Try it" extension of the same page (block crossing, derived by hand);
* pure-Python brute force on tiny inputs;
* closed forms (one key, uniform weights, equal keys, a dominant key);
* library special cases (torch SDPA in fp64, scipy logsumexp, torch bf16);
* the exactness claims of "Inside the engine: ..." (online softmax equals the
  full softmax; split-KV plus combine equals the unsplit result; paging and
  shared blocks change nothing);
* byte arithmetic the pages print.
Planted-mistake tests at the end show that each pin family catches a
plausible slip in the oracle.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import paged_attention as opa
from tests.conftest import read_golden

BS = 16


# ----------------------------------------------------------------------------
# small random steps built by hand (independent of the workloads package)
# ----------------------------------------------------------------------------

def same_bits(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def bf16_bits(x):
    """Round float64 values to bf16 (RNE) with torch; return uint16 bits."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def tiny_step(rng, shapes, Hq, Hkv, d, dtype, num_blocks=None, poison=True):
    """shapes: list of (prior, n).  Returns a dict of raw inputs."""
    need = [-(-(p + n) // BS) for p, n in shapes]
    NB = num_blocks or (sum(need) + 3)
    perm = rng.permutation(NB)
    tables, k = [], 0
    for nb in need:
        tables.append(list(perm[k:k + nb]))
        k += nb
    stride = max(need)
    bt = np.full((len(shapes), stride), -1, dtype=np.int32)
    for b, t in enumerate(tables):
        bt[b, :len(t)] = t
    qsl = np.zeros(len(shapes) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum([n for _, n in shapes])
    seq_lens = np.array([p + n for p, n in shapes], dtype=np.int32)
    Nt = int(qsl[-1])
    slots = []
    for (p, n), t in zip(shapes, tables):
        for pos in range(p, p + n):
            slots.append(t[pos // BS] * BS + pos % BS)
    slots = np.array(slots, dtype=np.int64)

    def vals(*shape):
        x = rng.standard_normal(shape)
        return bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)

    q = vals(Nt, Hq, d)
    key = vals(Nt, Hkv, d)
    value = vals(Nt, Hkv, d)
    kp = vals(NB, Hkv, BS, d)
    vp = vals(NB, Hkv, d, BS)
    if poison:
        nan = bf16_bits(np.nan)[()] if dtype == "bf16" else np.float32(np.nan)
        live = np.zeros(NB * BS, dtype=bool)
        for (p, n), t in zip(shapes, tables):
            for pos in range(p):
                live[t[pos // BS] * BS + pos % BS] = True
        live = live.reshape(NB, BS)
        for blk in range(NB):
            for off in range(BS):
                if not live[blk, off]:
                    kp[blk, :, off, :] = nan
                    vp[blk, :, :, off] = nan
    return dict(query=q, key=key, value=value, k_pool=kp, v_pool=vp, qsl=qsl,
                seq_lens=seq_lens, block_tables=bt, slot_mapping=slots,
                num_blocks=NB, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype)


def run_oracle(st, scale, fn=None, **kw):
    kp, vp = oracle.kv_write(st["key"], st["value"], st["k_pool"], st["v_pool"],
                             st["slot_mapping"])
    fn = fn or oracle.attention
    return fn(st["query"], kp, vp, st["qsl"], st["seq_lens"], st["block_tables"],
              scale, st["Hkv"], st["dtype"], **kw)


def brute_force(st, scale):
    """Pure-Python loops, straight from the definitions: KV write through the
    slots, then for each row and head the scores over visible positions read
    through the block table, softmax with math.exp, weighted sum of V."""
    w = lambda x: float(opa.to_f64(np.asarray(x), st["dtype"]))  # noqa: E731
    Hq, Hkv, d = st["Hq"], st["Hkv"], st["d"]
    G = Hq // Hkv
    # the write, slot by slot, into dictionaries keyed by (block, offset)
    Kc, Vc = {}, {}
    for t, s in enumerate(st["slot_mapping"]):
        Kc[(s // BS, s % BS)] = t
    out = {}
    for b in range(len(st["seq_lens"])):
        lo, hi = int(st["qsl"][b]), int(st["qsl"][b + 1])
        seq_len = int(st["seq_lens"][b])
        for t in range(lo, hi):
            pos = seq_len - (hi - lo) + (t - lo)
            for h in range(Hq):
                g = h // G
                scores, vrows = [], []
                for j in range(pos + 1):
                    blk, off = int(st["block_tables"][b][j // BS]), j % BS
                    if (blk, off) in Kc:
                        src = Kc[(blk, off)]
                        kv = [w(st["key"][src, g, c]) for c in range(d)]
                        vv = [w(st["value"][src, g, c]) for c in range(d)]
                    else:
                        kv = [w(st["k_pool"][blk, g, off, c]) for c in range(d)]
                        vv = [w(st["v_pool"][blk, g, c, off]) for c in range(d)]
                    s = sum(w(st["query"][t, h, c]) * kv[c] for c in range(d))
                    scores.append(scale * s)
                    vrows.append(vv)
                mx = max(scores)
                ex = [math.exp(s - mx) for s in scores]
                den = sum(ex)
                o = [sum(ex[j] * vrows[j][c] for j in range(len(ex))) / den
                     for c in range(d)]
                out[(t, h)] = (o, mx + math.log(den))
    return out


# ----------------------------------------------------------------------------
# metadata: the page's worked example
# ----------------------------------------------------------------------------

PAGE_SCHEDULE = [(0, 5, [7]), (37, 1, [2, 9, 4]), (32, 3, [11, 12, 3])]


def test_flatten_matches_printed_output():
    g = read_golden("flatten_batch_printed.txt")
    got = oracle.flatten_schedule(PAGE_SCHEDULE)
    for key in ("request_index", "positions", "query_start_loc", "seq_lens",
                "slot_mapping", "logits_indices"):
        assert got[key] == g[key][0], key


def test_slot_explanation_b_decode():
    # request B's position 37: third block (index 2) = physical 4, offset 5
    got = oracle.flatten_schedule([(37, 1, [2, 9, 4])])
    assert got["slot_mapping"] == [4 * 16 + 5] == [69]


def test_try_it_block_crossing():
    # 2 computed, 30 scheduled on blocks [5, 6]: positions 2..31; the slot
    # leaves block 5 after position 15 and continues in block 6
    got = oracle.flatten_schedule([(2, 30, [5, 6])])
    assert got["positions"] == list(range(2, 32))
    assert got["slot_mapping"] == list(range(82, 96)) + list(range(96, 112))
    assert got["seq_lens"] == [32]
    k = got["positions"].index(16)
    assert got["slot_mapping"][k - 1] == 5 * 16 + 15 and got["slot_mapping"][k] == 6 * 16


def test_capture_ladder_matches_printed_output():
    g = read_golden("capture_ladder_printed.txt")
    sizes = oracle.capture_sizes()
    assert len(sizes) == g["count"][0][0]
    assert sizes[:6] == g["first"][0]
    assert sizes[-3:] == g["last"][0]
    import bisect
    for n, used, padded in g["pad"]:
        k = bisect.bisect_left(sizes, n)
        if used < 0:
            assert k == len(sizes)
        else:
            assert sizes[k] == used and sizes[k] - n == padded


def test_validate_accepts_page_example_and_rejects_bad_slots():
    got = oracle.flatten_schedule(PAGE_SCHEDULE)
    bt = np.full((3, 3), -1, dtype=np.int32)
    for b, (_, _, t) in enumerate(PAGE_SCHEDULE):
        bt[b, :len(t)] = t
    oracle.validate_step(got["query_start_loc"], got["seq_lens"], bt,
                         got["slot_mapping"], 9, 16)
    bad = list(got["slot_mapping"])
    bad[5] = 70
    with pytest.raises(AssertionError):
        oracle.validate_step(got["query_start_loc"], got["seq_lens"], bt, bad, 9, 16)
    dup = list(got["slot_mapping"])
    dup[1] = dup[0]
    with pytest.raises(AssertionError):
        oracle.validate_step(got["query_start_loc"], got["seq_lens"], bt, dup, 9, 16)


# ----------------------------------------------------------------------------
# byte arithmetic printed on the pages
# ----------------------------------------------------------------------------

def test_byte_figures():
    # T x T fp16 score matrix at T = 8K: 128 MB (binary megabytes)
    assert 8192 * 8192 * 2 == 128 * 2 ** 20
    # KV bytes per token for 80 layers x 8 KV heads x d 128 in 16-bit, K and V
    assert 2 * 80 * 8 * 128 * 2 == 327_680


# ----------------------------------------------------------------------------
# KV write
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_write_gather_returns_inputs(dtype):
    rng = np.random.default_rng(11)
    st = tiny_step(rng, [(0, 21), (5, 1), (30, 4)], 4, 2, 8, dtype)
    kp, vp = oracle.kv_write(st["key"], st["value"], st["k_pool"], st["v_pool"],
                             st["slot_mapping"])
    for b in range(3):
        K, V = oracle.gather_context(kp, vp, st["block_tables"][b], int(st["seq_lens"][b]))
        lo, hi = st["qsl"][b], st["qsl"][b + 1]
        n = hi - lo
        assert same_bits(K[-n:], st["key"][lo:hi])
        assert same_bits(V[-n:], st["value"][lo:hi])
    # every slot not in slot_mapping is bit-identical to before
    touched = np.zeros(st["num_blocks"] * BS, dtype=bool)
    touched[st["slot_mapping"]] = True
    touched = touched.reshape(-1, BS)
    for blk in range(st["num_blocks"]):
        for off in range(BS):
            if not touched[blk, off]:
                assert same_bits(kp[blk, :, off, :], st["k_pool"][blk, :, off, :])
                assert same_bits(vp[blk, :, :, off], st["v_pool"][blk, :, :, off])


def test_kv_write_skips_negative_slots():
    rng = np.random.default_rng(12)
    st = tiny_step(rng, [(0, 5)], 2, 1, 4, "f32")
    sm = st["slot_mapping"].copy()
    sm[2] = -1
    kp, vp = oracle.kv_write(st["key"], st["value"], st["k_pool"], st["v_pool"], sm)
    s = st["slot_mapping"][2]
    assert same_bits(kp[s // BS, :, s % BS, :], st["k_pool"][s // BS, :, s % BS, :])
    assert same_bits(vp[s // BS, :, :, s % BS], st["v_pool"][s // BS, :, :, s % BS])


# ----------------------------------------------------------------------------
# attention: brute force, closed forms, library special cases
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shapes,Hq,Hkv", [
    ([(0, 7)], 2, 2),
    ([(0, 19), (4, 1), (16, 1), (33, 2)], 4, 2),
    ([(13, 6), (0, 3), (31, 1)], 6, 2),
    ([(17, 18)], 3, 1),
])
def test_brute_force_tiny(dtype, shapes, Hq, Hkv):
    rng = np.random.default_rng(hash((dtype, Hq, len(shapes))) % 2 ** 32)
    d = 5
    st = tiny_step(rng, shapes, Hq, Hkv, d, dtype)
    scale = 0.37
    out, lse = run_oracle(st, scale)
    bf = brute_force(st, scale)
    for (t, h), (o, l) in bf.items():
        np.testing.assert_allclose(out[t, h], o, rtol=0, atol=1e-12)
        assert abs(lse[t, h] - l) <= 1e-12
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


def test_closed_form_single_key_returns_v():
    rng = np.random.default_rng(3)
    st = tiny_step(rng, [(0, 1)], 4, 2, 8, "f32")
    out, lse = run_oracle(st, 0.125)
    v = st["value"][0].astype(np.float64)
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], v[h // 2])
        s = 0.125 * float(st["query"][0, h].astype(np.float64) @ st["key"][0, h // 2].astype(np.float64))
        assert abs(lse[0, h] - s) < 1e-12


def test_closed_form_zero_scale_is_prefix_mean():
    rng = np.random.default_rng(4)
    st = tiny_step(rng, [(9, 7)], 2, 1, 6, "f32")
    out, lse = run_oracle(st, 0.0)
    kp, vp = oracle.kv_write(st["key"], st["value"], st["k_pool"], st["v_pool"], st["slot_mapping"])
    _, V = oracle.gather_context(kp, vp, st["block_tables"][0], 16)
    V = V.astype(np.float64)[:, 0, :]
    csum = np.cumsum(V, axis=0)
    for i in range(7):
        p = 9 + i
        for h in range(2):
            np.testing.assert_allclose(out[i, h], csum[p] / (p + 1), atol=1e-13)
            assert abs(lse[i, h] - math.log(p + 1)) < 1e-13


def test_closed_form_equal_keys_is_mean_of_v_and_dominant_key():
    rng = np.random.default_rng(5)
    st = tiny_step(rng, [(20, 1)], 2, 1, 4, "f32", poison=False)
    # all cached keys equal -> uniform weights over the visible positions
    st["k_pool"][:] = 0.5
    st["key"][:] = 0.5
    out, _ = run_oracle(st, 1.0)
    kp, vp = oracle.kv_write(st["key"], st["value"], st["k_pool"], st["v_pool"], st["slot_mapping"])
    _, V = oracle.gather_context(kp, vp, st["block_tables"][0], 21)
    np.testing.assert_allclose(out[0, 0], V[:, 0, :].astype(np.float64).mean(axis=0), atol=1e-13)
    # one key far above the rest -> its value row
    K, _ = oracle.gather_context(kp, vp, st["block_tables"][0], 21)
    j = 7
    blk, off = st["block_tables"][0][j // BS], j % BS
    st["k_pool"][blk, 0, off, :] = 40.0
    st["query"][0] = 1.0
    out, _ = run_oracle(st, 1.0)
    np.testing.assert_allclose(out[0, 0], V[j, 0, :].astype(np.float64), atol=1e-12)


def _sdpa(q, k, v, scale, mask=None, causal=False):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(q)[None], torch.as_tensor(k)[None], torch.as_tensor(v)[None],
        attn_mask=mask, is_causal=causal, scale=scale)[0].numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sdpa_prefill_from_empty_context(dtype):
    rng = np.random.default_rng(6)
    Hq, Hkv, d, n = 8, 2, 16, 45
    st = tiny_step(rng, [(0, n)], Hq, Hkv, d, dtype)
    scale = 1 / math.sqrt(d)
    out, _ = run_oracle(st, scale)
    q = opa.to_f64(st["query"], dtype).transpose(1, 0, 2)             # [Hq, n, d]
    k = opa.to_f64(st["key"], dtype).transpose(1, 0, 2)
    v = opa.to_f64(st["value"], dtype).transpose(1, 0, 2)
    G = Hq // Hkv
    k = np.repeat(k, G, axis=0)
    v = np.repeat(v, G, axis=0)
    ref = _sdpa(q, k, v, scale, causal=True).transpose(1, 0, 2)
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_sdpa_decode_sees_whole_context():
    rng = np.random.default_rng(7)
    Hq, Hkv, d, prior = 4, 1, 8, 50
    st = tiny_step(rng, [(prior, 1)], Hq, Hkv, d, "bf16")
    out, _ = run_oracle(st, 0.3)
    kp, vp = oracle.kv_write(st["key"], st["value"], st["k_pool"], st["v_pool"], st["slot_mapping"])
    K, V = oracle.gather_context(kp, vp, st["block_tables"][0], prior + 1)
    K = opa.to_f64(K, "bf16").transpose(1, 0, 2).repeat(Hq, axis=0)
    V = opa.to_f64(V, "bf16").transpose(1, 0, 2).repeat(Hq, axis=0)
    q = opa.to_f64(st["query"], "bf16").transpose(1, 0, 2)
    ref = _sdpa(q, K, V, 0.3).transpose(1, 0, 2)
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_lse_matches_scipy_logsumexp():
    rng = np.random.default_rng(8)
    st = tiny_step(rng, [(10, 3)], 2, 2, 8, "f32")
    out, lse = run_oracle(st, 0.7)
    kp, vp = oracle.kv_write(st["key"], st["value"], st["k_pool"], st["v_pool"], st["slot_mapping"])
    K, _ = oracle.gather_context(kp, vp, st["block_tables"][0], 13)
    for i in range(3):
        for h in range(2):
            s = 0.7 * (K[: 11 + i, h, :].astype(np.float64) @ st["query"][i, h].astype(np.float64))
            assert abs(lse[i, h] - scipy.special.logsumexp(s)) < 1e-12


def test_bf16_widening_is_exact():
    x = np.random.default_rng(9).standard_normal(1000) * 100
    bits = bf16_bits(x)
    ref = torch.as_tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(opa.to_f64(bits, "bf16"), ref)
    assert np.isnan(opa.to_f64(bf16_bits(np.nan), "bf16"))


# ----------------------------------------------------------------------------
# exactness claims: online = full, split + combine = unsplit, paging invariance
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("tiles", [[1], [3, 16, 5], [16], [64, 7]])
def test_online_softmax_equals_full(tiles):
    rng = np.random.default_rng(21)
    st = tiny_step(rng, [(0, 23), (40, 1), (17, 5)], 4, 2, 8, "bf16")
    full, lf = run_oracle(st, 0.2)
    onl, lo = run_oracle(st, 0.2, fn=oracle.attention_online, tile_sizes=tiles)
    np.testing.assert_allclose(onl, full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lo, lf, rtol=0, atol=1e-12)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64])
def test_split_combine_equals_unsplit(splits):
    rng = np.random.default_rng(22)
    st = tiny_step(rng, [(70, 1), (0, 9), (3, 1), (100, 4)], 4, 1, 8, "bf16")
    full, lf = run_oracle(st, 0.2)
    po, pl = run_oracle(st, 0.2, fn=oracle.attention_split_partials, num_splits=splits)
    out, lse = oracle.combine_partials(po, pl)
    np.testing.assert_allclose(out, full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lf, rtol=0, atol=1e-12)
    if splits == 64:
        assert np.isneginf(pl).any()  # empty splits occur and weigh nothing


def test_combine_against_direct_weights():
    # two splits with known lse: weights are e^lse_s / sum e^lse
    po = np.array([[[[1.0, 2.0]]], [[[3.0, -1.0]]]])
    pl = np.array([[[0.0]], [[math.log(3.0)]]])
    out, lse = oracle.combine_partials(po, pl)
    np.testing.assert_allclose(out[0, 0], [0.25 * 1 + 0.75 * 3, 0.25 * 2 - 0.75], atol=1e-15)
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-15


def test_combine_empty_entries():
    # an entry with one non-empty split is that split; an entry with none saw
    # no key: the sum over splits is empty, so lse = ln 0 = -inf and o = 0/0
    po = np.array([[[[1.0, 2.0]], [[5.0, 6.0]]],
                   [[[np.nan, np.nan]], [[np.nan, np.nan]]],
                   [[[7.0, -8.0]], [[np.inf, np.nan]]]])       # [S=3, Nt=2, Hq=1, d=2]
    pl = np.array([[[-np.inf], [-np.inf]],
                   [[-np.inf], [-np.inf]],
                   [[0.75], [-np.inf]]])                        # [S=3, Nt=2, Hq=1]
    out, lse = oracle.combine_partials(po, pl)
    assert np.array_equal(out[0, 0], [7.0, -8.0]) and lse[0, 0] == 0.75
    assert np.isneginf(lse[1, 0]) and np.isnan(out[1, 0]).all()


def test_block_permutation_invariance():
    rng = np.random.default_rng(23)
    st = tiny_step(rng, [(33, 1), (0, 20), (5, 3)], 4, 2, 8, "bf16")
    out, lse = run_oracle(st, 0.3)
    NB = st["num_blocks"]
    perm = np.random.default_rng(24).permutation(NB)       # old block -> new block
    inv = np.argsort(perm)
    st2 = dict(st)
    st2["k_pool"] = st["k_pool"][inv]
    st2["v_pool"] = st["v_pool"][inv]
    bt = st["block_tables"].copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    st2["block_tables"] = bt
    sm = st["slot_mapping"]
    st2["slot_mapping"] = perm[sm // BS] * BS + sm % BS
    out2, lse2 = run_oracle(st2, 0.3)
    np.testing.assert_array_equal(out2, out)
    np.testing.assert_array_equal(lse2, lse)


def test_shared_prefix_blocks_equal_private_copies():
    rng = np.random.default_rng(25)
    # two decodes with a 32-token common prefix: shared blocks vs private copies
    st = tiny_step(rng, [(40, 1), (50, 1)], 4, 2, 8, "bf16", num_blocks=12)
    bt = st["block_tables"]
    kp, vp = st["k_pool"].copy(), st["v_pool"].copy()
    # make request 1's first two blocks private copies of request 0's
    for j in range(2):
        kp[bt[1, j]] = kp[bt[0, j]]
        vp[bt[1, j]] = vp[bt[0, j]]
    priv = dict(st, k_pool=kp, v_pool=vp)
    out_p, lse_p = run_oracle(priv, 0.4)
    shared_bt = bt.copy()
    shared_bt[1, :2] = bt[0, :2]
    shared = dict(priv, block_tables=shared_bt)
    out_s, lse_s = run_oracle(shared, 0.4)
    np.testing.assert_array_equal(out_s, out_p)
    np.testing.assert_array_equal(lse_s, lse_p)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(26)
    st = tiny_step(rng, [(0, 17), (9, 1)], 2, 1, 8, "f32")
    out, lse = run_oracle(st, 0.5)
    rows = [0, 5, 16, 17]
    o2, l2 = run_oracle(st, 0.5, rows=rows)
    np.testing.assert_array_equal(o2[rows], out[rows])
    assert np.isnan(o2[1]).all()


# ----------------------------------------------------------------------------
# planted mistakes: each plausible slip must fail a pin above
# ----------------------------------------------------------------------------

def _brute_fails(monkeypatch, target, replacement, d=4):
    monkeypatch.setattr(opa, target, replacement)
    rng = np.random.default_rng(31)
    st = tiny_step(rng, [(0, 9), (20, 2)], 4, 2, d, "f32")
    out, _ = run_oracle(st, 0.5)
    bf = brute_force(st, 0.5)
    return any(not np.allclose(out[t, h], o, atol=1e-9) for (t, h), (o, _) in bf.items())


def test_planted_wrong_gqa_mapping_is_caught(monkeypatch):
    assert _brute_fails(monkeypatch, "kv_head_of", lambda h, hq, hkv: h % hkv)


def test_planted_transposed_v_block_is_caught(monkeypatch):
    real = opa.gather_context

    def wrong(k_pool, v_pool, table_row, seq_len, block_size=BS):
        K, _ = real(k_pool, v_pool, table_row, seq_len, block_size)
        j = np.arange(seq_len)
        blk = np.asarray(table_row)[j // block_size]
        V = v_pool[blk, :, j % block_size, :]        # reads V as if token-major
        return K, V
    # head_dim 16 = block_size, so the wrong read has the right shape
    assert _brute_fails(monkeypatch, "gather_context", wrong, d=16)


def test_planted_strict_causal_mask_is_caught(monkeypatch):
    real_rows = opa._rows_of

    def attention_strict(query, k_pool, v_pool, qsl, seq_lens, bt, scale, hkv, dtype, **kw):
        # a copy of the oracle that hides the diagonal key (j < p instead of j <= p)
        q = opa.to_f64(query, dtype)
        out = np.full(q.shape, np.nan)
        for b in range(len(seq_lens)):
            ts = real_rows(qsl, b, None)
            ql = int(qsl[b + 1]) - int(qsl[b])
            K, V = opa.gather_context(k_pool, v_pool, bt[b], int(seq_lens[b]))
            K, V = opa.to_f64(K, dtype), opa.to_f64(V, dtype)
            for t in ts:
                p = int(seq_lens[b]) - ql + t - int(qsl[b])
                for h in range(q.shape[1]):
                    g = h // (q.shape[1] // hkv)
                    if p == 0:
                        out[t, h] = V[0, g]
                        continue
                    s = scale * K[:p, g] @ q[t, h]
                    w = np.exp(s - s.max())
                    out[t, h] = (w / w.sum()) @ V[:p, g]
        return out, None
    rng = np.random.default_rng(32)
    st = tiny_step(rng, [(0, 6)], 2, 1, 4, "f32")
    bad, _ = run_oracle(st, 0.5, fn=attention_strict)
    bf = brute_force(st, 0.5)
    assert any(not np.allclose(bad[t, h], o, atol=1e-9) for (t, h), (o, _) in bf.items())


def test_cascade_equals_plain_attention():
    # three decodes (one with 2 new tokens) and a prefill share a 2-block
    # prefix; one decode's context is shorter than the prefix
    rng = np.random.default_rng(27)
    st = tiny_step(rng, [(40, 1), (50, 2), (20, 1), (0, 9), (70, 1)], 4, 2, 8, "bf16",
                   num_blocks=24)
    bt = st["block_tables"].copy()
    prefix = list(bt[0, :2])
    for b in (1, 2, 4):
        bt[b, :2] = prefix
    st = dict(st, block_tables=bt)
    full, lf = run_oracle(st, 0.3)
    casc, lc = run_oracle(st, 0.3, fn=oracle.attention_cascade, sharers=[0, 1, 2, 4],
                          prefix_blocks=prefix)
    np.testing.assert_allclose(casc, full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lc, lf, rtol=0, atol=1e-12)
    # planted: a sharer whose table does not start with the prefix reads the
    # shared blocks instead (so the prefix list is what the cascade reads)
    rng2 = np.random.default_rng(27)
    orig = tiny_step(rng2, [(40, 1), (50, 2), (20, 1), (0, 9), (70, 1)], 4, 2, 8, "bf16",
                     num_blocks=24)["block_tables"]
    bt2 = bt.copy()
    bt2[4, :2] = [orig[1, 0], prefix[1]]    # a fully written block of another request
    st2 = dict(st, block_tables=bt2)
    full2, _ = run_oracle(st2, 0.3)
    casc2, _ = run_oracle(st2, 0.3, fn=oracle.attention_cascade, sharers=[4],
                          prefix_blocks=prefix)
    t4 = int(st["qsl"][4])
    assert np.abs(casc2[t4] - full2[t4]).max() > 1e-3
