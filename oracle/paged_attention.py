"""fp64 reference for the KV write and causal paged attention of one flat step.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Data conventions shared with the library only as a written contract (no code
is shared):

* bf16 tensors travel as raw ``uint16`` bit patterns, fp32 as ``float32``.
* ``query``: [num_tokens, num_q_heads, head_dim].
* ``key``/``value`` (the step's new tokens): [num_tokens, num_kv_heads, head_dim].
* K pool: [num_blocks, num_kv_heads, block_size, head_dim]  (token-major block).
* V pool: [num_blocks, num_kv_heads, head_dim, block_size]  (dim-major block).
* ``query_start_loc`` [B+1], ``seq_lens`` [B], ``block_tables`` [B, stride],
  ``slot_mapping`` [num_tokens] (negative = padded token, nothing written).

The placement of a token inside a block never changes a result; the oracle
indexes both pools by (slot // block_size, slot % block_size) under the
layouts above.
"""

from __future__ import annotations

import math

import numpy as np

BLOCK_SIZE = 16


# ----------------------------------------------------------------------------
# exact widening
# ----------------------------------------------------------------------------

def to_f64(x, dtype: str) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) or float32 values to float64 exactly
    (float64 input passes through).

    A bf16 value is the upper half of the float32 with the same bits, so the
    widening is a 16-bit left shift followed by a reinterpretation.
    """
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# flat metadata ("Model execution", section "Flattening a step")
# ----------------------------------------------------------------------------

def flatten_schedule(schedule, block_size: int = BLOCK_SIZE) -> dict:
    """Build the flat tensors of one step from a schedule.

    ``schedule`` is a list of ``(done, n, table)``: tokens already computed,
    tokens scheduled this step, and the request's physical block ids.  Each
    output is the page's definition of that flat tensor, evaluated over all
    rows at once:

    * query_start_loc: cumulative token counts, starting at 0
    * request_index: the request a flat row belongs to (its count repeated)
    * positions: done of the row's request plus the row's offset inside it
    * seq_lens: total context after the step, done + n
    * slot_mapping: block_id * block_size + offset, block_id the table entry of
      the block holding the position
    * logits_indices: the last flat row of each request (next start - 1)
    """
    done = np.array([int(s[0]) for s in schedule], dtype=np.int64)
    count = np.array([int(s[1]) for s in schedule], dtype=np.int64)
    qsl = np.concatenate([[0], np.cumsum(count)]).astype(np.int64)
    req = np.repeat(np.arange(len(schedule), dtype=np.int64), count)
    offset = np.arange(int(qsl[-1]), dtype=np.int64) - qsl[req]
    pos = done[req] + offset
    block_id = np.array([int(schedule[r][2][p // block_size]) for r, p in zip(req, pos)],
                        dtype=np.int64)
    slots = block_id * block_size + pos % block_size
    return {
        "request_index": req.tolist(),
        "positions": pos.tolist(),
        "query_start_loc": qsl.tolist(),
        "seq_lens": (done + count).tolist(),
        "slot_mapping": slots.tolist(),
        "logits_indices": (qsl[1:] - 1).tolist(),
    }


def capture_sizes(top: int = 512) -> list:
    """Capture-size ladder of the same page, from its stated rule: 1, 2 and 4,
    then every multiple of 8 below 256, then every multiple of 16 from 256 up
    to ``top``."""
    def on_ladder(n: int) -> bool:
        if n < 8:
            return n in (1, 2, 4)
        return n % (8 if n < 256 else 16) == 0
    return [n for n in range(1, top + 1) if on_ladder(n)]


def validate_step(query_start_loc, seq_lens, block_tables, slot_mapping,
                  num_tokens: int, num_blocks: int,
                  block_size: int = BLOCK_SIZE) -> None:
    """Assert that the metadata of a step is consistent.

    Checks what the definitions of the flat tensors imply: offsets start at 0
    and never decrease, each request's context holds its new tokens, the block
    table covers the context with valid block ids, new-token slots are
    distinct, and every new token's slot is the one its request's block table
    gives for its position (position = context before the step + row index).
    """
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    bt = np.asarray(block_tables, dtype=np.int64)
    sm = np.asarray(slot_mapping, dtype=np.int64)
    B = sl.shape[0]
    assert qsl.shape == (B + 1,), "query_start_loc must have num_seqs + 1 entries"
    assert qsl[0] == 0, "query_start_loc[0] must be 0"
    assert np.all(np.diff(qsl) >= 0), "query_start_loc must not decrease"
    assert qsl[-1] <= num_tokens, "query_start_loc[-1] exceeds num_tokens"
    assert sm.shape[0] >= qsl[-1], "slot_mapping shorter than the scheduled tokens"
    q_len = np.diff(qsl)
    assert np.all(sl >= q_len), "seq_len must include the new tokens"
    if B:
        nblk = -(-sl // block_size)
        assert np.all(nblk <= bt.shape[1]), "block table narrower than context"
    for b in range(B):
        used = bt[b, : -(-sl[b] // block_size)]
        assert np.all((used >= 0) & (used < num_blocks)), "block id out of range"
    live = sm[sm >= 0]
    assert np.unique(live).size == live.size, "duplicate slots in slot_mapping"
    assert np.all(live < num_blocks * block_size), "slot out of range"
    for b in range(B):
        ctx = sl[b] - q_len[b]
        for i in range(q_len[b]):
            p = ctx + i
            want = bt[b, p // block_size] * block_size + p % block_size
            assert sm[qsl[b] + i] == want, "slot does not match the block table"


# ----------------------------------------------------------------------------
# KV write (slot_mapping) and gather (block table)
# ----------------------------------------------------------------------------

def kv_write(key, value, k_pool, v_pool, slot_mapping,
             block_size: int = BLOCK_SIZE):
    """Return copies of the pools with each new token's K and V at its slot.

    The write is a copy of bits: nothing is converted.  A negative slot marks a
    padded token whose K/V are not written.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    sm = np.asarray(slot_mapping, dtype=np.int64)
    for t in range(sm.shape[0]):
        s = int(sm[t])
        if s < 0:
            continue
        blk, off = divmod(s, block_size)
        k_out[blk, :, off, :] = key[t]
        v_out[blk, :, :, off] = value[t]
    return k_out, v_out


def gather_context(k_pool, v_pool, table_row, seq_len: int,
                   block_size: int = BLOCK_SIZE):
    """Read a request's first ``seq_len`` cached tokens through its block table.

    Returns K and V as [seq_len, num_kv_heads, head_dim] in the pools' dtype;
    logical position j lives in block ``table_row[j // block_size]`` at offset
    ``j % block_size``.
    """
    j = np.arange(seq_len)
    blk = np.asarray(table_row, dtype=np.int64)[j // block_size]
    off = j % block_size
    K = k_pool[blk, :, off, :]          # [seq_len, Hkv, d]
    V = v_pool[blk, :, :, off]          # [seq_len, Hkv, d]
    return K, V


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Grouped-query mapping: query head h reads KV head h // (Hq / Hkv)."""
    return h // (num_q_heads // num_kv_heads)


# ----------------------------------------------------------------------------
# attention, full softmax ("Never materialise the T x T matrix": the textbook
# definition the tiled method must equal)
# ----------------------------------------------------------------------------

def _rows_of(query_start_loc, b, rows):
    lo, hi = int(query_start_loc[b]), int(query_start_loc[b + 1])
    if rows is None:
        return list(range(lo, hi))
    return [t for t in rows if lo <= t < hi]


def attention(query, k_pool, v_pool, query_start_loc, seq_lens, block_tables,
              scale: float, num_kv_heads: int, dtype: str,
              block_size: int = BLOCK_SIZE, rows=None):
    """Causal attention of every scheduled row through the block tables.

    For request b with q_len new rows and context seq_len, row i sits at
    position p = (seq_len - q_len) + i and sees the keys at positions 0..p.
    Per query head h (KV head h // G): S = scale * q K^T over those keys,
    P = softmax(S), o = P V, and lse = m + ln(l) with m = max S and
    l = sum exp(S - m).

    Returns (out [num_tokens, Hq, d], lse [num_tokens, Hq]) in float64; rows
    not computed (not scheduled, or not in ``rows``) are NaN.
    """
    q = to_f64(query, dtype)
    Nt, Hq, d = q.shape
    out = np.full((Nt, Hq, d), np.nan)
    lse = np.full((Nt, Hq), np.nan)
    B = len(seq_lens)
    for b in range(B):
        ts = _rows_of(query_start_loc, b, rows)
        if not ts:
            continue
        q_len = int(query_start_loc[b + 1]) - int(query_start_loc[b])
        seq_len = int(seq_lens[b])
        ctx = seq_len - q_len
        Kr, Vr = gather_context(k_pool, v_pool, block_tables[b], seq_len, block_size)
        K = to_f64(Kr, dtype)
        V = to_f64(Vr, dtype)
        pos = np.array([ctx + (t - int(query_start_loc[b])) for t in ts])
        visible = np.arange(seq_len)[None, :] <= pos[:, None]      # [rows, seq_len]
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, num_kv_heads)
            S = scale * (q[ts, h, :] @ K[:, kvh, :].T)              # [rows, seq_len]
            S = np.where(visible, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            w = np.exp(S - m)
            l = w.sum(axis=1, keepdims=True)
            out[ts, h, :] = (w / l) @ V[:, kvh, :]
            lse[ts, h] = (m + np.log(l))[:, 0]
    return out, lse


# ----------------------------------------------------------------------------
# self-check variants
# ----------------------------------------------------------------------------

def attention_online(query, k_pool, v_pool, query_start_loc, seq_lens,
                     block_tables, scale: float, num_kv_heads: int, dtype: str,
                     tile_sizes, block_size: int = BLOCK_SIZE, rows=None):
    """The same attention through the online-softmax recurrence.

    Keys are visited in consecutive tiles whose lengths cycle through
    ``tile_sizes``.  State per (row, head): running max m (starts at -inf),
    running denominator l (starts at 0) and accumulator acc (starts at 0).
    For each tile: m_new = max(m, max S_tile); the old state is rescaled by
    e^(m - m_new) (taken as 0 while m is still -inf); P = e^(S_tile - m_new);
    l = rescale * l + sum P; acc = rescale * acc + P V_tile.  At the end
    o = acc / l and lse = m + ln l.
    """
    q = to_f64(query, dtype)
    Nt, Hq, d = q.shape
    out = np.full((Nt, Hq, d), np.nan)
    lse = np.full((Nt, Hq), np.nan)
    tile_sizes = list(tile_sizes)
    for b in range(len(seq_lens)):
        ts = _rows_of(query_start_loc, b, rows)
        if not ts:
            continue
        q_len = int(query_start_loc[b + 1]) - int(query_start_loc[b])
        seq_len = int(seq_lens[b])
        ctx = seq_len - q_len
        Kr, Vr = gather_context(k_pool, v_pool, block_tables[b], seq_len, block_size)
        K = to_f64(Kr, dtype)
        V = to_f64(Vr, dtype)
        for t in ts:
            p = ctx + (t - int(query_start_loc[b]))
            for h in range(Hq):
                kvh = kv_head_of(h, Hq, num_kv_heads)
                m, l, acc = -math.inf, 0.0, np.zeros(d)
                start, k = 0, 0
                while start <= p:
                    stop = min(start + tile_sizes[k % len(tile_sizes)], p + 1)
                    k += 1
                    s_tile = scale * (K[start:stop, kvh, :] @ q[t, h, :])
                    m_new = max(m, float(s_tile.max()))
                    rescale = 0.0 if m == -math.inf else math.exp(m - m_new)
                    pt = np.exp(s_tile - m_new)
                    l = rescale * l + float(pt.sum())
                    acc = rescale * acc + pt @ V[start:stop, kvh, :]
                    m = m_new
                    start = stop
                out[t, h, :] = acc / l
                lse[t, h] = m + math.log(l)
    return out, lse


def attention_split_partials(query, k_pool, v_pool, query_start_loc, seq_lens,
                             block_tables, scale: float, num_kv_heads: int,
                             dtype: str, num_splits: int,
                             block_size: int = BLOCK_SIZE, rows=None):
    """Split-KV partials ("Prefill has a full grid; decode at batch 1 has
    almost none").

    A request's ceil(seq_len / block_size) blocks are cut into ``num_splits``
    consecutive ranges of ceil(nblocks / num_splits) blocks (the last ranges
    may be short or empty).  Each split computes full-softmax attention over
    the visible keys in its range and reports (o_s, lse_s); a split that sees
    no key reports o_s = 0 and lse_s = -inf.

    Returns (partial_out [S, Nt, Hq, d], partial_lse [S, Nt, Hq]).
    """
    q = to_f64(query, dtype)
    Nt, Hq, d = q.shape
    po = np.full((num_splits, Nt, Hq, d), np.nan)
    pl = np.full((num_splits, Nt, Hq), np.nan)
    for b in range(len(seq_lens)):
        ts = _rows_of(query_start_loc, b, rows)
        if not ts:
            continue
        q_len = int(query_start_loc[b + 1]) - int(query_start_loc[b])
        seq_len = int(seq_lens[b])
        ctx = seq_len - q_len
        Kr, Vr = gather_context(k_pool, v_pool, block_tables[b], seq_len, block_size)
        K = to_f64(Kr, dtype)
        V = to_f64(Vr, dtype)
        nblocks = -(-seq_len // block_size)
        per = -(-nblocks // num_splits)
        for t in ts:
            p = ctx + (t - int(query_start_loc[b]))
            for s in range(num_splits):
                lo = s * per * block_size
                hi = min((s + 1) * per * block_size, p + 1)
                for h in range(Hq):
                    if lo >= hi:
                        po[s, t, h, :] = 0.0
                        pl[s, t, h] = -np.inf
                        continue
                    kvh = kv_head_of(h, Hq, num_kv_heads)
                    S = scale * (K[lo:hi, kvh, :] @ q[t, h, :])
                    m = S.max()
                    w = np.exp(S - m)
                    l = w.sum()
                    po[s, t, h, :] = (w / l) @ V[lo:hi, kvh, :]
                    pl[s, t, h] = m + math.log(l)
    return po, pl


def combine_partials(partial_out, partial_lse):
    """Merge split partials into the unsplit result.

    With M = max_s lse_s: LSE = M + ln sum_s e^(lse_s - M) and
    o = sum_s e^(lse_s - LSE) o_s.  Splits with lse_s = -inf weigh 0 (their
    o_s is never read).  An entry whose every split is -inf saw no key at
    all: its sum is empty, so LSE = ln 0 = -inf, and o (0 / 0) is NaN.
    """
    po = np.asarray(partial_out, dtype=np.float64)
    pl = np.asarray(partial_lse, dtype=np.float64)
    empty = np.isneginf(pl)
    none = empty.all(axis=0)                       # no split saw a key
    M = np.where(none, 0.0, pl.max(axis=0))        # finite reference for the sums
    w = np.where(empty, 0.0, np.exp(np.where(empty, 0.0, pl) - M[None]))
    total = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        LSE = np.where(none, -np.inf, M + np.log(np.where(none, 1.0, total)))
    coef = w / np.where(none, 1.0, total)[None]
    out = (coef[..., None] * np.where(empty[..., None], 0.0, po)).sum(axis=0)
    out = np.where(none[..., None], np.nan, out)
    return out, LSE


def attention_cascade(query, k_pool, v_pool, query_start_loc, seq_lens, block_tables,
                      scale: float, num_kv_heads: int, dtype: str, sharers, prefix_blocks,
                      block_size: int = BLOCK_SIZE):
    """Shared-prefix (cascade) attention: requests in ``sharers`` read their
    first len(prefix_blocks) blocks from the one shared list ``prefix_blocks``
    (the blocks several requests' tables point at: "Model execution",
    "Flattening a step" -- block tables may share physical blocks; "Anatomy of
    a serving engine" -- prefix caching) as a partial (o_A, lse_A) over those
    keys, and the rest of their context through their own tables as (o_B,
    lse_B); the two merge as split partials do.  Every other request is plain
    attention.  Equals ``attention`` whenever each sharer's table starts with
    ``prefix_blocks``.
    """
    out, lse = attention(query, k_pool, v_pool, query_start_loc, seq_lens, block_tables,
                         scale, num_kv_heads, dtype)
    q = to_f64(query, dtype)
    Nt, Hq, d = q.shape
    P = len(prefix_blocks)
    pref_tab = np.asarray(prefix_blocks, dtype=np.int64)
    for b in sharers:
        q_len = int(query_start_loc[b + 1]) - int(query_start_loc[b])
        if q_len == 0:
            continue
        seq_len = int(seq_lens[b])
        ctx = seq_len - q_len
        npre = min(P * block_size, seq_len)
        Ka, Va = gather_context(k_pool, v_pool, pref_tab, npre, block_size)
        Kall, Vall = gather_context(k_pool, v_pool, block_tables[b], seq_len, block_size)
        Ka, Va = to_f64(Ka, dtype), to_f64(Va, dtype)
        Kb, Vb = to_f64(Kall, dtype)[npre:], to_f64(Vall, dtype)[npre:]
        for i in range(q_len):
            t = int(query_start_loc[b]) + i
            p = ctx + i
            for h in range(Hq):
                kvh = kv_head_of(h, Hq, num_kv_heads)
                po, pl = [], []
                for K, V, lo in ((Ka, Va, 0), (Kb, Vb, npre)):
                    hi = min(K.shape[0], p + 1 - lo)
                    if hi <= 0:
                        po.append(np.zeros(d))
                        pl.append(-np.inf)
                        continue
                    S = scale * (K[:hi, kvh, :] @ q[t, h, :])
                    m = S.max()
                    w = np.exp(S - m)
                    po.append((w / w.sum()) @ V[:hi, kvh, :])
                    pl.append(m + math.log(w.sum()))
                o, L = combine_partials(np.array(po)[:, None, :], np.array(pl)[:, None])
                out[t, h, :] = o[0]
                lse[t, h] = L[0]
    return out, lse
