"""Host-side check of a step's flat metadata (debug aid).

The kernels read the metadata on the device and never synchronise with the
host, so they cannot check it: an out-of-range block id or a slot that breaks
the flattening rule is undefined behaviour there ("Model execution",
"Flattening a step" defines the tensors; "The runner must not synchronize"
is why the launch path does not look).  ``validate_step`` copies the metadata
to the host and reports every violation it finds.  It computes nothing of the
attention itself and is never called by the launch path.
"""

from __future__ import annotations

import numpy as np


def _host(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor, possibly on the GPU
        x = x.detach().to("cpu").numpy()
    return np.asarray(x).astype(np.int64, copy=False)


def step_problems(query_start_loc, seq_lens, block_tables, slot_mapping, num_blocks: int,
                  block_size: int = 16, max_query_len: int | None = None,
                  max_seq_len: int | None = None) -> list[str]:
    """Every inconsistency of a step's metadata, as messages (empty: valid).

    Checked: offsets start at 0, never decrease and stay within slot_mapping;
    each context holds its new tokens; the host bounds cover the step; the
    block table covers each context with block ids in [0, num_blocks); each
    scheduled token's slot is block_table[b][p / 16] * 16 + p % 16 for its
    position p; written slots are in the pool and distinct; and no block that
    receives a new token is read by another request (shared blocks must be
    read-only during the step).
    """
    qsl, sl = _host(query_start_loc), _host(seq_lens)
    bt, sm = _host(block_tables), _host(slot_mapping)
    out: list[str] = []
    B = sl.shape[0]
    if qsl.shape != (B + 1,):
        return [f"query_start_loc has {qsl.shape[0]} entries, expected num_seqs + 1 = {B + 1}"]
    if B and (bt.ndim != 2 or bt.shape[0] < B):
        return [f"block_tables shape {bt.shape} does not hold {B} requests"]
    nt = sm.shape[0]
    if qsl[0] != 0:
        out.append(f"query_start_loc[0] = {qsl[0]}, expected 0")
    bad = np.nonzero(np.diff(qsl) < 0)[0]
    if bad.size:
        out.append(f"query_start_loc decreases after request {int(bad[0])}")
    if qsl[-1] > nt:
        out.append(f"query_start_loc[-1] = {qsl[-1]} exceeds the {nt} tokens of slot_mapping")
    if out:
        return out
    q_len = np.diff(qsl)
    ctx = sl - q_len
    bad = np.nonzero(ctx < 0)[0]
    if bad.size:
        b = int(bad[0])
        out.append(f"request {b}: seq_len {sl[b]} < its {q_len[b]} new tokens")
    if max_query_len is not None and B and q_len.max() > max_query_len:
        out.append(f"max_query_len {max_query_len} < largest q_len {int(q_len.max())}")
    if max_seq_len is not None and B and sl.max() > max_seq_len:
        out.append(f"max_seq_len {max_seq_len} < largest seq_len {int(sl.max())}")
    nblk = -(-np.maximum(sl, 0) // block_size)
    if B and nblk.max() > bt.shape[1]:
        b = int(np.argmax(nblk))
        out.append(f"request {b}: {nblk[b]} blocks needed, block table has {bt.shape[1]} columns")
        return out
    # block ids of every context
    cols = np.arange(bt.shape[1] if B else 0)
    used = cols[None, :] < nblk[:, None]
    ids = bt[:B][used]
    owner = np.nonzero(used)[0]
    bad = np.nonzero((ids < 0) | (ids >= num_blocks))[0]
    if bad.size:
        out.append(f"request {int(owner[bad[0]])}: block id {int(ids[bad[0]])} "
                   f"outside [0, {num_blocks})")
        return out
    if ctx.min(initial=0) < 0:
        return out
    # the flattening rule for every scheduled token
    req = np.repeat(np.arange(B), q_len)
    tok = np.arange(int(qsl[-1]))
    pos = ctx[req] + (tok - qsl[req])
    want = bt[req, pos // block_size] * block_size + pos % block_size
    bad = np.nonzero(sm[: tok.size] != want)[0]
    if bad.size:
        t = int(bad[0])
        out.append(f"token {t} (request {int(req[t])}, position {int(pos[t])}): slot "
                   f"{int(sm[t])}, the block table gives {int(want[t])}")
    live = sm[sm >= 0]
    if live.size and live.max() >= num_blocks * block_size:
        out.append(f"slot {int(live.max())} outside the pool of {num_blocks * block_size}")
    uniq, counts = np.unique(live, return_counts=True)
    if (counts > 1).any():
        out.append(f"slot {int(uniq[counts > 1][0])} is written by more than one token")
    # a block that receives a new token must be read by its own request only
    wblk = sm[: tok.size][sm[: tok.size] >= 0] // block_size
    wreq = req[sm[: tok.size] >= 0]
    if wblk.size:
        order = np.argsort(wblk, kind="stable")
        wblk, wreq = wblk[order], wreq[order]
        hit = np.searchsorted(wblk, ids)
        inside = hit < wblk.size
        same = np.zeros_like(inside)
        same[inside] = wblk[hit[inside]] == ids[inside]
        other = same.copy()
        other[same] = wreq[hit[same]] != owner[same]
        if other.any():
            k = int(np.nonzero(other)[0][0])
            out.append(f"block {int(ids[k])} receives a new token of request "
                       f"{int(wreq[hit[k]])} but is also read by request {int(owner[k])}")
    return out


def validate_step(query_start_loc, seq_lens, block_tables, slot_mapping, num_blocks: int,
                  block_size: int = 16, max_query_len: int | None = None,
                  max_seq_len: int | None = None) -> None:
    """Raise ValueError listing every inconsistency of a step's metadata."""
    probs = step_problems(query_start_loc, seq_lens, block_tables, slot_mapping, num_blocks,
                          block_size, max_query_len, max_seq_len)
    if probs:
        raise ValueError("invalid step metadata:\n  " + "\n  ".join(probs))
