"""Seeded step generator.

A step is a list of requests, each with a context already in the cache
(``prior`` tokens), ``n`` tokens scheduled this step, and a block table.  The
flat metadata follows the definitions in "Model execution", section
"Flattening a step": query_start_loc are cumulative token counts, seq_lens are
prior + n, and each new token's slot is ``table[pos // 16] * 16 + pos % 16``.

Values are N(0,1) draws from a seeded ``torch.Generator`` on the device the
step is built on, rounded once to the step's dtype.  Prior-context K/V are
written straight into the pools; slots of the new tokens, the tail of each
last block and all unreferenced blocks are filled with ``fill`` (NaN for
correctness runs, so that a value that should never be read shows up).

Draw order (fixed): numpy ``default_rng(seed)`` for shapes and placement
(config-specific, see ``config_step``), then torch draws in the order query,
key, value, K pool, V pool.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

BLOCK = 16

CONFIG_NAMES = {
    1: "tiny mixed step, fp32 (Hq 4 / Hkv 2, d 64; prefill 37 + decodes at 5, 17, 64)",
    2: "long-context single decode, bf16 (1 x 32768, Hq 32 / Hkv 8, d 128)",
    3: "large-batch decode, bf16 (256 x U[512, 8192], Hq 32 / Hkv 8, d 128)",
    4: "long prefill, bf16 (4 x 8192 new tokens, Hq 32 / Hkv 8, d 128)",
    5: "mixed chunked-prefill step, bf16 (2 x 2048 chunks + 4096 decodes, 25% shared 1024-token prefix)",
}


@dataclass
class Request:
    prior: int              # tokens already in the cache
    n: int                  # tokens scheduled this step
    table: list             # physical block ids covering prior + n tokens


@dataclass
class StepInputs:
    name: str
    dtype: str                      # "bf16" or "f32"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    num_blocks: int
    query_start_loc: np.ndarray     # int32 [B+1]
    seq_lens: np.ndarray            # int32 [B]
    block_tables: np.ndarray        # int32 [B, stride], -1 past the context
    slot_mapping: np.ndarray        # int64 [Nt]
    query: torch.Tensor = None      # [Nt, Hq, d]
    key: torch.Tensor = None        # [Nt, Hkv, d]
    value: torch.Tensor = None      # [Nt, Hkv, d]
    k_pool: torch.Tensor = None     # [NB, Hkv, 16, d] before the write
    v_pool: torch.Tensor = None     # [NB, Hkv, d, 16] before the write
    info: dict = field(default_factory=dict)
    kv_cache: str = "same"          # "same" (pools in dtype) or "fp8" (E4M3 codes)
    k_scale: torch.Tensor = None    # fp8: float32 [Hkv]
    v_scale: torch.Tensor = None

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc.astype(np.int64))

    @property
    def max_query_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


def raw_numpy(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor: bf16 as its uint16 bit pattern."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def unique_block_count(step: StepInputs) -> int:
    """Number of distinct physical blocks the step's requests reference."""
    ids = []
    for b in range(step.num_seqs):
        nb = -(-int(step.seq_lens[b]) // step.block_size)
        ids.append(step.block_tables[b, :nb])
    if not ids:
        return 0
    return int(np.unique(np.concatenate(ids)).size)


def build_step(name, requests, *, dtype, num_q_heads, num_kv_heads, head_dim,
               num_blocks, seed, device="cpu", fill="nan", stride=None,
               scale=None, pad_tokens=0, order=None, info=None,
               with_values=True) -> StepInputs:
    """Flatten ``requests`` (in ``order`` if given) and draw the step's values."""
    if order is not None:
        requests = [requests[i] for i in order]
    B = len(requests)
    counts = [r.n for r in requests]
    qsl = np.zeros(B + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(counts, dtype=np.int64)
    seq_lens = np.array([r.prior + r.n for r in requests], dtype=np.int32)
    need = [-(-(r.prior + r.n) // BLOCK) for r in requests]
    if stride is None:
        stride = max(need) if need else 1
    tables = np.full((B, max(stride, 1)), -1, dtype=np.int32)
    for b, r in enumerate(requests):
        assert len(r.table) >= need[b]
        tables[b, : need[b]] = r.table[: need[b]]
    nt = int(qsl[-1]) + pad_tokens
    slots = np.full(nt, -1, dtype=np.int64)
    t = 0
    for r in requests:
        tab = np.asarray(r.table, dtype=np.int64)
        pos = np.arange(r.prior, r.prior + r.n, dtype=np.int64)
        slots[t: t + r.n] = tab[pos // BLOCK] * BLOCK + pos % BLOCK
        t += r.n
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    step = StepInputs(name=name, dtype=dtype, num_q_heads=num_q_heads,
                      num_kv_heads=num_kv_heads, head_dim=head_dim,
                      block_size=BLOCK, scale=float(scale), num_blocks=num_blocks,
                      query_start_loc=qsl, seq_lens=seq_lens, block_tables=tables,
                      slot_mapping=slots, info=dict(info or {}))
    if with_values:
        _draw_values(step, requests, seed, device, fill)
    return step


def _prior_slot_mask(step: StepInputs, requests, device) -> torch.Tensor:
    """Boolean [num_blocks * 16]: True where a prior-context token lives."""
    chunks = []
    for r in requests:
        if r.prior == 0:
            continue
        tab = torch.as_tensor(np.asarray(r.table, dtype=np.int64))
        pos = torch.arange(r.prior, dtype=torch.int64)
        chunks.append(tab[pos // BLOCK] * BLOCK + pos % BLOCK)
    mask = torch.zeros(step.num_blocks * BLOCK, dtype=torch.bool, device=device)
    if chunks:
        mask[torch.cat(chunks).to(device)] = True
    return mask


def _draw_values(step: StepInputs, requests, seed, device, fill) -> None:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    dt = step.torch_dtype
    Nt, Hq, Hkv, d = step.num_tokens, step.num_q_heads, step.num_kv_heads, step.head_dim
    NB = step.num_blocks

    def randn(*shape):
        # draw in fp32 and round once (RNE) to the step dtype
        if dt == torch.float32:
            return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
        out = torch.empty(*shape, device=device, dtype=dt)
        flat = out.view(-1)
        chunk = 1 << 28
        for s in range(0, flat.numel(), chunk):
            e = min(s + chunk, flat.numel())
            flat[s:e] = torch.randn(e - s, generator=g, device=device,
                                    dtype=torch.float32).to(dt)
        return out

    step.query = randn(Nt, Hq, d)
    step.key = randn(Nt, Hkv, d)
    step.value = randn(Nt, Hkv, d)
    step.k_pool = randn(NB, Hkv, BLOCK, d)
    step.v_pool = randn(NB, Hkv, d, BLOCK)
    live = _prior_slot_mask(step, requests, device).view(NB, BLOCK)
    dead = ~live
    fv = float("nan") if fill == "nan" else 0.0
    step.k_pool.masked_fill_(dead.view(NB, 1, BLOCK, 1), fv)
    step.v_pool.masked_fill_(dead.view(NB, 1, 1, BLOCK), fv)
    # padded tokens (slot < 0) carry poison too: they must never be read
    pad = torch.as_tensor(step.slot_mapping < 0).to(device)
    if bool(pad.any()):
        step.query[pad] = fv
        step.key[pad] = fv
        step.value[pad] = fv


def shared_prefix_step(num_requests: int, prefix_tokens: int, suffix_lo: int, suffix_hi: int,
                       seed: int, *, num_q_heads=32, num_kv_heads=8, head_dim=128,
                       dtype="bf16", device="cpu", fill="nan", with_values=True) -> StepInputs:
    """Decode requests that all share one prefix of ``prefix_tokens`` tokens
    (a multiple of 16; its blocks appear at the head of every table) followed
    by a private suffix of U[suffix_lo, suffix_hi] tokens; one new token each.
    Placement: numpy ``default_rng(seed)``; block ids a permutation of the pool
    (prefix blocks first).  info["shared_blocks"] lists the prefix blocks."""
    assert prefix_tokens % BLOCK == 0
    rng = np.random.default_rng(seed)
    P = prefix_tokens // BLOCK
    suffix = rng.integers(suffix_lo, suffix_hi + 1, size=num_requests)
    need = [-(-(prefix_tokens + int(x) + 1) // BLOCK) - P for x in suffix]
    nb = P + sum(need)
    perm = rng.permutation(nb)
    prefix = [int(x) for x in perm[:P]]
    reqs, k = [], P
    for i in range(num_requests):
        reqs.append(Request(prefix_tokens + int(suffix[i]), 1,
                            prefix + [int(x) for x in perm[k:k + need[i]]]))
        k += need[i]
    return build_step(f"shared-prefix {num_requests} x {prefix_tokens}", reqs, dtype=dtype,
                      num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                      num_blocks=nb, seed=seed, device=device, fill=fill,
                      info={"shared_blocks": prefix, "num_sharers": num_requests},
                      with_values=with_values)


def fp8_cache(step: StepInputs, seed: int, device="cpu", fill="nan") -> StepInputs:
    """The same step over an E4M3 cache: per-KV-head scales and pools of
    codes drawn directly (no quantisation here).

    Scales: k_scale[h] = 2^-5 (1 + h/4), v_scale[h] = 2^-4 (1 + h/8).  Every
    prior-context code has a random sign, an exponent field uniform in
    [3, 10] and a uniform mantissa (magnitudes 2^-4 .. 2^3.9 before scaling);
    dead slots hold the NaN code 0x7F (``fill="nan"``) or 0.  The query and
    the new tokens' K/V stay as drawn (they reach the cache through the
    quantising write).  Codes come from ``torch.Generator(seed + 1000)``: K
    pool, then V pool.
    """
    hkv = step.num_kv_heads
    h = torch.arange(hkv, dtype=torch.float32)
    k_scale = (2.0 ** -5) * (1.0 + h / 4.0)
    v_scale = (2.0 ** -4) * (1.0 + h / 8.0)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) + 1000)

    def codes(shape):
        sign = torch.randint(0, 2, shape, generator=g, device=device, dtype=torch.int32)
        e = torch.randint(3, 11, shape, generator=g, device=device, dtype=torch.int32)
        m = torch.randint(0, 8, shape, generator=g, device=device, dtype=torch.int32)
        return ((sign << 7) | (e << 3) | m).to(torch.uint8)

    NB, d = step.num_blocks, step.head_dim
    kp = codes((NB, hkv, BLOCK, d))
    vp = codes((NB, hkv, d, BLOCK))
    # prior-context slots from the metadata: positions 0 .. seq_len - q_len - 1
    chunks = []
    q_lens = step.q_lens
    for b in range(step.num_seqs):
        prior = int(step.seq_lens[b]) - int(q_lens[b])
        if prior <= 0:
            continue
        pos = np.arange(prior, dtype=np.int64)
        chunks.append(step.block_tables[b, pos // BLOCK].astype(np.int64) * BLOCK + pos % BLOCK)
    live = torch.zeros(NB * BLOCK, dtype=torch.bool, device=device)
    if chunks:
        live[torch.as_tensor(np.concatenate(chunks)).to(device)] = True
    dead = ~live.view(NB, BLOCK)
    fv = 0x7F if fill == "nan" else 0
    kp.masked_fill_(dead.view(NB, 1, BLOCK, 1), fv)
    vp.masked_fill_(dead.view(NB, 1, 1, BLOCK), fv)
    return replace(step, k_pool=kp, v_pool=vp, info=dict(step.info), kv_cache="fp8",
                   k_scale=k_scale.to(device), v_scale=v_scale.to(device))


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------

def _assign_tables(rng_perm, need_list, shared=None):
    """Hand out physical blocks from a permutation, request by request."""
    tables, k = [], 0
    for i, nb in enumerate(need_list):
        if shared is not None and shared[i] is not None:
            pre = list(shared[i])
            rest = nb - len(pre)
            tables.append(pre + list(rng_perm[k: k + rest]))
            k += rest
        else:
            tables.append(list(rng_perm[k: k + nb]))
            k += nb
    return tables, k


def config_step(cfg: int, *, device="cpu", fill="nan", variant=None,
                scale_down=None, with_values=True) -> StepInputs:
    """Build workload ``cfg`` (1..5) with seed = cfg.

    ``variant="alt"`` for config 1 reads the decode contexts as prior tokens
    (seq_lens 6, 18, 65) instead of totals (5, 17, 64).  ``scale_down`` gives
    smaller versions of configs 3-5 with the same structure, for tests the CPU
    oracle finishes in seconds: a dict of overrides (see below).  For configs 2
    and 3 it may also set ``q_heads`` / ``kv_heads``: with 4 / 1 the step is
    one GPU's share of the workload under 8-way tensor parallelism by KV head
    (same requests, contexts and block placement, one eighth of the heads).
    """
    seed = cfg
    rng = np.random.default_rng(seed)
    sd = dict(scale_down or {})
    if cfg == 1:
        dec = [6, 18, 65] if variant == "alt" else [5, 17, 64]
        shapes = [(0, 37)] + [(s - 1, 1) for s in dec]
        need = [-(-(p + n) // BLOCK) for p, n in shapes]
        perm = rng.permutation(32)
        tables, _ = _assign_tables(perm, need)
        reqs = [Request(p, n, t) for (p, n), t in zip(shapes, tables)]
        return build_step(f"config1{'-alt' if variant == 'alt' else ''}", reqs,
                          dtype="f32", num_q_heads=4, num_kv_heads=2, head_dim=64,
                          num_blocks=32, seed=seed, device=device, fill=fill,
                          scale=1.0 / math.sqrt(64), with_values=with_values)
    if cfg == 2:
        ctx = sd.get("context", 32768)
        pool = sd.get("pool_blocks", 4096)
        need = -(-ctx // BLOCK)
        table = list(rng.permutation(pool)[:need])
        reqs = [Request(ctx - 1, 1, table)]
        return build_step("config2", reqs, dtype="bf16", num_q_heads=sd.get("q_heads", 32),
                          num_kv_heads=sd.get("kv_heads", 8), head_dim=128, num_blocks=pool,
                          seed=seed,
                          device=device, fill=fill, stride=need,
                          with_values=with_values)
    if cfg == 3:
        B = sd.get("batch", 256)
        lo, hi = sd.get("lo", 512), sd.get("hi", 8192)
        ctx = rng.integers(lo, hi + 1, size=B)
        need = [-(-int(c) // BLOCK) for c in ctx]
        total = int(sum(need))
        pool = 2 * total
        perm = rng.permutation(pool)
        tables, _ = _assign_tables(perm, need)
        reqs = [Request(int(c) - 1, 1, t) for c, t in zip(ctx, tables)]
        return build_step("config3", reqs, dtype="bf16", num_q_heads=sd.get("q_heads", 32),
                          num_kv_heads=sd.get("kv_heads", 8), head_dim=128, num_blocks=pool,
                          seed=seed,
                          device=device, fill=fill, stride=-(-hi // BLOCK),
                          with_values=with_values)
    if cfg == 4:
        B = sd.get("batch", 4)
        n = sd.get("new", 8192)
        pool = sd.get("pool_blocks", 4096)
        need = [-(-n // BLOCK)] * B
        perm = rng.permutation(pool)
        tables, _ = _assign_tables(perm, need)
        reqs = [Request(0, n, t) for t in tables]
        return build_step("config4", reqs, dtype="bf16", num_q_heads=32,
                          num_kv_heads=8, head_dim=128, num_blocks=pool, seed=seed,
                          device=device, fill=fill, stride=need[0],
                          with_values=with_values)
    if cfg == 5:
        chunk = sd.get("chunk", 2048)
        priors = sd.get("priors", (4096, 16384))
        ndec = sd.get("decodes", 4096)
        lo, hi = sd.get("lo", 128), sd.get("hi", 16384)
        prefix = sd.get("prefix", 1024)
        nshare = sd.get("sharers", ndec // 4)
        stride = sd.get("stride", 1152)
        # contexts: log-uniform on [lo, hi], floored and clipped
        u = rng.uniform(math.log(lo), math.log(hi + 1), size=ndec)
        ctx = np.clip(np.floor(np.exp(u)).astype(np.int64), lo, hi)
        eligible = np.nonzero(ctx >= prefix + 1)[0]
        sharers = set(rng.choice(eligible, size=min(nshare, eligible.size),
                                 replace=False).tolist())
        shapes = [(p, chunk) for p in priors] + [(int(c) - 1, 1) for c in ctx]
        need = [-(-(p + n) // BLOCK) for p, n in shapes]
        pre_blocks = prefix // BLOCK
        unique = pre_blocks + sum(
            need[i] - (pre_blocks if (i - len(priors)) in sharers else 0)
            for i in range(len(shapes)))
        pool = int(math.ceil(1.25 * unique))
        perm = rng.permutation(pool)
        shared_ids = list(perm[:pre_blocks])
        shared = [None] * len(priors) + [
            shared_ids if j in sharers else None for j in range(ndec)]
        tables, _ = _assign_tables(perm[pre_blocks:], need, shared)
        reqs = [Request(p, n, t) for (p, n), t in zip(shapes, tables)]
        order = rng.permutation(len(reqs))
        info = {"shared_blocks": shared_ids, "num_sharers": len(sharers),
                "unique_blocks": unique}
        return build_step("config5", reqs, dtype="bf16", num_q_heads=32,
                          num_kv_heads=8, head_dim=128, num_blocks=pool, seed=seed,
                          device=device, fill=fill, stride=stride, order=order,
                          info=info, with_values=with_values)
    raise ValueError(f"no config {cfg}")


def extract_requests(step: StepInputs, req_ids, device="cpu") -> tuple:
    """A small step holding only the requests ``req_ids`` of ``step``.

    The referenced blocks are copied into a compact pool (renumbered in order
    of first use) and the metadata is rebuilt for those requests' rows only.
    Returns (small_step, token_index) where ``token_index[k]`` is the flat row
    of ``step`` that row k of the small step came from.  Values are the same
    bits as in ``step`` (pre-write pools, queries and new K/V).
    """
    req_ids = list(req_ids)
    qsl = step.query_start_loc.astype(np.int64)
    blocks, remap = [], {}
    tables, rows = [], []
    for b in req_ids:
        nb = -(-int(step.seq_lens[b]) // step.block_size)
        tab = []
        for pb in step.block_tables[b, :nb]:
            pb = int(pb)
            if pb not in remap:
                remap[pb] = len(blocks)
                blocks.append(pb)
            tab.append(remap[pb])
        tables.append(tab)
        rows.extend(range(int(qsl[b]), int(qsl[b + 1])))
    B = len(req_ids)
    stride = max(len(t) for t in tables) if tables else 1
    bt = np.full((B, stride), -1, dtype=np.int32)
    for i, t in enumerate(tables):
        bt[i, : len(t)] = t
    q_lens = [int(qsl[b + 1] - qsl[b]) for b in req_ids]
    new_qsl = np.zeros(B + 1, dtype=np.int32)
    new_qsl[1:] = np.cumsum(q_lens)
    seq_lens = step.seq_lens[req_ids].astype(np.int32)
    # rebuild slots from the renumbered tables (positions are unchanged)
    slots = np.empty(len(rows), dtype=np.int64)
    k = 0
    for i, b in enumerate(req_ids):
        ctx = int(step.seq_lens[b]) - q_lens[i]
        for j in range(q_lens[i]):
            p = ctx + j
            slots[k] = bt[i, p // BLOCK] * BLOCK + p % BLOCK
            k += 1
    idx_blocks = torch.as_tensor(np.asarray(blocks, dtype=np.int64))
    idx_rows = torch.as_tensor(np.asarray(rows, dtype=np.int64))
    src_dev = step.k_pool.device
    small = replace(
        step, name=step.name + "-extract", num_blocks=len(blocks),
        query_start_loc=new_qsl, seq_lens=seq_lens, block_tables=bt,
        slot_mapping=slots,
        query=step.query[idx_rows.to(src_dev)].to(device),
        key=step.key[idx_rows.to(src_dev)].to(device),
        value=step.value[idx_rows.to(src_dev)].to(device),
        k_pool=step.k_pool[idx_blocks.to(src_dev)].to(device),
        v_pool=step.v_pool[idx_blocks.to(src_dev)].to(device),
        info=dict(step.info))
    return small, np.asarray(rows, dtype=np.int64)


def token_positions(step: StepInputs) -> np.ndarray:
    """Position of every flat token in its own sequence ("Model execution",
    "Flattening a step": context before the step plus the row's offset);
    -1 for padded tokens."""
    pos = np.full(step.num_tokens, -1, dtype=np.int64)
    qsl = step.query_start_loc.astype(np.int64)
    for b in range(step.num_seqs):
        n = int(qsl[b + 1] - qsl[b])
        pos[qsl[b]: qsl[b + 1]] = int(step.seq_lens[b]) - n + np.arange(n)
    return pos


def rope_table(max_position: int, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """The usual rotary table, an input of the fused rotary write: float32
    [max_position, head_dim], row p = cos(p * w_i) for i < d/2, then
    sin(p * w_i), with w_i = base^(-2i/d)."""
    half = head_dim // 2
    w = base ** (-2.0 * np.arange(half, dtype=np.float64) / head_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * w[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
