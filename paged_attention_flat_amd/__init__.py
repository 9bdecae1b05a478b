"""Paged attention for one flat engine step on MI355X (gfx950).

Thin Python binding over libpa.so (include/pa.h).  PyTorch is used only for
device memory and the current stream; every step of the computation runs in
the library's HIP kernels.  The cache layouts are

    key_cache   [num_blocks, num_kv_heads, 16, head_dim]
    value_cache [num_blocks, num_kv_heads, head_dim, 16]

and the flat-batch metadata follows "Model execution", section "Flattening a
step" (query_start_loc, seq_lens, block tables, slot_mapping).
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import LIB, PA_BF16, PA_F32, PA_BLOCK_SIZE, PA_MAX_SPLITS  # noqa: F401
from .validate import step_problems, validate_step  # noqa: F401

__all__ = [
    "PaError", "kv_write", "attention", "split_combine", "workspace_size",
    "kv_write_fp8", "attention_fp8", "alloc_cache_fp8", "rope_kv_write", "attention_cascade",
    "decode_step", "decode_step_fp8", "decode_step_cascade",
    "decode_step_noalloc", "choose_num_splits", "capture_size", "alloc_cache", "workspace", "trace_begin", "trace_end",
    "trace_read",
    "kernel_name", "version", "set_unshared_blocks", "validate_step", "step_problems",
]


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = LIB.pa_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


def _check(status: int, where: str) -> None:
    if status != _lib.PA_OK:
        raise PaError(status, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float32:
        return PA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def version() -> int:
    return int(LIB.pa_version())


def set_unshared_blocks(mode) -> int:
    """pa_set_unshared_blocks: the decode rows' cache-read policy for V in
    later calls.  1 (or True): every request's blocks are its own (V streamed
    past L2/MALL); 0 (or False, the default): automatic, a request whose
    first block is no other request's first block counts as unshared; -1:
    every request's blocks count as shared.  Returns the previous mode."""
    m = int(mode)
    return int(LIB.pa_set_unshared_blocks(1 if m > 0 else (-1 if m < 0 else 0)))


def alloc_cache(num_blocks: int, num_kv_heads: int, head_dim: int, dtype, device="cuda"):
    """Allocate an (uninitialised) K and V cache pair in the library's layout."""
    k = torch.empty(num_blocks, num_kv_heads, PA_BLOCK_SIZE, head_dim, dtype=dtype,
                    device=device)
    v = torch.empty(num_blocks, num_kv_heads, head_dim, PA_BLOCK_SIZE, dtype=dtype,
                    device=device)
    return k, v


def kv_write(key, value, key_cache, value_cache, slot_mapping, stream=None) -> None:
    """Write the step's new K/V rows ([Nt, Hkv, d]) at their slots."""
    nt, hkv, d = key.shape
    if value.shape != key.shape or value.dtype != key.dtype:
        raise ValueError("key and value must match")
    if key_cache.dtype != key.dtype or value_cache.dtype != key.dtype:
        raise ValueError("cache dtype must equal the K/V dtype")
    nb = key_cache.shape[0]
    if tuple(key_cache.shape) != (nb, hkv, PA_BLOCK_SIZE, d) or \
            tuple(value_cache.shape) != (nb, hkv, d, PA_BLOCK_SIZE):
        raise ValueError("cache shapes must be [NB, Hkv, 16, d] and [NB, Hkv, d, 16]")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (nt,):
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    st = LIB.pa_kv_write(_dev(key, "key"), _dev(value, "value"), _dev(key_cache, "key_cache"),
                         _dev(value_cache, "value_cache"), _dev(slot_mapping, "slot_mapping"),
                         nt, hkv, d, PA_BLOCK_SIZE, nb, _dtype_code(key), _stream(stream))
    _check(st, "pa_kv_write")


_FP8_DTYPES = (torch.uint8,) + ((torch.float8_e4m3fn,) if hasattr(torch, "float8_e4m3fn") else ())


def _check_fp8_cache(key_cache, value_cache, hkv, d):
    nb = key_cache.shape[0]
    if key_cache.dtype not in _FP8_DTYPES or value_cache.dtype not in _FP8_DTYPES:
        raise ValueError("an FP8 cache holds E4M3 codes: uint8 or float8_e4m3fn tensors")
    if tuple(key_cache.shape) != (nb, hkv, PA_BLOCK_SIZE, d) or \
            tuple(value_cache.shape) != (nb, hkv, d, PA_BLOCK_SIZE):
        raise ValueError("cache shapes must be [NB, Hkv, 16, d] and [NB, Hkv, d, 16]")
    return nb


def _check_scales(k_scale, v_scale, hkv):
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if t.dtype != torch.float32 or tuple(t.shape) != (hkv,):
            raise ValueError(f"{name} must be float32 [num_kv_heads]")


def alloc_cache_fp8(num_blocks: int, num_kv_heads: int, head_dim: int, device="cuda"):
    """Allocate an (uninitialised) E4M3 K and V cache pair (uint8 codes)."""
    k = torch.empty(num_blocks, num_kv_heads, PA_BLOCK_SIZE, head_dim, dtype=torch.uint8,
                    device=device)
    v = torch.empty(num_blocks, num_kv_heads, head_dim, PA_BLOCK_SIZE, dtype=torch.uint8,
                    device=device)
    return k, v


def kv_write_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale,
                 stream=None) -> None:
    """Quantise the step's new K/V ([Nt, Hkv, d], bf16 or fp32) into an E4M3
    cache at their slots, with per-KV-head scales."""
    nt, hkv, d = key.shape
    if value.shape != key.shape or value.dtype != key.dtype:
        raise ValueError("key and value must match")
    nb = _check_fp8_cache(key_cache, value_cache, hkv, d)
    _check_scales(k_scale, v_scale, hkv)
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (nt,):
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    st = LIB.pa_kv_write_fp8(_dev(key, "key"), _dev(value, "value"),
                             _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
                             _dev(slot_mapping, "slot_mapping"), _dev(k_scale, "k_scale"),
                             _dev(v_scale, "v_scale"), nt, hkv, d, PA_BLOCK_SIZE, nb,
                             _dtype_code(key), _stream(stream))
    _check(st, "pa_kv_write_fp8")


def attention_fp8(query, key_cache, value_cache, k_scale, v_scale, query_start_loc, seq_lens,
                  block_tables, max_query_len: int, max_seq_len: int, scale: float,
                  num_splits: int = 0, out=None, lse=None, want_lse: bool = True,
                  workspace=None, stream=None):
    """attention() over an E4M3 cache (bf16 query and output).  Returns (out, lse)."""
    nt, hq, d = query.shape
    hkv = key_cache.shape[1]
    if query.dtype != torch.bfloat16:
        raise ValueError("an FP8 cache is read with a bf16 query")
    nb = _check_fp8_cache(key_cache, value_cache, hkv, d)
    _check_scales(k_scale, v_scale, hkv)
    for name, t in (("query_start_loc", query_start_loc), ("seq_lens", seq_lens),
                    ("block_tables", block_tables)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    ns = seq_lens.shape[0]
    if query_start_loc.shape != (ns + 1,) or block_tables.dim() != 2 or \
            block_tables.shape[0] != ns:
        raise ValueError("metadata shapes disagree")
    splits = num_splits
    if splits == 0:
        splits = choose_num_splits(ns, max_query_len, max_seq_len, hq, hkv)
    if out is None:
        out = torch.empty_like(query)
    if lse is None and want_lse:
        lse = torch.empty(nt, hq, dtype=torch.float32, device=query.device)
    need = workspace_size(ns, nt, hq, d, splits)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=query.device)
    st = LIB.pa_attention_fwd_fp8(
        _dev(query, "query"), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"),
        _dev(query_start_loc, "query_start_loc"), _dev(seq_lens, "seq_lens"),
        _dev(block_tables, "block_tables"), ns, nt, int(max_query_len), int(max_seq_len),
        hq, hkv, d, PA_BLOCK_SIZE, block_tables.shape[1], nb, float(scale), splits,
        _dev(out, "out"), None if lse is None else _dev(lse, "lse"),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "pa_attention_fwd_fp8")
    return out, lse


def _check_step_args(key, value, key_cache, value_cache, slot_mapping, query,
                     query_start_loc, seq_lens, block_tables):
    nt, hq, d = query.shape
    nb, hkv = key_cache.shape[0], key_cache.shape[1]
    if key.shape != (nt, hkv, d) or value.shape != key.shape:
        raise ValueError("key / value must be [num_tokens, num_kv_heads, head_dim]")
    if len({t.dtype for t in (query, key, value, key_cache, value_cache)}) != 1:
        raise ValueError("query, key, value and the cache must share a dtype")
    if tuple(key_cache.shape) != (nb, hkv, PA_BLOCK_SIZE, d) or \
            tuple(value_cache.shape) != (nb, hkv, d, PA_BLOCK_SIZE):
        raise ValueError("cache shapes must be [NB, Hkv, 16, d] and [NB, Hkv, d, 16]")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (nt,):
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    for name, t in (("query_start_loc", query_start_loc), ("seq_lens", seq_lens),
                    ("block_tables", block_tables)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    ns = seq_lens.shape[0]
    if query_start_loc.shape != (ns + 1,) or block_tables.dim() != 2 or \
            block_tables.shape[0] != ns:
        raise ValueError("metadata shapes disagree")
    return nt, hq, d, nb, hkv, ns


def decode_step(key, value, key_cache, value_cache, slot_mapping, query, query_start_loc,
                seq_lens, block_tables, max_query_len: int, max_seq_len: int, scale: float,
                num_splits: int = 0, out=None, lse=None, want_lse: bool = True, workspace=None,
                stream=None):
    """kv_write then attention as one call (one launch for bf16 decode steps).
    Returns (out, lse)."""
    nt, hq, d, nb, hkv, ns = _check_step_args(key, value, key_cache, value_cache, slot_mapping,
                                              query, query_start_loc, seq_lens, block_tables)
    splits = num_splits
    if splits == 0:
        splits = choose_num_splits(ns, max_query_len, max_seq_len, hq, hkv)
    if out is None:
        out = torch.empty_like(query)
    if lse is None and want_lse:
        lse = torch.empty(nt, hq, dtype=torch.float32, device=query.device)
    need = workspace_size(ns, nt, hq, d, splits)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=query.device)
    st = LIB.pa_decode_step(
        _dev(key, "key"), _dev(value, "value"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(slot_mapping, "slot_mapping"),
        _dev(query, "query"), _dev(query_start_loc, "query_start_loc"),
        _dev(seq_lens, "seq_lens"), _dev(block_tables, "block_tables"), ns, nt,
        int(max_query_len), int(max_seq_len), hq, hkv, d, PA_BLOCK_SIZE, block_tables.shape[1],
        nb, float(scale), splits, _dev(out, "out"), None if lse is None else _dev(lse, "lse"),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _dtype_code(query), _stream(stream))
    _check(st, "pa_decode_step")
    return out, lse


def decode_step_noalloc(key, value, key_cache, value_cache, slot_mapping, query,
                        query_start_loc, seq_lens, block_tables, max_query_len: int,
                        max_seq_len: int, scale: float, out, lse=None, num_splits: int = 0,
                        stream=None):
    """decode_step with the library's own per-GPU workspace: no device memory
    is allocated (out, and lse if wanted, are the caller's).  Calls that
    overlap on one GPU race.  Returns (out, lse)."""
    nt, hq, d, nb, hkv, ns = _check_step_args(key, value, key_cache, value_cache, slot_mapping,
                                              query, query_start_loc, seq_lens, block_tables)
    if out.shape != query.shape or out.dtype != query.dtype:
        raise ValueError("out must match the query")
    st = LIB.pa_decode_step_noalloc(
        _dev(key, "key"), _dev(value, "value"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(slot_mapping, "slot_mapping"),
        _dev(query, "query"), _dev(query_start_loc, "query_start_loc"),
        _dev(seq_lens, "seq_lens"), _dev(block_tables, "block_tables"), ns, nt,
        int(max_query_len), int(max_seq_len), hq, hkv, d, PA_BLOCK_SIZE, block_tables.shape[1],
        nb, float(scale), int(num_splits), _dev(out, "out"),
        None if lse is None else _dev(lse, "lse"), _dtype_code(query), _stream(stream))
    _check(st, "pa_decode_step_noalloc")
    return out, lse


def decode_step_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale, query,
                    query_start_loc, seq_lens, block_tables, max_query_len: int,
                    max_seq_len: int, scale: float, num_splits: int = 0, out=None, lse=None,
                    want_lse: bool = True, workspace=None, stream=None):
    """kv_write_fp8 then attention_fp8 as one call (one launch for decode
    steps with bf16 inputs).  Returns (out, lse)."""
    nt, hq, d = query.shape
    hkv = key_cache.shape[1]
    if query.dtype != torch.bfloat16:
        raise ValueError("an FP8 cache is read with a bf16 query")
    if key.shape != (nt, hkv, d) or value.shape != key.shape or value.dtype != key.dtype:
        raise ValueError("key / value must be [num_tokens, num_kv_heads, head_dim], one dtype")
    nb = _check_fp8_cache(key_cache, value_cache, hkv, d)
    _check_scales(k_scale, v_scale, hkv)
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (nt,):
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    for name, t in (("query_start_loc", query_start_loc), ("seq_lens", seq_lens),
                    ("block_tables", block_tables)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    ns = seq_lens.shape[0]
    splits = num_splits
    if splits == 0:
        splits = choose_num_splits(ns, max_query_len, max_seq_len, hq, hkv)
    if out is None:
        out = torch.empty_like(query)
    if lse is None and want_lse:
        lse = torch.empty(nt, hq, dtype=torch.float32, device=query.device)
    need = workspace_size(ns, nt, hq, d, splits)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=query.device)
    st = LIB.pa_decode_step_fp8(
        _dev(key, "key"), _dev(value, "value"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(slot_mapping, "slot_mapping"),
        _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale"), _dev(query, "query"),
        _dev(query_start_loc, "query_start_loc"), _dev(seq_lens, "seq_lens"),
        _dev(block_tables, "block_tables"), ns, nt, int(max_query_len), int(max_seq_len), hq,
        hkv, d, PA_BLOCK_SIZE, block_tables.shape[1], nb, float(scale), splits,
        _dev(out, "out"), None if lse is None else _dev(lse, "lse"), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _dtype_code(key), _stream(stream))
    _check(st, "pa_decode_step_fp8")
    return out, lse


def attention_cascade(query, key_cache, value_cache, query_start_loc, seq_lens, block_tables,
                      max_query_len: int, max_seq_len: int, scale: float, sharers,
                      prefix_blocks, num_splits: int = 0, out=None, lse=None,
                      want_lse: bool = True, workspace=None, stream=None):
    """attention() with a shared prefix read once: ``sharers`` (int32 request
    indices) have block tables starting with ``prefix_blocks`` (int32
    physical block ids).  bf16 only.  Returns (out, lse)."""
    nt, hq, d = query.shape
    nb, hkv = key_cache.shape[0], key_cache.shape[1]
    if query.dtype != torch.bfloat16 or key_cache.dtype != torch.bfloat16 or \
            value_cache.dtype != torch.bfloat16:
        raise ValueError("shared-prefix attention is bf16")
    if tuple(key_cache.shape) != (nb, hkv, PA_BLOCK_SIZE, d) or \
            tuple(value_cache.shape) != (nb, hkv, d, PA_BLOCK_SIZE):
        raise ValueError("cache shapes must be [NB, Hkv, 16, d] and [NB, Hkv, d, 16]")
    for name, t in (("query_start_loc", query_start_loc), ("seq_lens", seq_lens),
                    ("block_tables", block_tables), ("sharers", sharers),
                    ("prefix_blocks", prefix_blocks)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    ns = seq_lens.shape[0]
    if query_start_loc.shape != (ns + 1,) or block_tables.dim() != 2 or \
            block_tables.shape[0] != ns:
        raise ValueError("metadata shapes disagree")
    splits = num_splits
    if splits == 0:
        splits = choose_num_splits(ns, max_query_len, max_seq_len, hq, hkv)
    if out is None:
        out = torch.empty_like(query)
    if lse is None and want_lse:
        lse = torch.empty(nt, hq, dtype=torch.float32, device=query.device)
    need = int(LIB.pa_cascade_workspace_size(ns, nt, hq, hkv, d, max(1, splits),
                                             sharers.numel(), int(max_query_len),
                                             prefix_blocks.numel()))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=query.device)
    st = LIB.pa_attention_fwd_cascade(
        _dev(query, "query"), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        _dev(query_start_loc, "query_start_loc"), _dev(seq_lens, "seq_lens"),
        _dev(block_tables, "block_tables"), ns, nt, int(max_query_len), int(max_seq_len),
        hq, hkv, d, PA_BLOCK_SIZE, block_tables.shape[1], nb, float(scale), splits,
        _dev(sharers, "sharers"), sharers.numel(), _dev(prefix_blocks, "prefix_blocks"),
        prefix_blocks.numel(), _dev(out, "out"), None if lse is None else _dev(lse, "lse"),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "pa_attention_fwd_cascade")
    return out, lse


def decode_step_cascade(key, value, key_cache, value_cache, slot_mapping, query,
                        query_start_loc, seq_lens, block_tables, max_query_len: int,
                        max_seq_len: int, scale: float, sharers, prefix_blocks,
                        num_splits: int = 0, out=None, lse=None, want_lse: bool = True,
                        workspace=None, stream=None):
    """kv_write then attention_cascade as one call (bf16): the write shares
    its launch with the shared-prefix setup.  Returns (out, lse)."""
    nt, hq, d, nb, hkv, ns = _check_step_args(key, value, key_cache, value_cache, slot_mapping,
                                              query, query_start_loc, seq_lens, block_tables)
    if query.dtype != torch.bfloat16:
        raise ValueError("the shared-prefix step is bf16")
    for name, t in (("sharers", sharers), ("prefix_blocks", prefix_blocks)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    splits = num_splits
    if splits == 0:
        splits = choose_num_splits(ns, max_query_len, max_seq_len, hq, hkv)
    if out is None:
        out = torch.empty_like(query)
    if lse is None and want_lse:
        lse = torch.empty(nt, hq, dtype=torch.float32, device=query.device)
    need = int(LIB.pa_cascade_workspace_size(ns, nt, hq, hkv, d, max(1, splits),
                                             sharers.numel(), int(max_query_len),
                                             prefix_blocks.numel()))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=query.device)
    st = LIB.pa_decode_step_cascade(
        _dev(key, "key"), _dev(value, "value"), _dev(key_cache, "key_cache"),
        _dev(value_cache, "value_cache"), _dev(slot_mapping, "slot_mapping"),
        _dev(query, "query"), _dev(query_start_loc, "query_start_loc"),
        _dev(seq_lens, "seq_lens"), _dev(block_tables, "block_tables"), ns, nt,
        int(max_query_len), int(max_seq_len), hq, hkv, d, PA_BLOCK_SIZE, block_tables.shape[1],
        nb, float(scale), splits, _dev(sharers, "sharers"), sharers.numel(),
        _dev(prefix_blocks, "prefix_blocks"), prefix_blocks.numel(), _dev(out, "out"),
        None if lse is None else _dev(lse, "lse"), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "pa_decode_step_cascade")
    return out, lse


def rope_kv_write(query, key, value, key_cache, value_cache, slot_mapping, positions, cos_sin,
                  stream=None) -> None:
    """Rotate query ([Nt, Hq, d], in place) and the new keys by each token's
    position (cos_sin: float32 [max_position, d], cos then sin of the d/2
    angles), writing the rotated K and V at their slots."""
    nt, hkv, d = key.shape
    hq = query.shape[1]
    if value.shape != key.shape or value.dtype != key.dtype or query.dtype != key.dtype:
        raise ValueError("query, key and value must share a dtype; key and value a shape")
    if tuple(query.shape) != (nt, hq, d):
        raise ValueError("query must be [num_tokens, num_q_heads, head_dim]")
    nb = key_cache.shape[0]
    if tuple(key_cache.shape) != (nb, hkv, PA_BLOCK_SIZE, d) or \
            tuple(value_cache.shape) != (nb, hkv, d, PA_BLOCK_SIZE):
        raise ValueError("cache shapes must be [NB, Hkv, 16, d] and [NB, Hkv, d, 16]")
    if key_cache.dtype != key.dtype or value_cache.dtype != key.dtype:
        raise ValueError("cache dtype must equal the K/V dtype")
    for name, t in (("slot_mapping", slot_mapping), ("positions", positions)):
        if t.dtype != torch.int64 or t.shape != (nt,):
            raise ValueError(f"{name} must be int64 [num_tokens]")
    if cos_sin.dtype != torch.float32 or cos_sin.dim() != 2 or cos_sin.shape[1] != d:
        raise ValueError("cos_sin must be float32 [max_position, head_dim]")
    st = LIB.pa_rope_kv_write(_dev(query, "query"), _dev(key, "key"), _dev(value, "value"),
                              _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
                              _dev(slot_mapping, "slot_mapping"), _dev(positions, "positions"),
                              _dev(cos_sin, "cos_sin"), cos_sin.shape[0], nt, hq, hkv, d,
                              PA_BLOCK_SIZE, nb, _dtype_code(key), _stream(stream))
    _check(st, "pa_rope_kv_write")


def workspace_size(num_seqs: int, num_tokens: int, num_q_heads: int, head_dim: int,
                   num_splits: int) -> int:
    return int(LIB.pa_attention_workspace_size(num_seqs, num_tokens, num_q_heads, head_dim,
                                               max(1, num_splits)))


def choose_num_splits(num_seqs: int, max_query_len: int, max_seq_len: int, num_q_heads: int,
                      num_kv_heads: int, num_cus: int = 0) -> int:
    return int(LIB.pa_choose_num_splits(num_seqs, max_query_len, max_seq_len, num_q_heads,
                                        num_kv_heads, num_cus))


def capture_size(num_tokens: int, max_size: int = 512):
    """Ladder size a step of num_tokens is replayed at, or None (no graph)."""
    n = int(LIB.pa_capture_size(int(num_tokens), int(max_size)))
    return None if n < 0 else n


def attention(query, key_cache, value_cache, query_start_loc, seq_lens, block_tables,
              max_query_len: int, max_seq_len: int, scale: float, num_splits: int = 0,
              out=None, lse=None, want_lse: bool = True, workspace=None, stream=None):
    """Causal paged attention for every scheduled row.  Returns (out, lse)."""
    nt, hq, d = query.shape
    nb, hkv = key_cache.shape[0], key_cache.shape[1]
    if tuple(key_cache.shape) != (nb, hkv, PA_BLOCK_SIZE, d) or \
            tuple(value_cache.shape) != (nb, hkv, d, PA_BLOCK_SIZE):
        raise ValueError("cache shapes must be [NB, Hkv, 16, d] and [NB, Hkv, d, 16]")
    if key_cache.dtype != query.dtype or value_cache.dtype != query.dtype:
        raise ValueError("cache dtype must equal the query dtype")
    for name, t in (("query_start_loc", query_start_loc), ("seq_lens", seq_lens),
                    ("block_tables", block_tables)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    ns = seq_lens.shape[0]
    if query_start_loc.shape != (ns + 1,) or block_tables.dim() != 2 or \
            block_tables.shape[0] != ns:
        raise ValueError("metadata shapes disagree")
    splits = num_splits
    if splits == 0:
        splits = choose_num_splits(ns, max_query_len, max_seq_len, hq, hkv)
    if out is None:
        out = torch.empty_like(query)
    if lse is None and want_lse:
        lse = torch.empty(nt, hq, dtype=torch.float32, device=query.device)
    need = workspace_size(ns, nt, hq, d, splits)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        # zero-filled: the split-merge counters must start at zero
        workspace = torch.zeros(need, dtype=torch.uint8, device=query.device)
    st = LIB.pa_attention_fwd(
        _dev(query, "query"), _dev(key_cache, "key_cache"), _dev(value_cache, "value_cache"),
        _dev(query_start_loc, "query_start_loc"), _dev(seq_lens, "seq_lens"),
        _dev(block_tables, "block_tables"), ns, nt, int(max_query_len), int(max_seq_len),
        hq, hkv, d, PA_BLOCK_SIZE, block_tables.shape[1], nb, float(scale), splits,
        _dev(out, "out"), None if lse is None else _dev(lse, "lse"),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _dtype_code(query), _stream(stream))
    _check(st, "pa_attention_fwd")
    return out, lse


def split_combine(partial_out, partial_lse, out=None, lse=None, dtype=torch.bfloat16,
                  stream=None):
    """Merge [S, Nt, Hq, d] fp32 partials and their [S, Nt, Hq] lse."""
    s, nt, hq, d = partial_out.shape
    if partial_out.dtype != torch.float32 or partial_lse.dtype != torch.float32 or \
            tuple(partial_lse.shape) != (s, nt, hq):
        raise ValueError("partials must be float32 [S, Nt, Hq, d] and [S, Nt, Hq]")
    if out is None:
        out = torch.empty(nt, hq, d, dtype=dtype, device=partial_out.device)
    if lse is None:
        lse = torch.empty(nt, hq, dtype=torch.float32, device=partial_out.device)
    st = LIB.pa_split_combine(_dev(partial_out, "partial_out"), _dev(partial_lse, "partial_lse"),
                              s, nt, hq, d, _dev(out, "out"), _dev(lse, "lse"),
                              _dtype_code(out), _stream(stream))
    _check(st, "pa_split_combine")
    return out, lse


def workspace(num_seqs: int, num_tokens: int, num_q_heads: int, head_dim: int,
              num_splits: int, device="cuda", stream=None):
    """A ready-to-use attention workspace (counters zeroed by the library)."""
    n = workspace_size(num_seqs, num_tokens, num_q_heads, head_dim, num_splits)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device=device)
    _check(LIB.pa_attention_workspace_init(_dev(ws, "workspace"), ws.numel(), _stream(stream)),
           "pa_attention_workspace_init")
    return ws


def trace_begin(capacity: int = 4096) -> None:
    _check(LIB.pa_trace_begin(capacity), "pa_trace_begin")


def trace_end() -> None:
    _check(LIB.pa_trace_end(), "pa_trace_end")


def kernel_name(kid: int) -> str:
    return LIB.pa_kernel_name(kid).decode()


def trace_read(capacity: int = 1 << 16):
    """[(kernel_name, milliseconds)] of the launches recorded since
    trace_begin.  Synchronise the device first."""
    ids = (ctypes.c_int32 * capacity)()
    ms = (ctypes.c_float * capacity)()
    n = LIB.pa_trace_read(ids, ms, capacity)
    if n < 0:
        raise PaError(_lib.PA_ERR_INVALID, "pa_trace_read")
    return [(kernel_name(ids[i]), float(ms[i])) for i in range(n)]
