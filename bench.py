#!/usr/bin/env python3
"""Throughput of one flat paged-attention step on one MI355X.

A step is the whole hot path over one batch of synthetic input: the KV write
of the step's new tokens through slot_mapping, then causal attention of
every scheduled row through the block tables (decode kernel with split-KV
partials merged by the last split to finish, and/or the matrix-core prefill
kernel).  The headline decode step goes through pa_decode_step, where the
decode launch performs the KV write itself; the two-call time is reported
beside it.

Headline workload: long-context single decode (1 request, 1 new token,
context 32768, 32 query / 8 KV heads, head_dim 128, bf16, 16-token blocks
scattered over a 4096-block pool).  value = algorithmic HBM bytes of a step /
wall time per step (GB/s).  Eight replicas of the inputs (separate pools)
are cycled so that no step finds its 128 MiB of K/V in the 256 MiB Infinity
Cache left by the previous one.  Steps are replayed from HIP graphs (one
graph holds one step on each replica in turn) so the host launch path is not
what is measured.

Also reported, in the same JSON line: the dominant kernel against its
roofline (durations from HIP events on the kernel's own stream, GPU kept
ahead of the host), the fp64 CPU oracle on a bounded sample of the same
workload, and the other workloads (large-batch decode, long prefill, mixed
chunked-prefill step) with their own rooflines.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attn HBM GB/s and prefill attn TFLOP/s, % of MI355X roofline"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s

WORKLOAD_NAMES = {
    2: "long-context single decode (B=1, context 32768, Hq 32/Hkv 8, d 128, bf16, 32 splits)",
    3: "large-batch decode (B=256, contexts U[512,8192], Hq 32/Hkv 8, d 128, bf16, no split)",
    4: "long prefill (4 x 8192 new tokens, causal, Hq 32/Hkv 8, d 128, bf16)",
    5: "mixed chunked-prefill step (2 x 2048-token chunks + 4096 decodes, 25% shared "
       "1024-token prefix, Hq 32/Hkv 8, d 128, bf16)",
}

# names of the per-workload rocprofv3 summaries in profiles/
PROFILE_NAMES = {2: "long_context_decode", 3: "large_batch_decode", 4: "long_prefill",
                 5: "mixed_chunked_prefill_step"}


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--eager", action="store_true", help="launch steps from Python, no graphs")
    ap.add_argument("--only-main", action="store_true", help="skip the other workloads")
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--skip-main", action="store_true",
                    help="profiling aid: run only --sections and print them (no headline line)")
    ap.add_argument("--sections", default="sweep,extra,fp8,rope,shared,shard,tiny,achievable",
                    help="comma list of the reports after the headline (profiling runs pick "
                         "a subset): sweep, extra, fp8, rope, shared, shard, tiny, "
                         "achievable")
    ap.add_argument("--profile", choices=WORKLOADS, default=None,
                    help="profiling aid: warm up and time one workload, nothing else")
    return ap.parse_args()


# ----------------------------------------------------------------------------
# algorithmic work of a step (what the method must move / compute)
# ----------------------------------------------------------------------------

def work_model(step):
    """Bytes and FLOPs the step must move/compute, independent of the kernels.

    * context K/V: every cached token a request attends to, 2 * Hkv * d * esize
      bytes, counted once per physical block (shared prefix blocks once);
    * Q read, output and lse written, block-table entries and metadata read;
    * the KV write: new K/V read and written, slot_mapping read;
    * FLOPs: 4 * d * Hq per visible (query, key) pair (QK^T and PV).
    Split partials are overhead, not counted.
    """
    import numpy as np
    es = 2 if step.dtype == "bf16" else 4
    ec = 1 if step.kv_cache == "fp8" else es      # bytes per cached element
    hq, hkv, d = step.num_q_heads, step.num_kv_heads, step.head_dim
    tok_bytes = 2 * hkv * d * ec
    tokens_in_block = {}
    table_entries = 0
    pairs = 0
    dec_tokens = 0
    pre_pairs = 0
    ql = step.q_lens
    for b in range(step.num_seqs):
        sl = int(step.seq_lens[b])
        nb = -(-sl // 16)
        table_entries += nb
        for j in range(nb):
            pb = int(step.block_tables[b, j])
            cnt = min(16, sl - 16 * j)
            if cnt > tokens_in_block.get(pb, 0):
                tokens_in_block[pb] = cnt
        q = int(ql[b])
        ctx = sl - q
        pr = q * ctx + q * (q + 1) // 2
        pairs += pr
        if q > 16 // (hq // hkv):
            pre_pairs += pr
        else:
            dec_tokens += sl
    ctx_tokens = sum(tokens_in_block.values())
    nt = int(step.query_start_loc[-1])
    kv_bytes = ctx_tokens * tok_bytes
    io = nt * hq * d * es * 2 + nt * hq * 4 + table_entries * 4 + (2 * step.num_seqs + 1) * 4
    write = nt * hkv * d * (es + ec) * 2 + nt * 8
    return {
        "bytes": kv_bytes + io + write,
        "kv_bytes": kv_bytes,
        "ctx_tokens": ctx_tokens,
        "tok_bytes": tok_bytes,
        "flops": 4.0 * d * hq * pairs,
        "prefill_flops": 4.0 * d * hq * pre_pairs,
        "pairs": pairs,
        "table_entries": table_entries,
        "q_bytes": nt * hq * d * es,
        "write_bytes": write,
    }


def decode_kernel_bytes(step):
    """Algorithmic bytes of the decode kernel alone: K/V of the decode rows'
    context (unique blocks), their Q, output/partials excluded, table reads."""
    es = 2 if step.dtype == "bf16" else 4
    ec = 1 if step.kv_cache == "fp8" else es
    hq, hkv, d = step.num_q_heads, step.num_kv_heads, step.head_dim
    dq = 16 // (hq // hkv)
    seen = {}
    entries = 0
    rows = 0
    ql = step.q_lens
    for b in range(step.num_seqs):
        if int(ql[b]) > dq or int(ql[b]) == 0:
            continue
        sl = int(step.seq_lens[b])
        nb = -(-sl // 16)
        entries += nb
        rows += int(ql[b])
        for j in range(nb):
            pb = int(step.block_tables[b, j])
            cnt = min(16, sl - 16 * j)
            if cnt > seen.get(pb, 0):
                seen[pb] = cnt
    toks = sum(seen.values())
    return toks * 2 * hkv * d * ec + rows * hq * d * es + entries * 4, toks


# ----------------------------------------------------------------------------
# step runners
# ----------------------------------------------------------------------------

class StepRunner:
    """Enqueues one step (KV write + attention) on the current stream, calling
    the C ABI directly with pre-marshalled arguments."""

    def __init__(self, step, dev, num_splits, pools=None, cascade=None, fused=False,
                 unshared=False):
        import ctypes

        import torch

        import paged_attention_flat_amd as pa
        from paged_attention_flat_amd import _lib
        self.pa, self.lib, self.ctypes, self.torch = pa, _lib.LIB, ctypes, torch
        self.step = step
        # pa_set_unshared_blocks(1) (every request taken as reading blocks
        # of its own, without the first-block test), in force for this
        # runner's launches only
        self.unshared = unshared
        g = {}
        for name in ("query", "key", "value"):
            g[name] = getattr(step, name).to(dev).contiguous()
        if pools is None:
            g["kc"] = step.k_pool.to(dev).contiguous()
            g["vc"] = step.v_pool.to(dev).contiguous()
        else:
            g["kc"], g["vc"] = pools
        g["qsl"] = torch.as_tensor(step.query_start_loc).to(dev)
        g["sl"] = torch.as_tensor(step.seq_lens).to(dev)
        g["bt"] = torch.as_tensor(step.block_tables).to(dev)
        g["sm"] = torch.as_tensor(step.slot_mapping).to(dev)
        nt, hq, d = g["query"].shape
        hkv = step.num_kv_heads
        self.splits = num_splits if num_splits > 0 else pa.choose_num_splits(
            step.num_seqs, step.max_query_len, step.max_seq_len, hq, hkv)
        g["out"] = torch.empty_like(g["query"])
        g["lse"] = torch.empty(nt, hq, dtype=torch.float32, device=dev)
        g["ws"] = pa.workspace(step.num_seqs, nt, hq, d, self.splits, device=dev)
        ws = g["ws"].numel()
        self.g = g
        code = _lib.PA_BF16 if step.dtype == "bf16" else _lib.PA_F32
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        self.fp8 = step.kv_cache == "fp8"
        if self.fp8:
            g["ks"] = step.k_scale.to(dev).contiguous()
            g["vs"] = step.v_scale.to(dev).contiguous()
            self.kv_args = [P(g["key"]), P(g["value"]), P(g["kc"]), P(g["vc"]), P(g["sm"]),
                            P(g["ks"]), P(g["vs"]), nt, hkv, d, 16, step.num_blocks, code]
            self.attn_args = [P(g["query"]), P(g["kc"]), P(g["vc"]), P(g["ks"]), P(g["vs"]),
                              P(g["qsl"]), P(g["sl"]), P(g["bt"]), step.num_seqs, nt,
                              step.max_query_len, step.max_seq_len, hq, hkv, d, 16,
                              g["bt"].shape[1], step.num_blocks, ctypes.c_float(step.scale),
                              self.splits, P(g["out"]), P(g["lse"]), P(g["ws"]), ws]
            self.kv_fn, self.attn_fn = self.lib.pa_kv_write_fp8, self.lib.pa_attention_fwd_fp8
        else:
            self.kv_args = [P(g["key"]), P(g["value"]), P(g["kc"]), P(g["vc"]), P(g["sm"]), nt,
                            hkv, d, 16, step.num_blocks, code]
            self.attn_args = [P(g["query"]), P(g["kc"]), P(g["vc"]), P(g["qsl"]), P(g["sl"]),
                              P(g["bt"]), step.num_seqs, nt, step.max_query_len,
                              step.max_seq_len, hq, hkv, d, 16, g["bt"].shape[1],
                              step.num_blocks, ctypes.c_float(step.scale), self.splits,
                              P(g["out"]), P(g["lse"]), P(g["ws"]), ws, code]
            self.kv_fn, self.attn_fn = self.lib.pa_kv_write, self.lib.pa_attention_fwd
        self.fused = fused
        if self.fused and self.fp8:
            # one call: quantising KV write + attention (pa_decode_step_fp8):
            # (key, value, caches, slots, scales, query) + attention's metadata on
            self.step_args = ([P(g["key"]), P(g["value"]), P(g["kc"]), P(g["vc"]), P(g["sm"]),
                               P(g["ks"]), P(g["vs"]), P(g["query"])] + self.attn_args[5:] +
                              [code])
            self.step_fn = self.lib.pa_decode_step_fp8
        elif self.fused:
            # one call: KV write + attention (pa_decode_step):
            # (key, value, caches, slots) + attention's arguments without its caches
            self.step_args = ([P(g["key"]), P(g["value"]), P(g["kc"]), P(g["vc"]), P(g["sm"])] +
                              self.attn_args[:1] + self.attn_args[3:])
            self.step_fn = self.lib.pa_decode_step
        if cascade is not None:
            # shared-prefix attention: (sharer request ids, prefix block ids)
            sh, pb = cascade
            g["sharers"] = torch.as_tensor(sh, dtype=torch.int32).to(dev)
            g["prefix"] = torch.as_tensor(pb, dtype=torch.int32).to(dev)
            need = self.lib.pa_cascade_workspace_size(step.num_seqs, nt, hq, hkv, d, self.splits,
                                                      g["sharers"].numel(), step.max_query_len,
                                                      g["prefix"].numel())
            g["ws"] = torch.zeros(need, dtype=torch.uint8, device=dev)
            self.attn_args = [P(g["query"]), P(g["kc"]), P(g["vc"]), P(g["qsl"]), P(g["sl"]),
                              P(g["bt"]), step.num_seqs, nt, step.max_query_len,
                              step.max_seq_len, hq, hkv, d, 16, g["bt"].shape[1],
                              step.num_blocks, ctypes.c_float(step.scale), self.splits,
                              P(g["sharers"]), g["sharers"].numel(), P(g["prefix"]),
                              g["prefix"].numel(), P(g["out"]), P(g["lse"]), P(g["ws"]), need]
            self.attn_fn = self.lib.pa_attention_fwd_cascade
            if self.fused:
                # one call: KV write + shared-prefix attention (pa_decode_step_cascade):
                # (key, value, caches, slots) + the cascade's arguments without its caches
                self.step_args = ([P(g["key"]), P(g["value"]), P(g["kc"]), P(g["vc"]),
                                   P(g["sm"])] + self.attn_args[:1] + self.attn_args[3:])
                self.step_fn = self.lib.pa_decode_step_cascade

    def __call__(self):
        if self.unshared:
            prev = self.lib.pa_set_unshared_blocks(1)
            try:
                self._launch()
            finally:
                self.lib.pa_set_unshared_blocks(prev)
        else:
            self._launch()

    def _launch(self):
        s = self.ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        if self.fused:
            st = self.step_fn(*self.step_args, s)
            if st != 0:
                raise RuntimeError(f"decode step failed: {st}")
            return
        st = self.kv_fn(*self.kv_args, s)
        if st != 0:
            raise RuntimeError(f"KV write failed: {st}")
        st = self.attn_fn(*self.attn_args, s)
        if st != 0:
            raise RuntimeError(f"attention failed: {st}")


def busy_gpu(ms):
    """Keep the GPU busy for about `ms` so that launches queued behind it run
    back-to-back (kernel events then measure GPU time, not host gaps)."""
    import torch
    try:
        torch.cuda._sleep(int(ms * 1e-3 * 2.4e9))
    except Exception:
        a = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
        for _ in range(max(1, int(ms / 0.1))):
            a = a @ a
            a = a / a.abs().max()


def time_steps(runners, steps, warmup, use_graph, log, per_graph=1):
    """Wall time of exactly `steps` steps (replicas cycled), bracketed by
    device synchronisation.  With graphs, `per_graph` consecutive steps (one
    per replica, in order) are captured into one graph; a remainder of steps
    runs from one-step graphs.  Returns (ms_per_step, launch_mode)."""
    import torch
    R = len(runners)
    mode = "eager"
    graphs = None
    per_graph = max(1, min(per_graph, R)) if use_graph else 1
    if use_graph:
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for r in runners:
                    r()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graphs = []
            for r in runners:
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    r()
                graphs.append(gr)
            chunks = []
            if per_graph > 1:
                for c0 in range(0, R - per_graph + 1, per_graph):
                    gr = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(gr):
                        for r in runners[c0:c0 + per_graph]:
                            r()
                    chunks.append(gr)
            torch.cuda.synchronize()
            mode = "hip-graph" if per_graph == 1 else f"hip-graph x{per_graph}"
        except Exception as e:  # capture unsupported: fall back, say so
            log(f"graph capture failed ({e!r}); timing eager launches")
            graphs = None
            per_graph = 1
    launch = [g.replay for g in graphs] if graphs else list(runners)

    def run(n):
        i = 0
        if per_graph > 1:
            nc = len(chunks)
            while n - i >= per_graph:
                chunks[(i // per_graph) % nc].replay()
                i += per_graph
        while i < n:
            launch[i % R]()
            i += 1

    run(warmup)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    run(steps)
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # HIP events on the stream the steps run on, bracketing the timed region
    time_steps.last_event_ms = ev0.elapsed_time(ev1) / steps
    return (t1 - t0) * 1e3 / steps, mode


def kernel_times(runners, steps, log):
    """Average duration per library kernel from HIP events recorded around
    each launch on its stream, with the GPU kept ahead of the host."""
    import torch

    import paged_attention_flat_amd as pa
    R = len(runners)
    for i in range(min(R, 4)):
        runners[i]()
    torch.cuda.synchronize()
    pa.trace_begin(8 * steps + 64)
    busy_gpu(max(20.0, steps * 0.08))
    for i in range(steps):
        runners[i % R]()
    pa.trace_end()
    torch.cuda.synchronize()
    recs = pa.trace_read()
    agg = {}
    for name, ms in recs:
        if ms < 0:
            continue
        agg.setdefault(name, []).append(1e3 * ms)
    out = {}
    for k, v in agg.items():
        v = sorted(v)
        q = lambda f: v[min(len(v) - 1, int(f * (len(v) - 1) + 0.5))]
        out[k] = {"avg_us": sum(v) / len(v), "launches": len(v), "p10_us": q(0.1),
                  "p50_us": q(0.5), "p90_us": q(0.9), "per_step_us": sum(v) / steps}
    return out


KERNELS_TIMING = ("kernels_us: the step time split over its kernels in proportion to their "
                  "HIP-event durations around traced eager launches (so they sum to "
                  "ms_per_step); kernels_us_eager_traced: those durations themselves (each "
                  "includes the events' own overhead, ~1-2 us per launch)")


def attributed_us(kt, ms):
    """The step time (ms) split over the kernels of kernel_times() in
    proportion to each kernel's traced time per step."""
    tot = sum(v["per_step_us"] for v in kt.values())
    return {k: round(v["per_step_us"] / tot * ms * 1e3, 2) for k, v in kt.items()} if tot else {}


class RopeRunner:
    """One rotary-embedding KV write of the long-prefill step's new tokens
    followed by the plain KV write of the same tokens (for comparison)."""

    def __init__(self, step, dev):
        import torch

        import paged_attention_flat_amd as pa
        self.pa = pa
        from workloads import rope_table, token_positions
        pos = torch.as_tensor(token_positions(step))
        maxp = int(pos.max()) + 1
        self.table = torch.as_tensor(rope_table(maxp, step.head_dim)).to(dev)
        self.pos = pos.to(dev)
        self.sm = torch.as_tensor(step.slot_mapping).to(dev)
        self.q = step.query.to(dev).clone()
        self.k, self.v = step.key.to(dev), step.value.to(dev)
        self.kc, self.vc = step.k_pool.to(dev), step.v_pool.to(dev)

    def __call__(self):
        self.pa.rope_kv_write(self.q, self.k, self.v, self.kc, self.vc, self.sm, self.pos,
                              self.table)
        self.pa.kv_write(self.k, self.v, self.kc, self.vc, self.sm)


# every workload a report times, by the name of its profile summary
WORKLOADS = ("long_context_decode", "large_batch_decode", "large_batch_decode_unshared",
             "large_batch_decode_fp8_unshared", "long_prefill",
             "mixed_chunked_prefill_step", "mixed_chunked_prefill_step_shared_prefix",
             "long_context_decode_fp8", "large_batch_decode_fp8", "long_prefill_fp8",
             "rope_kv_write", "shared_prefix_plain", "shared_prefix_read_once")


def workload_runners(name, dev, args, pools=None):
    """The runners of one workload exactly as its report times them.

    Returns (step, runners, per_graph, steps, warmup).  The long single decode
    cycles `args.replicas` pool replicas, one graph holding one step on each;
    the others run one step per graph.  Every plain step goes through
    pa_decode_step(_fp8), which performs the KV write inside the decode
    launch where it can and falls back to the two calls otherwise."""
    from workloads import config_step, fp8_cache, shared_prefix_step
    cfg_of = {v: k for k, v in PROFILE_NAMES.items()}
    unshared = name.endswith("_unshared")
    if unshared:
        name = name[:-len("_unshared")]
    base = name[:-4] if name.endswith("_fp8") else name
    if name.startswith("shared_prefix"):
        step = shared_prefix_step(256, 16384, 0, 512, 11, device=dev, fill="zero")
        casc = None
        if name == "shared_prefix_read_once":
            casc = (list(range(step.num_seqs)), list(step.info["shared_blocks"]))
        r = StepRunner(step, dev, 0, pools=pools, cascade=casc, fused=True)
        return step, [r], 1, args.extra_steps, 3
    if name == "rope_kv_write":
        step = config_step(4, device=dev, fill="zero")
        return step, [RopeRunner(step, dev)], 1, 20, 3
    casc = base.endswith("_shared_prefix")
    cfg = cfg_of[base[:-len("_shared_prefix")] if casc else base]
    step = config_step(cfg, device=dev, fill="zero")
    if name.endswith("_fp8"):
        step = fp8_cache(step, cfg, device=dev, fill="zero")
    if casc:
        prefix = list(step.info["shared_blocks"])
        P = len(prefix)
        bt = step.block_tables
        sharers = [b for b in range(step.num_seqs) if list(bt[b, :P]) == prefix]
        r = StepRunner(step, dev, 0, pools=pools, cascade=(sharers, prefix), fused=True)
        return step, [r], 1, args.extra_steps, 3
    first = StepRunner(step, dev, 0, pools=pools, fused=True, unshared=unshared)
    if cfg != 2:
        return step, [first], 1, args.extra_steps, 3
    runners = [first]
    for _ in range(args.replicas - 1):
        runners.append(StepRunner(step, dev, first.splits, fused=True,
                                  pools=(step.k_pool.to(dev).clone(),
                                         step.v_pool.to(dev).clone())))
    return step, runners, len(runners), args.steps, args.warmup


def profile_workload(name, args, log):
    """Warm-up plus the timed steps of one workload, nothing else (one
    rocprofv3 run per workload keeps every kernel record attributable)."""
    import torch
    dev = torch.device("cuda:0")
    step, runners, per_graph, n, warm = workload_runners(name, dev, args)
    ms, mode = time_steps(runners, n, warm, not args.eager, log, per_graph=per_graph)
    log(f"profile {name}: {ms * 1e3:.2f} us/step ({mode})")
    return {"profile": name, "ms_per_step": ms, "launch": mode, "steps": n, "warmup": warm,
            "event_ms_per_step": time_steps.last_event_ms}


def kernel_sources_sha256():
    """Hash of the kernel sources (and the ABI header) of this tree."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_attention_flat_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc)
                   if f.endswith((".hip", ".cpp", ".h")))
    for f in files + [os.path.join(ROOT, "include", "pa.h")]:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/hbm_traffic.json), or None when the kernels changed since the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256") != kernel_sources_sha256():
        return None
    k = t.get("kernels", {}).get(workload, {}).get(kernel)
    return None if k is None else k["hbm_bytes_per_launch"]


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

def bench_main(args, log):
    import torch

    dev = torch.device("cuda:0")
    # the step through pa_decode_step: KV write fused into the decode launch;
    # one graph holds one step on each replica in turn (R steps per replay)
    step, runners, per_graph, n, warm = workload_runners("long_context_decode", dev, args)
    base = runners[0]
    wm = work_model(step)
    ms, mode = time_steps(runners, n, warm, not args.eager, log, per_graph=per_graph)
    ev_ms = time_steps.last_event_ms   # one decode launch per step
    graph_ms = ms
    eager_ms = sep_ms = None
    if not args.eager:
        # the same steps launched one call at a time from the host (no graph);
        # the headline is the faster of the two launch paths (both measured
        # over the same steps, the GPU kept busy by the queued launches)
        eager_ms, _ = time_steps(runners, n, warm, False, log)
        if eager_ms < ms:
            ms, mode, ev_ms = eager_ms, "eager", time_steps.last_event_ms
        # and as two calls (pa_kv_write, pa_attention_fwd), from graphs
        sep = [StepRunner(step, dev, base.splits, pools=(r.g["kc"], r.g["vc"]))
               for r in runners]
        sep_ms, _ = time_steps(sep, args.steps, args.warmup, True, log, per_graph=len(sep))
        del sep
    kt = kernel_times(runners, min(args.steps, 200), log)
    kbytes, ktoks = decode_kernel_bytes(step)
    dom = "decode_split_partial" if base.splits > 1 else "decode"
    # each step is exactly one launch of the dominant kernel (the KV write is
    # fused into it), so its average launch duration is the event-timed
    # region over the steps; the per-launch events of kernel_times (which
    # include launch gaps) are reported in kernels_us
    dur_us = ev_ms * 1e3
    achieved = kbytes / (dur_us * 1e-6) / 1e9
    res = {
        "step": step, "ms": ms, "mode": mode, "splits": base.splits, "work": wm,
        "eager_ms": eager_ms, "sep_ms": sep_ms, "graph_ms": graph_ms,
        "kernels": kt,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": measured_traffic("long_context_decode", "decode"),
                     "bytes_per_launch": kbytes, "units_per_launch": ktoks,
                     "unit_def": "one context token of one request: K and V for 8 KV heads "
                                 "x 128 dims x 2 B = 4096 B (plus Q and table reads)",
                     "avg_launch_us": dur_us,
                     "timing": "HIP events around the timed steps of the reported launch "
                               "path, / launches",
                     "traffic_source": "not measured in this run: profiles/hbm_traffic.json "
                                       "(rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 per "
                                       "launch, scaled by a 1 GiB copy), reported only while "
                                       "the kernel sources hash to the value recorded there, "
                                       "else null"},
    }
    del runners, base
    torch.cuda.empty_cache()
    return res


def split_sweep(args, log, splits=(1, 8, 16, 32, 64, 128)):
    """Step time of the long single decode at fixed split counts (graph
    replay, the same eight rotating pool replicas as the headline)."""
    import torch

    from workloads import config_step
    dev = torch.device("cuda:0")
    step = config_step(2, device=dev, fill="zero")
    pools = [(step.k_pool, step.v_pool)]
    for _ in range(args.replicas - 1):
        pools.append((step.k_pool.clone(), step.v_pool.clone()))
    wm = work_model(step)
    out = []
    for S in splits:
        runners = [StepRunner(step, dev, S, pools=pl, fused=True) for pl in pools]
        n = args.replicas * (4 if S == 1 else 10)
        ms, _ = time_steps(runners, n, args.replicas, not args.eager, log,
                           per_graph=len(runners))
        out.append({"num_splits": S, "us_per_step": round(ms * 1e3, 2),
                    "step_GBps": round(wm["bytes"] / (ms * 1e-3) / 1e9, 1)})
        log(f"split sweep: S={S} {ms * 1e3:.2f} us/step")
        del runners
    del pools, step
    torch.cuda.empty_cache()
    return out


def bench_shard(args, log):
    """One GPU's share of the two decode workloads under 8-way tensor
    parallelism by KV head: the same requests, contexts and block placement at
    Hq 4 / Hkv 1 (an eighth of the heads and of the K/V bytes).  The long
    single decode also at fixed split counts beside the heuristic's."""
    import torch

    from workloads import config_step
    dev = torch.device("cuda:0")
    res = []
    for cfg in (2, 3):
        step = config_step(cfg, device=dev, fill="zero", scale_down={"q_heads": 4, "kv_heads": 1})
        wm = work_model(step)
        kb, _ = decode_kernel_bytes(step)
        pools = [(step.k_pool, step.v_pool)]
        if cfg == 2:
            for _ in range(args.replicas - 1):
                pools.append((step.k_pool.clone(), step.v_pool.clone()))
        rows = []
        for S in ((0, 32, 64, 128) if cfg == 2 else (0,)):
            runners = [StepRunner(step, dev, S, pools=pl, fused=True) for pl in pools]
            n = len(runners) * (20 if cfg == 2 else 5)
            ms, mode = time_steps(runners, n, len(runners), not args.eager, log,
                                  per_graph=len(runners))
            kt = kernel_times(runners, 20, log)
            name = "decode_split_partial" if runners[0].splits > 1 else "decode"
            gbs = kb / (kt[name]["avg_us"] * 1e-6) / 1e9
            rows.append({"num_splits": runners[0].splits, "heuristic": S == 0,
                         "us_per_step": round(ms * 1e3, 2), "launch": mode,
                         "step_GBps": round(wm["bytes"] / (ms * 1e-3) / 1e9, 1),
                         "decode_kernel_us": round(kt[name]["avg_us"], 2),
                         "decode_kernel_GBps": round(gbs, 1),
                         "decode_frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
            log(f"shard config{cfg}: {json.dumps(rows[-1])}")
            del runners
        res.append({"workload": WORKLOAD_NAMES[cfg] + " -- TP8 shard (Hq 4 / Hkv 1)",
                    "step_bytes": wm["bytes"], "runs": rows})
        del pools, step
        torch.cuda.empty_cache()
    return res


def achievable(log):
    """What plain library code reaches on this machine: a 1 GiB device copy
    (read + write bytes) and an 8192^3 bf16 GEMM through torch."""
    import torch
    res = {}
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 10
    res["device_copy_GBps"] = round(2 * (1 << 30) / dt / 1e9, 1)
    del src, dst
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(10):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 10
    res["gemm_bf16_8192_TFLOPps"] = round(2 * n ** 3 / dt / 1e12, 1)
    del a, b
    torch.cuda.empty_cache()
    log(f"achievable: {json.dumps(res)}")
    return res


def bench_fp8(args, log):
    """The decode and prefill workloads over an E4M3 cache (per-KV-head
    scales, codes drawn directly; the KV write quantises the new tokens).
    Algorithmic bytes count one byte per cached element."""
    import torch
    dev = torch.device("cuda:0")
    out = []
    for cfg in (2, 3, 4):
        step, runners, per_graph, n, warm = workload_runners(PROFILE_NAMES[cfg] + "_fp8", dev,
                                                             args)
        wm = work_model(step)
        ms, mode = time_steps(runners, n, warm, not args.eager, log, per_graph=per_graph)
        kt = kernel_times(runners, min(n, 200), log)
        rec = {"workload": WORKLOAD_NAMES[cfg].split(" (")[0] + ", FP8 (E4M3) KV cache",
               "ms_per_step": ms, "launch": mode, "num_splits": runners[0].splits,
               "step_GBps": wm["bytes"] / (ms * 1e-3) / 1e9,
               "kernels_us": attributed_us(kt, ms),
               "kernels_us_eager_traced": {k: round(v["avg_us"], 2) for k, v in kt.items()}}
        name = "decode_split_partial" if "decode_split_partial" in kt else "decode"
        if name in kt and cfg != 4:
            kb, _ = decode_kernel_bytes(step)
            gbs = kb / (kt[name]["avg_us"] * 1e-6) / 1e9
            rec["decode_kernel"] = {"bytes": kb, "GBps": gbs, "frac_hbm": gbs / PEAK_HBM_GBS,
                                    "traffic": measured_traffic(PROFILE_NAMES[cfg] + "_fp8",
                                                                "decode")}
        if "prefill_mfma" in kt:
            tf = wm["prefill_flops"] / (kt["prefill_mfma"]["avg_us"] * 1e-6) / 1e12
            rec["prefill_kernel"] = {"flops": wm["prefill_flops"], "TFLOPps": tf,
                                     "frac_mfma": tf / PEAK_BF16_TFLOPS,
                                     "traffic": measured_traffic(PROFILE_NAMES[cfg] + "_fp8",
                                                                 "prefill_mfma")}
        if cfg == 3:
            # under pa_set_unshared_blocks(1) (no first-block test)
            wname = PROFILE_NAMES[cfg] + "_fp8_unshared"
            _, (ru,), _, nu, wu = workload_runners(wname, dev, args,
                                                   pools=(runners[0].g["kc"], runners[0].g["vc"]))
            ums, umode = time_steps([ru], nu, wu, not args.eager, log)
            ukt = kernel_times([ru], min(nu, 20), log)
            kb, _ = decode_kernel_bytes(step)
            ugbs = kb / (ukt["decode"]["avg_us"] * 1e-6) / 1e9 if "decode" in ukt else None
            rec["all_unshared_mode"] = {
                "ms_per_step": ums, "launch": umode,
                "kernels_us": attributed_us(ukt, ums),
                "kernels_us_eager_traced": {k: round(v["avg_us"], 2) for k, v in ukt.items()},
                "decode_kernel": {"bytes": kb, "GBps": ugbs,
                                  "frac_hbm": None if ugbs is None else ugbs / PEAK_HBM_GBS,
                                  "traffic": measured_traffic(wname, "decode")}}
            del ru
        log(f"fp8 config{cfg}: {json.dumps(rec)}")
        out.append(rec)
        del runners, step
        torch.cuda.empty_cache()
    return out


def bench_rope(args, log):
    """The fused rotary embedding + KV write over the long-prefill step's
    32768 new tokens, beside the plain KV write of the same tokens.  Bytes:
    Q read and written, K and V read and written, one cos/sin row and the
    slot and position per token."""
    import torch

    import paged_attention_flat_amd as pa
    dev = torch.device("cuda:0")
    step, runners, _, n, warm = workload_runners("rope_kv_write", dev, args)
    r = runners[0]
    nt, hq, d = step.query.shape
    hkv = step.num_kv_heads
    for _ in range(warm):
        r()
    torch.cuda.synchronize()
    pa.trace_begin(4 * n)
    busy_gpu(20.0)
    for _ in range(n):
        r()
    pa.trace_end()
    torch.cuda.synchronize()
    agg = {}
    for name, ms in pa.trace_read():
        agg.setdefault(name, []).append(ms * 1e3)
    es = 2
    fused_bytes = nt * (2 * hq * d * es + 4 * hkv * d * es + d * 4 + 16)
    plain_bytes = nt * (4 * hkv * d * es + 8)
    f_us = sum(agg["rope_kv_write"]) / len(agg["rope_kv_write"])
    p_us = sum(agg["kv_write"]) / len(agg["kv_write"])
    out = {"workload": "rotary embedding + KV write of 4 x 8192 new tokens (Hq 32/Hkv 8, d 128, "
                       "bf16)",
           "fused_us": round(f_us, 2), "fused_bytes": fused_bytes,
           "fused_GBps": round(fused_bytes / (f_us * 1e-6) / 1e9, 1),
           "fused_frac_hbm": round(fused_bytes / (f_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
           "plain_kv_write_us": round(p_us, 2),
           "plain_kv_write_GBps": round(plain_bytes / (p_us * 1e-6) / 1e9, 1)}
    log(f"rope: {json.dumps(out)}")
    del step, runners, r
    torch.cuda.empty_cache()
    return out


def bench_shared_prefix(args, log):
    """256 decodes sharing a 16384-token prefix (private suffixes of 0..512
    tokens): plain attention re-reads the 64 MiB prefix per request, the
    cascade reads it once per tile of gathered rows."""
    import torch
    dev = torch.device("cuda:0")
    step, (r,), _, n, warm = workload_runners("shared_prefix_plain", dev, args)
    _, (rc,), _, _, _ = workload_runners("shared_prefix_read_once", dev, args,
                                         pools=(r.g["kc"], r.g["vc"]))
    wm = work_model(step)
    res = {"workload": "256 decodes sharing a 16384-token prefix + 0..512 private tokens "
                       "(Hq 32/Hkv 8, d 128, bf16)", "step_bytes_unique": wm["bytes"]}
    for name, run in (("plain", r), ("shared_prefix_read_once", rc)):
        ms, _ = time_steps([run], n, warm, not args.eager, log)
        kt = kernel_times([run], min(n, 20), log)
        res[name] = {"ms_per_step": ms, "step_GBps_unique": wm["bytes"] / (ms * 1e-3) / 1e9,
                     "kernels_us": attributed_us(kt, ms),
                     "kernels_us_eager_traced": {k: round(v["avg_us"], 2) for k, v in kt.items()}}
    # context: the same read-once step as two calls (pa_kv_write, then
    # pa_attention_fwd_cascade with its own setup launch)
    r2 = StepRunner(step, dev, 0, pools=(r.g["kc"], r.g["vc"]), cascade=(
        list(range(step.num_seqs)), list(step.info["shared_blocks"])), fused=False)
    ms2, _ = time_steps([r2], n, warm, not args.eager, log)
    res["shared_prefix_read_once"]["two_calls_ms_per_step"] = ms2
    log(f"shared prefix: {json.dumps(res)}")
    del r, rc, r2, step
    torch.cuda.empty_cache()
    return res


def bench_config1(args, log):
    """The tiny fp32 mixed step: GPU time per step and the oracle's
    CPU-seconds for the same step (correctness workload, no roofline)."""
    import torch

    import oracle
    from workloads import config_step, raw_numpy
    dev = torch.device("cuda:0")
    step = config_step(1, device=dev, fill="zero")
    r = StepRunner(step, dev, 0)
    ms, mode = time_steps([r], args.extra_steps, 3, not args.eager, log)
    cpu_step = config_step(1, device="cpu", fill="zero")
    t0 = time.process_time()
    kp, vp = oracle.kv_write(raw_numpy(cpu_step.key), raw_numpy(cpu_step.value),
                             raw_numpy(cpu_step.k_pool), raw_numpy(cpu_step.v_pool),
                             cpu_step.slot_mapping)
    oracle.attention(raw_numpy(cpu_step.query), kp, vp, cpu_step.query_start_loc,
                     cpu_step.seq_lens, cpu_step.block_tables, cpu_step.scale,
                     cpu_step.num_kv_heads, cpu_step.dtype)
    cpu_s = time.process_time() - t0
    out = {"workload": "tiny mixed fp32 step (prefill 37 + decodes at 5, 17, 64; Hq 4/Hkv 2, "
                       "d 64)", "us_per_step": round(ms * 1e3, 2), "launch": mode,
           "oracle_cpu_seconds": round(cpu_s, 4)}
    log(f"config1: {json.dumps(out)}")
    del r
    return out


def bench_extra(cfg, args, log):
    import torch

    dev = torch.device("cuda:0")
    step, (r,), _, n, warm = workload_runners(PROFILE_NAMES[cfg], dev, args)
    wm = work_model(step)
    ms, mode = time_steps([r], n, warm, not args.eager, log)
    kt = kernel_times([r], min(n, 20), log)
    out = {"workload": WORKLOAD_NAMES[cfg], "ms_per_step": ms, "launch": mode,
           "num_splits": r.splits, "tokens_per_s": step.num_tokens / (ms * 1e-3),
           "step_GBps": wm["bytes"] / (ms * 1e-3) / 1e9,
           "step_hbm_frac": wm["bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
           "step_TFLOPps": wm["flops"] / (ms * 1e-3) / 1e12,
           "kernels_us": attributed_us(kt, ms),
           "kernels_us_eager_traced": {k: round(v["avg_us"], 2) for k, v in kt.items()}}
    if "decode" in kt or "decode_split_partial" in kt:
        name = "decode" if "decode" in kt else "decode_split_partial"
        kb, _ = decode_kernel_bytes(step)
        gbs = kb / (kt[name]["avg_us"] * 1e-6) / 1e9
        out["decode_kernel"] = {"bytes": kb, "GBps": gbs, "frac_hbm": gbs / PEAK_HBM_GBS,
                                "traffic": measured_traffic(PROFILE_NAMES[cfg], "decode")}
    if "prefill_mfma" in kt:
        tf = wm["prefill_flops"] / (kt["prefill_mfma"]["avg_us"] * 1e-6) / 1e12
        out["prefill_kernel"] = {"flops": wm["prefill_flops"], "TFLOPps": tf,
                                 "frac_mfma": tf / PEAK_BF16_TFLOPS,
                                 "traffic": measured_traffic(PROFILE_NAMES[cfg], "prefill_mfma")}
    if "mixed_prefill_decode" in kt:
        # one persistent launch holds the step's prefill and decode work: its
        # roofline time is the larger of the decode bytes at peak HBM and the
        # prefill FLOPs at peak MFMA
        us = kt["mixed_prefill_decode"]["avg_us"]
        kb, _ = decode_kernel_bytes(step)
        t_roof = max(kb / (PEAK_HBM_GBS * 1e9), wm["prefill_flops"] / (PEAK_BF16_TFLOPS * 1e12))
        out["mixed_kernel"] = {"us": us, "decode_bytes": kb, "prefill_flops": wm["prefill_flops"],
                               "decode_GBps": kb / (us * 1e-6) / 1e9,
                               "prefill_TFLOPps": wm["prefill_flops"] / (us * 1e-6) / 1e12,
                               "roofline_frac": t_roof / (us * 1e-6),
                               "traffic": measured_traffic(PROFILE_NAMES[cfg],
                                                           "mixed_prefill_decode")}
    if cfg == 3:
        # the same step under pa_set_unshared_blocks(1): every request's V
        # streamed non-temporally without the first-block test (the default,
        # automatic policy marks all 256 requests unshared here as well)
        _, (ru,), _, nu, wu = workload_runners(PROFILE_NAMES[cfg] + "_unshared", dev, args,
                                               pools=(r.g["kc"], r.g["vc"]))
        ums, umode = time_steps([ru], nu, wu, not args.eager, log)
        ukt = kernel_times([ru], min(nu, 20), log)
        kb, _ = decode_kernel_bytes(step)
        ugbs = kb / (ukt["decode"]["avg_us"] * 1e-6) / 1e9 if "decode" in ukt else None
        out["all_unshared_mode"] = {
            "ms_per_step": ums, "launch": umode,
            "step_GBps": wm["bytes"] / (ums * 1e-3) / 1e9,
            "kernels_us": attributed_us(ukt, ums),
            "kernels_us_eager_traced": {k: round(v["avg_us"], 2) for k, v in ukt.items()},
            "decode_kernel": {"bytes": kb, "GBps": ugbs,
                              "frac_hbm": None if ugbs is None else ugbs / PEAK_HBM_GBS,
                              "traffic": measured_traffic(PROFILE_NAMES[cfg] + "_unshared",
                                                          "decode")}}
        del ru
    if cfg == 5:
        t_roof = max(wm["bytes"] / (PEAK_HBM_GBS * 1e9), wm["flops"] / (PEAK_BF16_TFLOPS * 1e12))
        out["step_roofline_frac"] = t_roof / (ms * 1e-3)
        # the same step with the shared 1024-token prefix read once
        _, (rc,), _, _, _ = workload_runners(PROFILE_NAMES[cfg] + "_shared_prefix", dev, args,
                                             pools=(r.g["kc"], r.g["vc"]))
        cms, _ = time_steps([rc], n, warm, not args.eager, log)
        ckt = kernel_times([rc], min(n, 20), log)
        # context: the same step as two calls (pa_kv_write, pa_attention_fwd_cascade)
        prefix = list(step.info["shared_blocks"])
        sharers = [b for b in range(step.num_seqs)
                   if list(step.block_tables[b, :len(prefix)]) == prefix]
        r2 = StepRunner(step, dev, 0, pools=(r.g["kc"], r.g["vc"]), cascade=(sharers, prefix),
                        fused=False)
        ms2, _ = time_steps([r2], n, warm, not args.eager, log)
        out["shared_prefix_read_once"] = {
            "sharers": int(rc.g["sharers"].numel()), "prefix_blocks": int(rc.g["prefix"].numel()),
            "ms_per_step": cms,
            "step_GBps": wm["bytes"] / (cms * 1e-3) / 1e9,
            "kernels_us": attributed_us(ckt, cms),
            "kernels_us_eager_traced": {k: round(v["avg_us"], 2) for k, v in ckt.items()},
            "two_calls_ms_per_step": ms2}
        del rc, r2
    log(f"config{cfg}: {json.dumps(out)}")
    del r
    torch.cuda.empty_cache()
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _cpu_workers():
    """Worker processes for the oracle: the host cores this process may run
    on, at most 16 (the host cores a machine with one MI355X per 16 cores
    gives each GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


ORACLE_ARRAYS = ("query", "key", "value", "k_pool", "v_pool")


def _dump_step(step, d, rows=None):
    """The step's inputs as .npy files (raw bits) for the oracle workers."""
    import numpy as np

    from workloads import raw_numpy
    os.makedirs(d, exist_ok=True)
    for n in ORACLE_ARRAYS:
        np.save(os.path.join(d, n + ".npy"), np.ascontiguousarray(raw_numpy(getattr(step, n))))
    for n in ("query_start_loc", "seq_lens", "block_tables", "slot_mapping"):
        np.save(os.path.join(d, n + ".npy"), np.asarray(getattr(step, n)))
    with open(os.path.join(d, "meta.json"), "w") as f:
        json.dump({"scale": step.scale, "num_kv_heads": step.num_kv_heads, "dtype": step.dtype,
                   "rows": None if rows is None else [int(r) for r in rows]}, f)


def _oracle_worker(task):
    """One worker process: repeat the oracle's KV write + attention (of the
    given rows, or every row) on memory-mapped inputs for about `seconds`,
    one BLAS thread.  Returns (repetitions, wall seconds)."""
    d, seconds = task
    import numpy as np
    import threadpoolctl

    import oracle
    ld = lambda n: np.load(os.path.join(d, n + ".npy"), mmap_mode="r")  # noqa: E731
    with open(os.path.join(d, "meta.json")) as f:
        meta = json.load(f)
    q, k, v, kp0, vp0 = (ld(n) for n in ORACLE_ARRAYS)
    qsl, sl, bt, sm = (np.asarray(ld(n)) for n in ("query_start_loc", "seq_lens",
                                                    "block_tables", "slot_mapping"))
    n = 0
    t0 = time.perf_counter()
    with threadpoolctl.threadpool_limits(1):
        while True:
            kp, vp = oracle.kv_write(k, v, kp0, vp0, sm)
            oracle.attention(q, kp, vp, qsl, sl, bt, meta["scale"], meta["num_kv_heads"],
                             meta["dtype"], rows=meta["rows"])
            n += 1
            if time.perf_counter() - t0 >= seconds:
                break
    return n, time.perf_counter() - t0


def _run_oracle_pool(d, workers, seconds):
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    t0 = time.perf_counter()
    with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as ex:
        res = list(ex.map(_oracle_worker, [(d, seconds)] * workers))
    wall = time.perf_counter() - t0
    return sum(r[0] for r in res), max(r[1] for r in res), wall


def cpu_baseline(args, log):
    """The fp64 oracle (as it stands) on the host cores of the machine the GPU
    sits in: N worker
    processes (one BLAS thread each, N = the cores this process may use, at
    most 16) repeat whole steps of the headline workload for about
    args.cpu_seconds, and bounded samples of the large-batch decode (16
    requests), of the long prefill (48 rows) and of the mixed step (its
    chunks with 64 decodes; decode rows and 48 chunk rows timed apart) for a
    third of that each.
    Inputs are generated on the host with the workloads' own seeds and shared
    with the workers as memory-mapped files."""
    import shutil
    import tempfile

    import numpy as np

    from workloads import config_step
    workers = _cpu_workers()
    model = _cpu_model()
    base = "/dev/shm" if os.path.isdir("/dev/shm") else None
    tmp = tempfile.mkdtemp(prefix="pa_oracle_", dir=base)
    try:
        step = config_step(2, device="cpu", fill="zero")
        wm = work_model(step)
        _dump_step(step, os.path.join(tmp, "c2"))
        del step
        n, t_work, wall = _run_oracle_pool(os.path.join(tmp, "c2"), workers, args.cpu_seconds)
        head = {"value": wm["bytes"] * n / t_work / 1e9, "unit": "GB/s", "cores": workers,
                "kind": "oracle", "cpu_model": model, "threads_per_worker": 1,
                "sample": f"{n} whole steps of the same workload (KV write + attention of the "
                          f"decode row, 32 heads x 32768 keys) in fp64 over {workers} worker "
                          f"processes, {t_work:.1f} s each ({wall:.1f} s wall incl. start-up)"}
        log(f"cpu oracle: {n} steps on {workers} workers ({model})")
        samples = {}
        # large-batch decode: 16 requests drawn like the workload's 256
        step = config_step(3, device="cpu", fill="zero", scale_down={"batch": 16})
        wm3 = work_model(step)
        _dump_step(step, os.path.join(tmp, "c3"))
        del step
        n, t_work, _ = _run_oracle_pool(os.path.join(tmp, "c3"), workers, args.cpu_seconds / 3)
        samples["large_batch_decode"] = {
            "value": wm3["bytes"] * n / t_work / 1e9, "unit": "GB/s", "cores": workers,
            "sample": f"{n} steps of 16 requests with contexts U[512, 8192] (the workload's "
                      f"draw rule; {wm3['ctx_tokens']} context tokens per step)"}
        # long prefill: the full step's KV write and 48 of its 32768 rows
        step = config_step(4, device="cpu", fill="zero")
        rng = np.random.default_rng(4)
        qsl = step.query_start_loc
        rows = sorted(set(int(x) for b in range(step.num_seqs)
                          for x in rng.integers(int(qsl[b]), int(qsl[b + 1]), 12)))
        pos = [r - int(qsl[int(np.searchsorted(qsl, r, side="right")) - 1]) for r in rows]
        flops = 4.0 * step.head_dim * step.num_q_heads * sum(p + 1 for p in pos)
        _dump_step(step, os.path.join(tmp, "c4"), rows=rows)
        del step
        n, t_work, _ = _run_oracle_pool(os.path.join(tmp, "c4"), workers, args.cpu_seconds / 3)
        samples["long_prefill"] = {
            "value": flops * n / t_work / 1e12, "unit": "TFLOP/s", "cores": workers,
            "sample": f"{n} passes of the full step's KV write (32768 tokens) plus "
                      f"attention of {len(rows)} seeded rows ({flops / 1e9:.2f} GFLOP)"}
        # mixed chunked-prefill step: its two chunks with 64 decodes drawn by
        # the workload's rule; the decode rows and 48 seeded chunk rows are
        # timed apart, and the full step is extrapolated from the two rates
        step = config_step(5, device="cpu", fill="zero", scale_down={"decodes": 64})
        qsl = np.asarray(step.query_start_loc)
        ql = np.diff(qsl)
        dec_rows = [int(qsl[b]) for b in range(step.num_seqs) if ql[b] == 1]
        chunks = [b for b in range(step.num_seqs) if ql[b] > 1]
        pre_rows = sorted(set(int(x) for b in chunks
                              for x in rng.integers(int(qsl[b]), int(qsl[b + 1]), 24)))
        pre_flops = 0.0
        for r in pre_rows:
            b = int(np.searchsorted(qsl, r, side="right")) - 1
            pos = int(step.seq_lens[b]) - int(ql[b]) + (r - int(qsl[b]))
            pre_flops += 4.0 * step.head_dim * step.num_q_heads * (pos + 1)
        dec_bytes, _ = decode_kernel_bytes(step)
        _dump_step(step, os.path.join(tmp, "c5d"), rows=dec_rows)
        _dump_step(step, os.path.join(tmp, "c5p"), rows=pre_rows)
        del step
        nd, td, _ = _run_oracle_pool(os.path.join(tmp, "c5d"), workers, args.cpu_seconds / 3)
        npf, tp, _ = _run_oracle_pool(os.path.join(tmp, "c5p"), workers, args.cpu_seconds / 3)
        dec_rate = dec_bytes * nd / td          # B/s, KV write included
        pre_rate = pre_flops * npf / tp         # FLOP/s, KV write included
        full = config_step(5, device="cpu", with_values=False)
        full_dec, _ = decode_kernel_bytes(full)
        full_pre = work_model(full)["prefill_flops"]
        del full
        est_ms = (full_dec / dec_rate + full_pre / pre_rate) * 1e3
        samples["mixed_chunked_prefill_step"] = {
            "value": est_ms, "unit": "ms per step (extrapolated)", "cores": workers,
            "decode_GBps": dec_rate / 1e9, "prefill_TFLOPps": pre_rate / 1e12,
            "sample": f"the step's two 2048-token chunks with 64 decodes drawn by the "
                      f"workload's rule: {nd} passes of the KV write plus the 64 decode rows "
                      f"and {npf} passes of the KV write plus {len(pre_rows)} seeded chunk "
                      f"rows; the full step (4096 decodes) extrapolated from the two rates"}
        head["other_workloads"] = samples
        log(f"cpu oracle samples: {json.dumps(samples)}")
        return head
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the library has no "
              "multi-GPU path (attention shards by KV head or by request with no exchange "
              "inside the step)", file=sys.stderr)
        sys.exit(2)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 copies of 1073741824 bytes")
        del src, dst
    if args.profile:
        print(json.dumps(profile_workload(args.profile, args, log)), flush=True)
        return
    if args.skip_main:
        sec = set(x.strip() for x in args.sections.split(",") if x.strip())
        part = {}
        if "fp8" in sec:
            part["fp8_kv_cache"] = bench_fp8(args, log)
        if "rope" in sec:
            part["rope_kv_write"] = bench_rope(args, log)
        if "shared" in sec:
            part["shared_prefix"] = bench_shared_prefix(args, log)
        if "shard" in sec:
            part["tensor_parallel_shard"] = bench_shard(args, log)
        if "extra" in sec:
            part["extra_workloads"] = [bench_extra(c, args, log) for c in (3, 4, 5)]
        print(json.dumps(part, default=str), flush=True)
        return
    log("main workload: " + WORKLOAD_NAMES[2])
    res = bench_main(args, log)
    wm = res["work"]
    ms = res["ms"]
    value = wm["bytes"] / (ms * 1e-3) / 1e9
    log(f"main: {ms * 1e3:.2f} us/step, {value:.1f} GB/s, kernels "
        f"{json.dumps({k: round(v['avg_us'], 2) for k, v in res['kernels'].items()})}")
    extras = []
    sweep = None
    ach = None
    cfg1 = None
    fp8 = None
    rope = None
    shared = None
    shard = None
    if not args.only_main:
        sec = set(x.strip() for x in args.sections.split(",") if x.strip())
        if "sweep" in sec:
            sweep = split_sweep(args, log)
        if "extra" in sec:
            for cfg in (3, 4, 5):
                log("extra workload: " + WORKLOAD_NAMES[cfg])
                extras.append(bench_extra(cfg, args, log))
        if "fp8" in sec:
            fp8 = bench_fp8(args, log)
        if "rope" in sec:
            rope = bench_rope(args, log)
        if "shared" in sec:
            shared = bench_shared_prefix(args, log)
        if "shard" in sec:
            shard = bench_shard(args, log)
        if "tiny" in sec:
            cfg1 = bench_config1(args, log)
        if "achievable" in sec:
            ach = achievable(log)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, log)
        # the oracle's samples beside the GPU numbers of the same workloads
        by_cfg = {3: "large_batch_decode", 4: "long_prefill", 5: "mixed_chunked_prefill_step"}
        for cfg, e in zip((3, 4, 5), extras):
            if cfg in by_cfg:
                e["oracle_cpu"] = cpu["other_workloads"][by_cfg[cfg]]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V rounded to bf16, random block placement",
        "config": {"workload": WORKLOAD_NAMES[2], "batch": 1, "context": 32768,
                   "q_heads": 32, "kv_heads": 8, "head_dim": 128, "block_size": 16,
                   "pool_blocks": 4096, "num_splits": res["splits"], "launch": res["mode"],
                   "replicas": args.replicas, "step_bytes": wm["bytes"],
                   "step_hbm_frac": value / PEAK_HBM_GBS},
        "roofline": {k: (round(v, 4) if isinstance(v, float) else v)
                     for k, v in res["roofline"].items()},
        "cpu_baseline": cpu,
        "kernels_us": attributed_us(res["kernels"], ms),
        "kernels_us_eager_traced": {k: {m: round(v[m], 2) for m in ("avg_us", "p10_us", "p50_us",
                                                                     "p90_us")}
                                    for k, v in res["kernels"].items()},
        "kernels_timing": KERNELS_TIMING,
        "launch_path": {"graph_us_per_step": round(res["graph_ms"] * 1e3, 2),
                        "eager_us_per_step": None if res["eager_ms"] is None
                        else round(res["eager_ms"] * 1e3, 2),
                        "two_calls_graph_us_per_step": None if res["sep_ms"] is None
                        else round(res["sep_ms"] * 1e3, 2)},
        "split_sweep": sweep,
        "extra_workloads": extras,
        "fp8_kv_cache": fp8,
        "rope_kv_write": rope,
        "shared_prefix": shared,
        "tensor_parallel_shard": shard,
        "correctness_workload": cfg1,
        "achievable": ach,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
