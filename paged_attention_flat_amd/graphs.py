"""HIP-graph replay of decode steps at the capture ladder's padded sizes.

"Model execution", section "Code": graphs are recorded for a ladder of batch
sizes and a step replays the graph of the smallest size that holds it, with
the extra rows padded; "Inside the engine", section "Record the launch stream
once, replay it as one operation".  A graph here holds one step of the path:
the KV write of the step's new tokens and attention for every row, which
pa_decode_step performs in a single decode launch.

Each ladder size gets its own fixed device buffers (inputs, outputs,
workspace), allocated and captured on first use.  A step is copied into the
buffers of its size (device-to-device copies on the caller's stream) with the
padding the C ABI defines for pa_capture_size: padded tokens have slot -1,
padded requests have no new tokens and no context.  Steps larger than the
top size run the same calls without a graph.  Decode steps only: every
request has exactly one new token.
"""

from __future__ import annotations

import torch

from . import (PA_BLOCK_SIZE, attention, capture_size, choose_num_splits, decode_step, kv_write,
               workspace)


class DecodeGraphs:
    def __init__(self, key_cache, value_cache, num_q_heads: int, table_stride: int,
                 scale: float, max_size: int = 512, want_lse: bool = True):
        self.kc, self.vc = key_cache, value_cache
        self.nb, self.hkv = key_cache.shape[0], key_cache.shape[1]
        self.d = key_cache.shape[3]
        self.hq = num_q_heads
        self.stride = table_stride
        self.max_seq_len = table_stride * PA_BLOCK_SIZE
        self.scale = float(scale)
        self.max_size = max_size
        self.want_lse = want_lse
        self.dev = key_cache.device
        self.dtype = key_cache.dtype
        self.graphs = {}

    def _buffers(self, P: int):
        dev, dt = self.dev, self.dtype
        b = {
            "q": torch.zeros(P, self.hq, self.d, dtype=dt, device=dev),
            "k": torch.zeros(P, self.hkv, self.d, dtype=dt, device=dev),
            "v": torch.zeros(P, self.hkv, self.d, dtype=dt, device=dev),
            "slots": torch.full((P,), -1, dtype=torch.int64, device=dev),
            "qsl": torch.zeros(P + 1, dtype=torch.int32, device=dev),
            "seq_lens": torch.zeros(P, dtype=torch.int32, device=dev),
            "tables": torch.zeros(P, self.stride, dtype=torch.int32, device=dev),
            "ramp": torch.arange(P + 1, dtype=torch.int32, device=dev),
            "out": torch.zeros(P, self.hq, self.d, dtype=dt, device=dev),
            "lse": torch.zeros(P, self.hq, dtype=torch.float32, device=dev)
            if self.want_lse else None,
        }
        b["splits"] = choose_num_splits(P, 1, self.max_seq_len, self.hq, self.hkv)
        b["ws"] = workspace(P, P, self.hq, self.d, b["splits"], device=dev)
        return b

    def _launch(self, b, P: int):
        # one launch: the decode kernel performs the KV write (pa_decode_step)
        decode_step(b["k"], b["v"], self.kc, self.vc, b["slots"], b["q"], b["qsl"],
                    b["seq_lens"], b["tables"], 1, self.max_seq_len, self.scale,
                    num_splits=b["splits"], out=b["out"], lse=b["lse"], want_lse=self.want_lse,
                    workspace=b["ws"])

    def _graph(self, P: int):
        g = self.graphs.get(P)
        if g is None:
            b = self._buffers(P)
            # warm up on a side stream (library state, allocator), then capture
            side = torch.cuda.Stream(device=self.dev)
            side.wait_stream(torch.cuda.current_stream(self.dev))
            with torch.cuda.stream(side):
                self._launch(b, P)
            torch.cuda.current_stream(self.dev).wait_stream(side)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                self._launch(b, P)
            g = (graph, b)
            self.graphs[P] = g
        return g

    def step(self, query, key, value, slot_mapping, seq_lens, block_tables):
        """One decode step of N = query.shape[0] requests (one new token each):
        write the new K/V, attend.  Returns (out[:N], lse[:N] or None); the
        views alias the size's fixed buffers until the next step of that size."""
        N = query.shape[0]
        P = capture_size(N, self.max_size)
        if P is None:
            qsl = torch.arange(N + 1, dtype=torch.int32, device=self.dev)
            kv_write(key, value, self.kc, self.vc, slot_mapping)
            return attention(query, self.kc, self.vc, qsl, seq_lens, block_tables, 1,
                             self.max_seq_len, self.scale, want_lse=self.want_lse)
        graph, b = self._graph(P)
        w = block_tables.shape[1]
        if w > self.stride:
            raise ValueError(f"block table width {w} exceeds the capture stride {self.stride}")
        b["q"][:N].copy_(query)
        b["k"][:N].copy_(key)
        b["v"][:N].copy_(value)
        b["slots"][:N].copy_(slot_mapping)
        b["slots"][N:].fill_(-1)
        torch.clamp(b["ramp"], max=N, out=b["qsl"])
        b["seq_lens"][:N].copy_(seq_lens)
        b["seq_lens"][N:].zero_()
        b["tables"][:N, :w].copy_(block_tables)
        graph.replay()
        return b["out"][:N], (b["lse"][:N] if self.want_lse else None)
