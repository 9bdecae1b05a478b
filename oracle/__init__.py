"""Plain fp64 CPU oracle for one flat engine step of paged attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use it.  It shares no code with the HIP path.

What it computes, and where each piece comes from (page titles from the
reference pages):

* "Model execution", section "Flattening a step": the flat metadata
  (positions, query_start_loc, seq_lens, slot_mapping, logits_indices) built
  from a schedule of (tokens already computed, tokens scheduled, block table)
  and the slot rule ``block_id * block_size + offset``.
* Same page and section: the KV write puts each new token's K and V at its
  slot; attention reads each request's context through its block table.
* "Inside the engine: kernels, CUDA graphs and the life of a request",
  section "Never materialise the T x T matrix": attention is
  softmax(S) V with S = Q K^T, computed here in full (the textbook form the
  tiled method must equal), plus the online (running m, l) recurrence of the
  same section as a self-check variant.
* Same page, section "Prefill has a full grid; decode at batch 1 has almost
  none": the split-KV partials and their combine as a self-check variant.
* ``rope``: rotary position embedding of Q and the new K fused with the
  KV write (positions as in "Flattening a step").
* ``fp8``: an FP8 (OCP E4M3) KV cache with per-KV-head scales -- the
  quantising write and attention over the dequantised pools.

Every function works in float64.  bf16 data is carried as its raw uint16 bit
pattern and widened exactly.
"""

from .paged_attention import (  # noqa: F401
    BLOCK_SIZE,
    to_f64,
    flatten_schedule,
    capture_sizes,
    validate_step,
    kv_write,
    gather_context,
    kv_head_of,
    attention,
    attention_online,
    attention_split_partials,
    combine_partials,
    attention_cascade,
)
from .rope import rope, round_to, rope_kv_write  # noqa: F401
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    e4m3_decode,
    e4m3_encode,
    quantize,
    kv_write_fp8,
    dequantize_pool,
    attention_fp8,
)
