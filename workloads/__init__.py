"""Seeded synthetic inputs for one flat paged-attention step.

This package only draws inputs: request shapes, block placement, the flat
metadata of the step, and N(0,1) values for Q, the new K/V and the cached
context (or, for an FP8 cache, per-head scales and directly drawn codes).  It holds none of the attention arithmetic.  Both the tests (which
feed the CPU oracle and the HIP library the same inputs) and ``bench.py`` use
it; it imports neither side.
"""

from .gen import (  # noqa: F401
    Request,
    StepInputs,
    build_step,
    config_step,
    CONFIG_NAMES,
    raw_numpy,
    extract_requests,
    unique_block_count,
    fp8_cache,
    shared_prefix_step,
    token_positions,
    rope_table,
)
