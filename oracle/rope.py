"""fp64 reference for rotary position embedding fused with the KV write.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Inside the engine: kernels, CUDA graphs and the life of a request" keeps the
token positions of the flat batch "for rotary embeddings", and "Model
execution", section "Flattening a step", lists positions among the flat
tensors; neither page writes the rotation out.  Reading taken: the standard
rotary embedding with the half-split pairing -- dims i and i + d/2 of a head
form a pair rotated by the angle of (position, i):

    x'[i]       = x[i] cos - x[i + d/2] sin
    x'[i + d/2] = x[i + d/2] cos + x[i] sin

with cos / sin read from a caller-supplied float32 table [max_position, d]
(row p: cos of the d/2 angles, then their sin), so both sides use identical
angles.  The table is an input (the seeded generators build the usual one,
angle p * base^(-2i/d)); the oracle only reads it.  The fused step rotates every query head and the new keys, then writes the
rotated K and the unrotated V through slot_mapping; tokens whose position
falls outside the table are left alone (no rotation, nothing written).
"""

from __future__ import annotations

import numpy as np

from .paged_attention import BLOCK_SIZE, to_f64


def rope(x, positions, table, dtype: str) -> np.ndarray:
    """Rotate x [Nt, H, d] (bf16 bits or float32) by each token's position;
    float64 result.  Rows with a position outside the table are unchanged."""
    xf = to_f64(x, dtype)
    pos = np.asarray(positions, dtype=np.int64)
    tab = np.asarray(table, dtype=np.float32).astype(np.float64)
    d = xf.shape[-1]
    half = d // 2
    out = xf.copy()
    for t in range(xf.shape[0]):
        p = int(pos[t])
        if p < 0 or p >= tab.shape[0]:
            continue
        c, s = tab[p, :half], tab[p, half:]
        a, b = xf[t, :, :half], xf[t, :, half:]
        out[t, :, :half] = a * c - b * s
        out[t, :, half:] = b * c + a * s
    return out


def round_to(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype, to nearest even: bf16 bit
    patterns (uint16) or float32."""
    if dtype == "f32":
        return x64.astype(np.float32)
    f = x64.astype(np.float32)            # float64 -> float32 (RNE)
    bits = f.view(np.uint32).astype(np.uint64)
    # float32 -> bf16 RNE on the bit pattern (inputs here are finite)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def rope_kv_write(query, key, value, k_pool, v_pool, slot_mapping, positions, table,
                  dtype: str, block_size: int = BLOCK_SIZE):
    """(rotated query [float64], K pool, V pool): the pools after writing the
    rotated K (rounded to dtype) and V at their slots."""
    pos = np.asarray(positions, dtype=np.int64)
    qr = rope(query, pos, table, dtype)
    kr = round_to(rope(key, pos, table, dtype), dtype)
    vr = np.asarray(value)
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    for t, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        p = int(pos[t])
        if s < 0 or p < 0 or p >= table.shape[0]:
            continue
        blk, off = divmod(int(s), block_size)
        kp[blk, :, off, :] = kr[t]
        vp[blk, :, :, off] = vr[t]
    return qr, kp, vp
