"""CPU oracle for the decode-time rotary embedding fused into the KV append.

TEST INFRASTRUCTURE ONLY (imported by ``tests/`` and never by the HIP library).

What it computes ("The prefill path: flowing the entire prompt at once", section "RoPE: a
rotation that references a table"): within each 64-wide head, element i (i < 32) is paired with
element i + 32 and the pair is rotated by the angle stored in the tables at slot 2i of the token's
position row:

    c = cos_table[pos][2i], s = sin_table[pos][2i]
    y_i      = x_i * c - x_{i+32} * s
    y_{i+32} = x_i * s + x_{i+32} * c

The page does this in FP32 on BF16 inputs and stores BF16.  The oracle takes each operation as
written, in FP32 with its own rounding (two products, then the difference or sum; no fused
multiply-add), and rounds the result to BF16 to nearest even.  Because every step is a correctly
rounded IEEE operation in the stated order, the result is a unique bit pattern and the GPU must
match it exactly.  Queries and keys are rotated; values are not.

The decode step rotates each sequence's query heads and its new key row at the sequence's absolute
position and then appends the rotated key and the unrotated value exactly like
``paged_oracle.kv_append``.  A sequence whose position has no row in the tables or no slot in the
pool is skipped entirely (the library's error rule): its q rows come back unchanged and nothing
is written to the pool.
"""

from __future__ import annotations

import numpy as np

from .paged_oracle import bf16_round_nearest_even, kv_append, slot_in_pool


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact BF16 -> FP32 (the pattern is the upper half of an FP32 pattern)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def rope_pair_index(i: int, half: int) -> int:
    """Partner of element i (< half) in the rotation: the element half a head further on."""
    return i + half


def rope_rotate(x_bits: np.ndarray, pos: int, cos_table: np.ndarray, sin_table: np.ndarray) -> np.ndarray:
    """Rotate every head of ``x_bits`` (uint16 [..., D]) at position ``pos``; returns BF16 bits."""
    x = bf16_bits_to_f32(x_bits)
    d = x.shape[-1]
    half = d // 2
    out = np.empty_like(x)
    for i in range(half):
        j = rope_pair_index(i, half)
        c = np.float32(cos_table[pos, 2 * i])
        s = np.float32(sin_table[pos, 2 * i])
        x1 = x[..., i]
        x2 = x[..., j]
        out[..., i] = np.float32(x1 * c) - np.float32(x2 * s)
        out[..., j] = np.float32(x1 * s) + np.float32(x2 * c)
    return bf16_round_nearest_even(out)


def rope_kv_append(k_pool, v_pool, block_tables, positions, q, k_new, v_new, cos_table, sin_table):
    """Decode step front half: returns (rotated q, new K pool, new V pool).

    ``q`` uint16 [B][Hq][D]; ``k_new``/``v_new`` uint16 [B][Hkv][D]; tables FP32 [rows][D].
    """
    q_out = np.array(q, copy=True)
    k_rot = np.array(k_new, copy=True)
    used = np.array(positions, dtype=np.int64, copy=True)
    for b, pos in enumerate(np.asarray(positions)):
        pos = int(pos)
        if not (0 <= pos < len(cos_table)) or not slot_in_pool(block_tables[b], pos, np.shape(k_pool)[0]):
            used[b] = -1  # the whole sequence is skipped: q_out keeps q, the pool is not written
            continue
        q_out[b] = rope_rotate(q[b], pos, cos_table, sin_table)
        k_rot[b] = rope_rotate(k_new[b], pos, cos_table, sin_table)
    k_out, v_out = kv_append(k_pool, v_pool, block_tables, used, k_rot, v_new)
    return q_out, k_out, v_out
