"""FP64 CPU oracle for paged KV append and paged decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this module.  The HIP library never calls it and shares no code with
it; the two meet only through the seeded inputs of the ``workloads`` package.

What it computes, in the plainest reading of the pages:

* **Append** ("6 Hours of YouTube and 85 handtyped pages of notes on LLM Inference", section "What works so far": decode appends one new token at its absolute
  position into a shared BF16 page pool; "The prefill path: flowing the entire prompt at once", section "Distributing K/V
  into paged blocks": logical block ``pos // 16`` is looked up in the block table).  The new
  pool equals the old one except that slot ``pos % 16`` of page ``table[pos // 16]`` holds the
  new row, for every KV head.  Pure bit copy, applied in batch order.
* **Attention** ("6 Hours of YouTube and 85 handtyped pages of notes on LLM Inference", section "What works so far": each query head streams its sequence's
  pages; "The prefill path: flowing the entire prompt at once", sections "Per-head attention scores and GQA" and
  "causalMask and online softmax").  The oracle does what the GPU path must avoid: it gathers
  the ``L`` cached tokens into a contiguous prefix, upcasts BF16 exactly to FP64, and runs a
  two-pass softmax per query head, with query head ``h`` reading KV head ``h // 4`` and the
  score scale ``1/sqrt(64) = 1/8``.

Pool layout: ``[page][kv_head][token_in_page][dim]`` for K and V separately.

Out-of-range inputs (the pages assume none) follow the library's error rule: an append row whose
position lies outside the table's span or whose entry names no page of the pool is not written,
and a sequence whose context does not map to pages of the pool gets an all-zero output.

Every oracle function is pinned by ``tests/test_oracle_pins.py`` against closed forms, an
independent brute-force implementation, invariants and ``torch`` scaled-dot-product attention.
"""

from __future__ import annotations

import math

import numpy as np

BLOCK_SIZE = 16


# --------------------------------------------------------------------------------------------
# BF16 <-> wider floats
# --------------------------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact BF16 -> FP64: a BF16 pattern is the upper half of an FP32 pattern."""
    wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


def bf16_round_nearest_even(x: np.ndarray) -> np.ndarray:
    """Round FP32 values to BF16 bit patterns, ties to even, by comparing both neighbours.

    For each finite value the two candidates are the truncated pattern and the next pattern away
    from zero; the nearer one wins and an exact tie picks the one with an even last bit.  Used by
    the tests to state what the BF16 output store must equal.
    """
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    bits = x32.view(np.uint32)
    lo = (bits >> np.uint32(16)).astype(np.uint32)  # truncation toward zero
    hi = lo + np.uint32(1)
    lo_val = (lo << np.uint32(16)).view(np.float32).astype(np.float64)
    hi_val = (hi << np.uint32(16)).view(np.float32).astype(np.float64)
    exact = x32.astype(np.float64)
    # Past the largest finite BF16 the next candidate is infinity; IEEE rounding measures the
    # distance to it as if the exponent range continued, i.e. to +-2^128.
    hi_val = np.where(np.isinf(hi_val) & np.isfinite(exact), np.copysign(2.0**128, exact), hi_val)
    d_lo = np.abs(exact - lo_val)
    d_hi = np.abs(hi_val - exact)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo & np.uint32(1)) == np.uint32(1)))
    out = np.where(pick_hi, hi, lo).astype(np.uint16)
    out[np.isnan(x32)] = np.uint16(0x7FC0)
    return out


# --------------------------------------------------------------------------------------------
# Append
# --------------------------------------------------------------------------------------------

def locate_slot(block_table_row: np.ndarray, pos: int) -> tuple[int, int]:
    """Physical (page, slot) of absolute token position ``pos`` through one block-table row."""
    return int(block_table_row[pos // BLOCK_SIZE]), pos % BLOCK_SIZE


# The pages assume valid inputs.  For the rest this oracle follows the library's error rule: a row
# whose position lies outside the table's span, or whose table entry names no page of the pool, is
# not written; a sequence whose context cannot be read that way gets an all-zero output.  (Python's
# negative indexing would otherwise turn position -1 or entry -1 into the last slot or page.)

def slot_in_pool(block_table_row: np.ndarray, pos: int, num_pages: int) -> bool:
    """Whether position ``pos`` maps through the row to a slot of a pool of ``num_pages`` pages."""
    if pos < 0 or pos >= len(block_table_row) * BLOCK_SIZE:
        return False
    return 0 <= int(block_table_row[pos // BLOCK_SIZE]) < num_pages


def context_in_pool(block_table_row: np.ndarray, length: int, num_pages: int) -> bool:
    """Whether positions ``0 .. length - 1`` all map to slots of the pool (``length`` 0 is valid)."""
    if length < 0 or length > len(block_table_row) * BLOCK_SIZE:
        return False
    entries = np.asarray(block_table_row[:(length + BLOCK_SIZE - 1) // BLOCK_SIZE], dtype=np.int64)
    return bool(np.all((entries >= 0) & (entries < num_pages)))


def kv_append(k_pool, v_pool, block_tables, positions, k_new, v_new):
    """Return copies of the pools with every sequence's new K/V row written at its position.

    ``k_pool``/``v_pool``: uint16 [P][Hkv][16][D]; ``block_tables``: int32 [B][T];
    ``positions``: [B]; ``k_new``/``v_new``: uint16 [B][Hkv][D].
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for b in range(len(positions)):
        if not slot_in_pool(block_tables[b], int(positions[b]), k_out.shape[0]):
            continue  # skipped, not written
        page, slot = locate_slot(block_tables[b], int(positions[b]))
        k_out[page, :, slot, :] = k_new[b]
        v_out[page, :, slot, :] = v_new[b]
    return k_out, v_out


# --------------------------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------------------------

def kv_head_of(q_head: int, group: int) -> int:
    """Grouped-query mapping: consecutive blocks of ``group`` query heads share one KV head."""
    return q_head // group


def gather_context(pool: np.ndarray, block_table_row: np.ndarray, length: int) -> np.ndarray:
    """Contiguous prefix [L][Hkv][D] of a sequence's cached rows, read through its block table."""
    n_pages = (length + BLOCK_SIZE - 1) // BLOCK_SIZE
    pages = np.asarray(block_table_row[:n_pages], dtype=np.int64)
    blocks = pool[pages]  # [n][Hkv][16][D]
    tokens = blocks.transpose(0, 2, 1, 3).reshape(n_pages * BLOCK_SIZE, pool.shape[1], pool.shape[3])
    return tokens[:length]


def softmax_two_pass(scores: np.ndarray) -> np.ndarray:
    """exp(x - max) / sum exp(x - max) along the last axis, in FP64."""
    m = scores.max(axis=-1, keepdims=True)
    w = np.exp(scores - m)
    return w / w.sum(axis=-1, keepdims=True)


def attend_one(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """Decode attention of one sequence.  q [Hq][D], keys/values [L][Hkv][D] (FP64)."""
    hq, d = q.shape
    group = hq // keys.shape[1]
    out = np.empty((hq, d), dtype=np.float64)
    for h in range(hq):
        g = kv_head_of(h, group)
        scores = (keys[:, g, :] @ q[h]) * scale
        probs = softmax_two_pass(scores)
        out[h] = probs @ values[:, g, :]
    return out


def paged_decode_attention(q, k_pool, v_pool, block_tables, context_lens, scale=0.125, sequences=None):
    """FP64 attention output [B][Hq][D] for a decode batch (context 0, or a context that does not
    map to pages of the pool, gives zeros).

    ``q``: uint16 [B][Hq][D]; pools uint16 [P][Hkv][16][D]; ``block_tables`` int32 [B][T];
    ``context_lens`` [B] counts the appended token.  ``sequences`` optionally restricts the work to
    some batch rows (other rows are left as NaN) so a large batch can be sampled.
    """
    q = np.asarray(q)
    batch, hq, d = q.shape
    out = np.full((batch, hq, d), np.nan, dtype=np.float64)
    rows = range(batch) if sequences is None else sequences
    for b in rows:
        L = int(context_lens[b])
        if L == 0 or not context_in_pool(block_tables[b], L, k_pool.shape[0]):
            out[b] = 0.0
            continue
        keys = bf16_bits_to_f64(gather_context(k_pool, block_tables[b], L))
        values = bf16_bits_to_f64(gather_context(v_pool, block_tables[b], L))
        out[b] = attend_one(bf16_bits_to_f64(q[b]), keys, values, scale)
    return out


# --------------------------------------------------------------------------------------------
# Test-only variant: online softmax with the pairwise merge rule
# --------------------------------------------------------------------------------------------

def merge_states(a, b):
    """Combine two (max, denominator, weighted-sum) softmax states over disjoint token sets.

    Both are re-anchored to the larger maximum: m = max(ma, mb), d = da*e^(ma-m) + db*e^(mb-m)
    ("The prefill path: flowing the entire prompt at once", section "causalMask and online softmax"); the weighted value
    sums are re-anchored the same way.  An empty state has d == 0 and is the identity.
    """
    ma, da, oa = a
    mb, db, ob = b
    if da == 0.0:
        return b
    if db == 0.0:
        return a
    m = max(ma, mb)
    ea, eb = math.exp(ma - m), math.exp(mb - m)
    return m, da * ea + db * eb, oa * ea + ob * eb


def attend_one_online(q, keys, values, scale, boundaries):
    """Like :func:`attend_one`, but each head's tokens are cut at ``boundaries`` into chunks,
    each chunk is reduced to its own (max, denominator, weighted sum) and the chunks are folded
    with :func:`merge_states`."""
    hq, d = q.shape
    L = keys.shape[0]
    group = hq // keys.shape[1]
    cuts = [0] + [int(c) for c in boundaries if 0 < int(c) < L] + [L]
    out = np.empty((hq, d), dtype=np.float64)
    for h in range(hq):
        g = kv_head_of(h, group)
        state = (-math.inf, 0.0, np.zeros(d))
        for lo, hi in zip(cuts[:-1], cuts[1:]):
            if hi <= lo:
                continue
            s = (keys[lo:hi, g, :] @ q[h]) * scale
            m = float(s.max())
            w = np.exp(s - m)
            state = merge_states(state, (m, float(w.sum()), w @ values[lo:hi, g, :]))
        out[h] = state[2] / state[1]
    return out
