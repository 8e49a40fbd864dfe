"""FP64 CPU oracle for paged prefill: write a prompt's K/V rows into pages, then causal
attention over those pages.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this module; the HIP library never calls it and shares no code with it.

What it computes ("The prefill path: flowing the entire prompt at once"):

* **Append** (section "Distributing K/V into paged blocks"): prompt token ``i`` of a sequence
  goes to logical block ``pos // 16`` of its block table, slot ``pos % 16``, with
  ``pos = start + i``.  A bit copy of every KV head's row.
* **Causal attention** (sections "Per-head attention scores and GQA", "causalMask and online
  softmax" and "Scores×V → O → residual → SwiGLU"): for query head ``h`` the scores are
  ``q . k / 8`` against KV head ``h // 4``; cells whose key position is later than the query's
  own position are excluded (their probability is 0); softmax along the row; the probabilities
  weight the V rows of the same KV head.

Readings: the article rounds the score and probability matrices to BF16 between its steps; this
oracle is the exact definition in FP64 with no intermediate rounding (the same target the
decode path is held to).  ``start > 0`` generalises the article's whole-prompt prefill to a prompt
chunk behind ``start`` cached tokens: query row ``i`` attends to positions ``0 .. start + i``.
Out-of-range inputs follow the library's error rule: a prompt with a negative start writes
nothing, a row whose position has no page of the pool is not written, and every output row of a
prompt whose positions ``0 .. start + n - 1`` do not all map to pages of the pool is zero.

Pinned by ``tests/test_oracle_prefill_pins.py``.
"""

from __future__ import annotations

import numpy as np

from .paged_oracle import (BLOCK_SIZE, bf16_bits_to_f64, context_in_pool, gather_context, kv_head_of, locate_slot,
                           slot_in_pool)


def prefill_kv_append(k_pool, v_pool, block_tables, cu_seqlens, start_pos, k_new, v_new):
    """Copies of the pools with every prompt row written at its absolute position.

    ``block_tables`` int32 [B][T]; ``cu_seqlens`` [B+1]; ``start_pos`` [B]; ``k_new``/``v_new``
    uint16 [N][Hkv][D] packed by ``cu_seqlens``.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for b in range(len(start_pos)):
        if int(start_pos[b]) < 0:
            continue  # the whole prompt is skipped
        for row in range(int(cu_seqlens[b]), int(cu_seqlens[b + 1])):
            pos = int(start_pos[b]) + row - int(cu_seqlens[b])
            if not slot_in_pool(block_tables[b], pos, k_out.shape[0]):
                continue  # this row is skipped
            page, slot = locate_slot(block_tables[b], pos)
            k_out[page, :, slot, :] = k_new[row]
            v_out[page, :, slot, :] = v_new[row]
    return k_out, v_out


def causal_attention_rows(q, keys, values, positions, scale):
    """Causal attention of query rows at absolute ``positions``.

    ``q`` FP64 [n][Hq][D]; ``keys``/``values`` FP64 [L][Hkv][D] with L > max(positions).  Row ``i``
    sees keys ``0 .. positions[i]`` only: the excluded cells have probability 0, so the row is
    computed over its visible prefix alone and later rows cannot reach it.
    """
    n, hq, d = q.shape
    group = hq // keys.shape[1]
    k_heads = np.ascontiguousarray(keys.transpose(1, 0, 2))  # [Hkv][L][D]: one head's rows contiguous
    v_heads = np.ascontiguousarray(values.transpose(1, 0, 2))
    out = np.empty((n, hq, d), dtype=np.float64)
    for i in range(n):
        visible = int(positions[i]) + 1
        for h in range(hq):
            g = kv_head_of(h, group)
            scores = (k_heads[g, :visible] @ q[i, h]) * scale
            m = scores.max()
            w = np.exp(scores - m)
            out[i, h] = (w / w.sum()) @ v_heads[g, :visible]
    return out


def paged_prefill_attention(q, k_pool, v_pool, block_tables, cu_seqlens, start_pos, scale=0.125, rows=None):
    """FP64 output [N][Hq][D] of causal attention for every packed prompt row, reading K/V
    (already appended) through each sequence's block table.  ``rows`` optionally restricts the
    work to some packed rows (the others are left as NaN) so a large step can be sampled."""
    q = np.asarray(q)
    out = np.full(q.shape, np.nan, dtype=np.float64)
    wanted = None if rows is None else set(int(r) for r in rows)
    for b in range(len(start_pos)):
        lo, hi = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        sel = [r for r in range(lo, hi) if wanted is None or r in wanted]
        if not sel:
            continue
        start = int(start_pos[b])
        if start < 0 or not context_in_pool(block_tables[b], start + hi - lo, k_pool.shape[0]):
            out[sel] = 0.0  # the whole prompt cannot be read through its table
            continue
        positions = np.array([start + r - lo for r in sel])
        L = int(positions.max()) + 1
        keys = bf16_bits_to_f64(gather_context(k_pool, block_tables[b], L))
        values = bf16_bits_to_f64(gather_context(v_pool, block_tables[b], L))
        out[sel] = causal_attention_rows(bf16_bits_to_f64(q[sel]), keys, values, positions, scale)
    return out


__all__ = ["BLOCK_SIZE", "prefill_kv_append", "causal_attention_rows", "paged_prefill_attention"]
