"""Seeded inputs of a paged prefill step (write the prompt's K/V rows into pages, then causal
attention over the pages).  Input construction only: no part of the method's arithmetic.

Sequences are packed: sequence ``b`` owns query/K/V rows ``cu_seqlens[b] .. cu_seqlens[b+1]-1``,
and its prompt token ``i`` sits at absolute position ``start_pos[b] + i`` (``start_pos`` = 0 is
a whole prompt; a positive value is a prompt chunk behind ``start_pos`` tokens that are already
cached, whose rows are the pool's random contents).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .configs import BLOCK_SIZE, HEAD_DIM, MAX_BLOCKS, NUM_KV_HEADS, NUM_Q_HEADS, normal_bf16


@dataclass
class PrefillWorkload:
    """Shapes (P pages, B sequences, N packed prompt tokens, T table width):

    * ``k_pool``, ``v_pool``: uint16 [P][Hkv][16][D] BF16 bits.
    * ``block_tables``: int32 [B][T] (-1 = unassigned); every page up to the prompt's last
      position is assigned.
    * ``cu_seqlens``: int32 [B+1] prefix sums of the prompt lengths; ``start_pos``: int32 [B].
    * ``q``: uint16 [N][Hq][D]; ``k_new``, ``v_new``: uint16 [N][Hkv][D].
    """

    name: str
    seed: int
    k_pool: np.ndarray
    v_pool: np.ndarray
    block_tables: np.ndarray
    cu_seqlens: np.ndarray
    start_pos: np.ndarray
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.block_tables.shape[0])

    @property
    def tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def prompt_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens).astype(np.int32)

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])


def make_prefill(seed: int, prompt_lens, start_pos=None, num_pages: int | None = None, max_blocks: int = MAX_BLOCKS,
                 num_kv_heads: int = NUM_KV_HEADS, group: int = NUM_Q_HEADS // NUM_KV_HEADS, head_dim: int = HEAD_DIM,
                 name: str = "prefill") -> PrefillWorkload:
    """Draw order: page permutation, K pool, V pool, q, k_new, v_new.  Pages come from the back
    of the shuffled free list, sequence by sequence in block order; ``num_pages`` defaults to the
    pages needed plus eight spares."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(prompt_lens, dtype=np.int32).reshape(-1)
    starts = np.zeros_like(lens) if start_pos is None else np.asarray(start_pos, dtype=np.int32).reshape(-1)
    if starts.shape != lens.shape or (lens < 0).any() or (starts < 0).any():
        raise ValueError("prompt_lens and start_pos must be non-negative and of one length")
    ends = starts + lens
    if ends.size and int(ends.max()) > max_blocks * BLOCK_SIZE:
        raise ValueError("a prompt runs past the block-table width")
    pages_needed = [(int(e) + BLOCK_SIZE - 1) // BLOCK_SIZE for e in ends]
    if num_pages is None:
        num_pages = sum(pages_needed) + 8
    if sum(pages_needed) > num_pages:
        raise ValueError(f"{sum(pages_needed)} pages needed but the pool has {num_pages}")
    free = [int(p) for p in rng.permutation(num_pages)]
    tables = np.full((len(lens), max_blocks), -1, dtype=np.int32)
    for b, n in enumerate(pages_needed):
        for j in range(n):
            tables[b, j] = free.pop()
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    total = int(cu[-1])
    hq = num_kv_heads * group
    k_pool = normal_bf16(rng, (num_pages, num_kv_heads, BLOCK_SIZE, head_dim))
    v_pool = normal_bf16(rng, (num_pages, num_kv_heads, BLOCK_SIZE, head_dim))
    q = normal_bf16(rng, (total, hq, head_dim))
    k_new = normal_bf16(rng, (total, num_kv_heads, head_dim))
    v_new = normal_bf16(rng, (total, num_kv_heads, head_dim))
    meta = {"tokens": total, "pages": int(sum(pages_needed)),
            "causal_pairs": int(sum(int(s) * int(n) + int(n) * (int(n) + 1) // 2 for s, n in zip(starts, lens)))}
    return PrefillWorkload(name, seed, k_pool, v_pool, tables, cu, starts, q, k_new, v_new, meta)


PREFILL_CONFIGS = ("prefill_tiny", "prefill512", "prefill_chunked", "prefill16x512")


def make_prefill_config(name: str) -> PrefillWorkload:
    """Named prefill workloads.

    * ``prefill_tiny``: one 37-token prompt (three pages, the last partial).
    * ``prefill512``: one 512-token prompt, the longest prompt of the engine the pages describe.
    * ``prefill_chunked``: six prompt chunks of uniform lengths in [1, 512] behind cached
      prefixes of uniform lengths in [0, 1536], so every row crosses page boundaries at its own
      offset.
    * ``prefill16x512``: sixteen 512-token prompts in one launch (8192 query rows).
    """
    if name == "prefill_tiny":
        return make_prefill(10, [37], name=name)
    if name == "prefill512":
        return make_prefill(11, [512], name=name)
    if name == "prefill_chunked":
        rng = np.random.default_rng(12)
        lens = rng.integers(1, 513, size=6)
        starts = rng.integers(0, 1537, size=6)
        return make_prefill(12, lens, starts, name=name)
    if name == "prefill16x512":
        return make_prefill(13, [512] * 16, name=name)
    raise KeyError(f"unknown prefill config {name!r}; expected one of {PREFILL_CONFIGS}")
