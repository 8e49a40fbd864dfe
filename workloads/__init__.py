"""Seeded synthetic decode-step workloads for the paged KV cache.

This package only *builds inputs*: BF16 page pools (as uint16 bit patterns), block tables,
positions, context lengths, queries and the new K/V rows of one decode step.  It holds none of
the attention or append arithmetic, so both the CPU oracle (``oracle/``) and the HIP path
(``paged_kv_cache_pages_amd``) can consume the same inputs without sharing any code.

Geometry follows the Llama-3.2-1B decode shape described in the pages:

* 16-token pages and a per-sequence block table whose entry -1 means "unassigned"
  ("The prefill path: flowing the entire prompt at once", section "Distributing K/V into paged blocks").
* 32 query heads sharing 8 KV heads in consecutive groups of four, head_dim 64
  (same page, section "Per-head attention scores and GQA").
* A 2048-token context cap and a shared 128 MiB pool whose size does not grow with the
  request count ("6 Hours of YouTube and 85 handtyped pages of notes on LLM Inference", section "Current scope").
"""

from .configs import (  # noqa: F401
    BLOCK_SIZE,
    CONFIG_NAMES,
    HEAD_DIM,
    MAX_BLOCKS,
    NUM_KV_HEADS,
    NUM_Q_HEADS,
    Workload,
    f32_to_bf16_bits,
    llama3_rope_tables,
    make_config,
    make_custom,
    normal_bf16,
)
from .prefill import PREFILL_CONFIGS, PrefillWorkload, make_prefill, make_prefill_config  # noqa: F401,E402
