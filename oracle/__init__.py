"""CPU oracle (FP64) for the paged KV cache decode path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py``; never by the library in ``paged_kv_cache_pages_amd``.
"""

from .paged_oracle import (  # noqa: F401
    attend_one,
    attend_one_online,
    bf16_bits_to_f64,
    bf16_round_nearest_even,
    context_in_pool,
    gather_context,
    kv_append,
    kv_head_of,
    locate_slot,
    merge_states,
    paged_decode_attention,
    slot_in_pool,
    softmax_two_pass,
)
from .rope_oracle import bf16_bits_to_f32, rope_kv_append, rope_pair_index, rope_rotate  # noqa: F401,E402
from .allocator_oracle import AllocatorModel  # noqa: F401,E402
from .prefill_oracle import causal_attention_rows, paged_prefill_attention, prefill_kv_append  # noqa: F401,E402
