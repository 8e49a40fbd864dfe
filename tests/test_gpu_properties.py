"""Property tests through the C ABI on random decode steps (hypothesis, derandomized): the fused
step, the two-call step and the oracle agree for random batches, lengths, KV-head counts,
partition sizes and physical page orders."""

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from gpu_helpers import assert_close, bf16_to_bits, to_gpu_i32, upload
from workloads import make_custom

pytestmark = pytest.mark.gpu


@settings(max_examples=25, deadline=None, derandomize=True)
@given(
    lengths=st.lists(st.integers(1, 700), min_size=1, max_size=9),
    hkv=st.sampled_from([1, 2, 8]),
    partition_pages=st.sampled_from([0, 4, 12, 128]),
    seed=st.integers(0, 2**16),
)
def test_random_steps(gpu, lengths, hkv, partition_pages, seed):
    import torch

    w = make_custom(seed=seed, lengths=lengths, num_kv_heads=hkv)
    d = upload(w)
    k2, v2 = d["k_pool"].clone(), d["v_pool"].clone()
    gpu.kv_append(d["k_pool"], d["v_pool"], d["block_tables"], d["positions"], d["k_new"], d["v_new"])
    a = gpu.paged_decode_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                                   out_dtype=torch.float32, partition_pages=partition_pages)
    b = gpu.decode_step(d["q"], k2, v2, d["block_tables"], d["positions"], d["k_new"], d["v_new"],
                        out_dtype=torch.float32, partition_pages=partition_pages)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    rk, rv = oracle.kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.k_new[0], w.v_new[0])
    assert np.array_equal(bf16_to_bits(k2), rk) and np.array_equal(bf16_to_bits(v2), rv)
    ref = oracle.paged_decode_attention(w.q[0], rk, rv, w.block_tables[0], w.context_lens)
    assert_close(b.cpu().numpy(), ref, f"lengths={lengths} hkv={hkv} pp={partition_pages}")
