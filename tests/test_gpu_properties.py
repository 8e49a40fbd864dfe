"""Property tests through the C ABI on random decode steps (hypothesis, derandomized): the fused
step, the two-call step and the oracle agree for random batches, lengths, KV-head counts,
partition sizes, physical page orders and query scales (q times 1, 4 or 32, exact in BF16: the
larger scales make peaked rows whose maximum sits at a random key, so the kernels' running
maxima and anchor moves are exercised at every position)."""

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from gpu_helpers import assert_close, bf16_to_bits, to_gpu_bf16, to_gpu_i32, upload
from workloads import f32_to_bf16_bits, make_custom

pytestmark = pytest.mark.gpu


def scale_bf16(bits, factor):
    """BF16 bit patterns times a power of two (exact for these N(0, 1) values)."""
    f = (np.asarray(bits, dtype=np.uint32) << np.uint32(16)).view(np.float32) * np.float32(factor)
    return f32_to_bf16_bits(f)


@settings(max_examples=25, deadline=None, derandomize=True)
@given(
    lengths=st.lists(st.integers(1, 700), min_size=1, max_size=9),
    hkv=st.sampled_from([1, 2, 8]),
    partition_pages=st.sampled_from([0, 4, 12, 128]),
    q_scale=st.sampled_from([1.0, 4.0, 32.0]),
    seed=st.integers(0, 2**16),
)
def test_random_steps(gpu, lengths, hkv, partition_pages, q_scale, seed):
    import torch

    w = make_custom(seed=seed, lengths=lengths, num_kv_heads=hkv)
    w.q = scale_bf16(w.q, q_scale)
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
    assert_close(b.cpu().numpy(), ref, f"lengths={lengths} hkv={hkv} pp={partition_pages} q x{q_scale}")


@settings(max_examples=15, deadline=None, derandomize=True)
@given(
    lengths=st.lists(st.integers(0, 200), min_size=1, max_size=5),
    starts=st.lists(st.integers(0, 700), min_size=5, max_size=5),
    q_scale=st.sampled_from([1.0, 4.0, 32.0]),
    seed=st.integers(0, 2**16),
)
def test_random_prefill_steps(gpu, lengths, starts, q_scale, seed):
    """Random prompt batches (empty prompts, chunks behind cached prefixes of any offset) through
    the prefill pair, against the prefill oracle."""
    import torch

    from workloads import make_prefill

    starts = starts[: len(lengths)]
    w = make_prefill(seed, lengths, starts)
    if w.tokens == 0:
        return
    w.q = scale_bf16(w.q, q_scale)
    d = {"block_tables": to_gpu_i32(w.block_tables), "cu_seqlens": to_gpu_i32(w.cu_seqlens),
         "start_pos": to_gpu_i32(w.start_pos)}
    kp, vp = to_gpu_bf16(w.k_pool), to_gpu_bf16(w.v_pool)
    gpu.prefill_kv_append(kp, vp, d["block_tables"], d["cu_seqlens"], d["start_pos"], to_gpu_bf16(w.k_new),
                          to_gpu_bf16(w.v_new))
    out = gpu.paged_prefill_attention(to_gpu_bf16(w.q), kp, vp, d["block_tables"], d["cu_seqlens"], d["start_pos"],
                                      out_dtype=torch.float32)
    torch.cuda.synchronize()
    rk, rv = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new, w.v_new)
    assert np.array_equal(bf16_to_bits(kp), rk) and np.array_equal(bf16_to_bits(vp), rv)
    ref = oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos)
    assert_close(out.cpu().numpy(), ref, f"lengths={lengths} starts={starts} q x{q_scale}")


@pytest.mark.parametrize("q_scale", [4.0, 32.0])
def test_vector_kernel_on_peaked_rows(gpu, q_scale):
    """The large-batch (VALU) kernel on peaked rows: 40 sequences of random lengths (40 x 8 pairs
    fill the chip, so the plan is unsplit and the VALU kernel runs) with q scaled by 4 or 32."""
    import torch

    rng = np.random.default_rng(int(q_scale))
    lengths = [int(x) for x in rng.integers(1, 701, 40)]
    w = make_custom(seed=90 + int(q_scale), lengths=lengths)
    w.q = scale_bf16(w.q, q_scale)
    d = upload(w)
    gpu.kv_append(d["k_pool"], d["v_pool"], d["block_tables"], d["positions"], d["k_new"], d["v_new"])
    out = gpu.paged_decode_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    rk, rv = oracle.kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.k_new[0], w.v_new[0])
    ref = oracle.paged_decode_attention(w.q[0], rk, rv, w.block_tables[0], w.context_lens)
    assert_close(out.cpu().numpy(), ref, f"VALU kernel, q x{q_scale}")
