"""Every compute call at KV-head counts other than the model's 8.

The group of four query heads per KV head is fixed; the number of KV heads is a runtime argument.
A tensor-parallel shard of the 8-KV-head model holds 1 (eight ways) or 2 (four ways) KV heads per
GPU, and 5 exercises a count that divides nothing. For each count: the fused decode step against
the two separate calls (bit for bit) and the FP64 oracle, unsplit and split; the RoPE append bit
for bit against the RoPE oracle; the prefill append bit for bit and the causal attention against
the prefill oracle. (The plain attention call is covered at these counts in test_gpu_parity.)
"""

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, bf16_to_bits, to_gpu_bf16, to_gpu_i32, upload
from workloads import llama3_rope_tables, make_custom, make_prefill

pytestmark = pytest.mark.gpu
COUNTS = (1, 2, 5)


@pytest.mark.parametrize("hkv", COUNTS)
def test_fused_step_at_other_kv_head_counts(gpu, hkv):
    import torch

    w = make_custom(seed=140 + hkv, lengths=[2048, 700, 33, 16, 1], num_kv_heads=hkv)
    planned = gpu.plan_partition_pages(w.batch, hkv, w.max_blocks, max_context=int(w.context_lens.max()))
    rk, rv = oracle.kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.k_new[0], w.v_new[0])
    ref = oracle.paged_decode_attention(w.q[0], rk, rv, w.block_tables[0], w.context_lens)
    for pp in sorted({w.max_blocks, planned, 8}):
        print(f"[kv heads] fused step hkv={hkv} B={w.batch} partition_pages={pp}", flush=True)
        d1, d2 = upload(w), upload(w)
        gpu.kv_append(d1["k_pool"], d1["v_pool"], d1["block_tables"], d1["positions"], d1["k_new"], d1["v_new"])
        a = gpu.paged_decode_attention(d1["q"], d1["k_pool"], d1["v_pool"], d1["block_tables"], d1["context_lens"],
                                       out_dtype=torch.float32, partition_pages=pp)
        b = gpu.decode_step(d2["q"], d2["k_pool"], d2["v_pool"], d2["block_tables"], d2["positions"], d2["k_new"],
                            d2["v_new"], out_dtype=torch.float32, partition_pages=pp)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"hkv={hkv} pp={pp}: fused step differs from the two calls"
        assert np.array_equal(bf16_to_bits(d2["k_pool"]), rk) and np.array_equal(bf16_to_bits(d2["v_pool"]), rv)
        assert_close(b.cpu().numpy(), ref, f"fused hkv={hkv} pp={pp}")


@pytest.mark.parametrize("hkv", COUNTS)
def test_rope_append_at_other_kv_head_counts(gpu, hkv):
    import torch

    w = make_custom(seed=150 + hkv, lengths=[2048, 513, 17, 1], num_kv_heads=hkv)
    print(f"[kv heads] rope append hkv={hkv} B={w.batch}", flush=True)
    cos, sin = llama3_rope_tables(2048)
    d = upload(w)
    q_out = torch.empty_like(d["q"])
    gpu.rope_kv_append(d["k_pool"], d["v_pool"], d["block_tables"], d["positions"], d["q"], d["k_new"], d["v_new"],
                       torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda(), q_out=q_out)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.rope_kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.q[0], w.k_new[0],
                                       w.v_new[0], cos, sin)
    assert np.array_equal(bf16_to_bits(q_out), rq)
    assert np.array_equal(bf16_to_bits(d["k_pool"]), rk)
    assert np.array_equal(bf16_to_bits(d["v_pool"]), rv)


@pytest.mark.parametrize("hkv", COUNTS)
def test_prefill_at_other_kv_head_counts(gpu, hkv):
    import torch

    lens, starts = [300, 17, 64, 1], [100, 0, 1000, 5]
    w = make_prefill(160 + hkv, lens, starts, num_kv_heads=hkv)
    print(f"[kv heads] prefill hkv={hkv} lens={lens} starts={starts}", flush=True)
    kp, vp = to_gpu_bf16(w.k_pool), to_gpu_bf16(w.v_pool)
    bt, cu, st = to_gpu_i32(w.block_tables), to_gpu_i32(w.cu_seqlens), to_gpu_i32(w.start_pos)
    gpu.prefill_kv_append(kp, vp, bt, cu, st, to_gpu_bf16(w.k_new), to_gpu_bf16(w.v_new))
    out = gpu.paged_prefill_attention(to_gpu_bf16(w.q), kp, vp, bt, cu, st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rk, rv = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new, w.v_new)
    assert np.array_equal(bf16_to_bits(kp), rk) and np.array_equal(bf16_to_bits(vp), rv)
    ref = oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos)
    assert_close(out.cpu().numpy(), ref, f"prefill hkv={hkv}")
