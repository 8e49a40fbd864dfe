"""A continuous-batching decode loop on the GPU driven by the C++ page allocator.

Requests are admitted by their page credits, their prompt K/V rows are written with kv_append
(one row per prompt token), then every decode step takes its block tables from
pkv_alloc_prepare_step and runs pkv_decode_step per layer.  Finished requests release their
pages, which later requests reuse while the old K/V rows are still in them.  Every step's
output is checked against the FP64 oracle run on the same tables, and the pools against the
oracle's appends, bit for bit.
"""

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, bf16_to_bits, to_gpu_bf16, to_gpu_i32
from workloads import normal_bf16

pytestmark = pytest.mark.gpu

HKV, HQ, D = 8, 32, 64


@pytest.mark.parametrize("static", [False, True])
def test_continuous_batching_loop(gpu, static):
    import torch

    rng = np.random.default_rng(11 + static)
    layers, max_blocks, num_pages = 2, 16, 2 * 30
    alloc = gpu.PageAllocator(num_pages, layers, max_blocks, free_order=rng.permutation(num_pages), static=static)
    k_ref = normal_bf16(rng, (num_pages, HKV, 16, D))  # stale rows the requests never wrote
    v_ref = normal_bf16(rng, (num_pages, HKV, 16, D))
    kp, vp = to_gpu_bf16(k_ref), to_gpu_bf16(v_ref)
    reqs = {rid: (int(rng.integers(1, 140)), int(rng.integers(0, 40))) for rid in range(12)}
    for rid, (p, n) in reqs.items():
        assert alloc.submit(rid, p, n) == 0
    pos, left, done, steps = {}, {}, 0, 0
    while done < len(reqs):
        for rid in alloc.admit():
            p, n = reqs[rid]
            for t in range(p):
                assert alloc.ensure(rid, t) == 0
            table = alloc.table(rid)
            positions = np.arange(p, dtype=np.int32)
            for layer in range(layers):
                bt = np.repeat(table[layer][None, :], p, axis=0)
                kn, vn = normal_bf16(rng, (p, HKV, D)), normal_bf16(rng, (p, HKV, D))
                gpu.kv_append(kp, vp, to_gpu_i32(bt), to_gpu_i32(positions), to_gpu_bf16(kn), to_gpu_bf16(vn))
                k_ref, v_ref = oracle.kv_append(k_ref, v_ref, bt, positions, kn, vn)
            pos[rid], left[rid] = p, min(n, max_blocks * 16 - p) - 1  # the first output comes from prefill
        rows = sorted(r for r in pos if left[r] > 0)
        if rows:
            st, bad, tables = alloc.prepare_step(rows, [pos[r] for r in rows])
            assert st == 0, (st, bad)
            positions = np.array([pos[r] for r in rows], dtype=np.int32)
            print(f"[loop static={static}] step {steps} batch {len(rows)} max_pos {positions.max()}", flush=True)
            # rotate: the plan from the longest context (which the loop knows), a forced 4-page
            # split, and the plan from the table width alone
            pp = (0, 4, 0)[steps % 3]
            longest = int(positions.max()) + 1 if steps % 3 == 0 else None
            for layer in range(layers):
                q = normal_bf16(rng, (len(rows), HQ, D))
                kn, vn = normal_bf16(rng, (len(rows), HKV, D)), normal_bf16(rng, (len(rows), HKV, D))
                out = gpu.decode_step(to_gpu_bf16(q), kp, vp, to_gpu_i32(tables[layer]), to_gpu_i32(positions),
                                      to_gpu_bf16(kn), to_gpu_bf16(vn), out_dtype=torch.float32, partition_pages=pp,
                                      max_context=longest)
                k_ref, v_ref = oracle.kv_append(k_ref, v_ref, tables[layer], positions, kn, vn)
                ref = oracle.paged_decode_attention(q, k_ref, v_ref, tables[layer], positions + 1)
                torch.cuda.synchronize()
                assert_close(out.cpu().numpy(), ref, f"step {steps} layer {layer}")
            steps += 1
        for r in list(pos):
            if left[r] > 0:
                pos[r] += 1
                left[r] -= 1
            if left[r] <= 0:
                assert alloc.release(r) == 0
                del pos[r], left[r]
                done += 1
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_bits(kp), k_ref) and np.array_equal(bf16_to_bits(vp), v_ref)
    s = alloc.stats()
    assert s["free_pages"] == num_pages and s["active"] == 0
    assert s["largest_batch"] >= 2 and steps > 20
    if not static:
        assert s["admission_waits"] > 0  # the pool is small enough that requests queue


def test_prefill_then_decode_loop(gpu):
    """Admitted prompts are written and attended by the paged prefill kernels in one batched call
    per layer (each prompt's causal attention checked against the prefill oracle), then decode
    steps continue from the pages prefill wrote, checked against the decode oracle."""
    import torch

    rng = np.random.default_rng(21)
    layers, max_blocks, num_pages = 2, 24, 2 * 48
    alloc = gpu.PageAllocator(num_pages, layers, max_blocks, free_order=rng.permutation(num_pages))
    k_ref = normal_bf16(rng, (num_pages, HKV, 16, D))
    v_ref = normal_bf16(rng, (num_pages, HKV, 16, D))
    kp, vp = to_gpu_bf16(k_ref), to_gpu_bf16(v_ref)
    reqs = {rid: (int(rng.integers(1, 200)), int(rng.integers(1, 30))) for rid in range(10)}
    for rid, (p, n) in reqs.items():
        assert alloc.submit(rid, p, n) == 0
    pos, left, done, steps, prefills = {}, {}, 0, 0, 0
    while done < len(reqs):
        admitted = alloc.admit()
        if admitted:
            lens = [reqs[r][0] for r in admitted]
            for rid, p in zip(admitted, lens):
                for t in range(0, p, 16):
                    assert alloc.ensure(rid, t) == 0
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            start = np.zeros(len(lens), dtype=np.int32)
            print(f"[prefill loop] prefill of {len(lens)} prompts, {int(cu[-1])} rows", flush=True)
            for layer in range(layers):
                bt = np.stack([alloc.table(r)[layer] for r in admitted]).astype(np.int32)
                q = normal_bf16(rng, (int(cu[-1]), HQ, D))
                kn, vn = normal_bf16(rng, (int(cu[-1]), HKV, D)), normal_bf16(rng, (int(cu[-1]), HKV, D))
                d_bt, d_cu, d_st = to_gpu_i32(bt), to_gpu_i32(cu), to_gpu_i32(start)
                gpu.prefill_kv_append(kp, vp, d_bt, d_cu, d_st, to_gpu_bf16(kn), to_gpu_bf16(vn))
                out = gpu.paged_prefill_attention(to_gpu_bf16(q), kp, vp, d_bt, d_cu, d_st, out_dtype=torch.float32)
                k_ref, v_ref = oracle.prefill_kv_append(k_ref, v_ref, bt, cu, start, kn, vn)
                ref = oracle.paged_prefill_attention(q, k_ref, v_ref, bt, cu, start)
                torch.cuda.synchronize()
                assert_close(out.cpu().numpy(), ref, f"prefill {prefills} layer {layer}")
            prefills += 1
            for rid, p in zip(admitted, lens):
                pos[rid], left[rid] = p, min(reqs[rid][1], max_blocks * 16 - p) - 1
        rows = sorted(r for r in pos if left[r] > 0)
        if rows:
            st, bad, tables = alloc.prepare_step(rows, [pos[r] for r in rows])
            assert st == 0, (st, bad)
            positions = np.array([pos[r] for r in rows], dtype=np.int32)
            for layer in range(layers):
                q = normal_bf16(rng, (len(rows), HQ, D))
                kn, vn = normal_bf16(rng, (len(rows), HKV, D)), normal_bf16(rng, (len(rows), HKV, D))
                out = gpu.decode_step(to_gpu_bf16(q), kp, vp, to_gpu_i32(tables[layer]), to_gpu_i32(positions),
                                      to_gpu_bf16(kn), to_gpu_bf16(vn), out_dtype=torch.float32,
                                      partition_pages=4 if steps % 2 else 0)
                k_ref, v_ref = oracle.kv_append(k_ref, v_ref, tables[layer], positions, kn, vn)
                ref = oracle.paged_decode_attention(q, k_ref, v_ref, tables[layer], positions + 1)
                torch.cuda.synchronize()
                assert_close(out.cpu().numpy(), ref, f"step {steps} layer {layer}")
            steps += 1
        for r in list(pos):
            if left[r] > 0:
                pos[r] += 1
                left[r] -= 1
            if left[r] <= 0:
                assert alloc.release(r) == 0
                del pos[r], left[r]
                done += 1
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_bits(kp), k_ref) and np.array_equal(bf16_to_bits(vp), v_ref)
    assert prefills >= 2 and steps > 10
    assert alloc.stats()["free_pages"] == num_pages
