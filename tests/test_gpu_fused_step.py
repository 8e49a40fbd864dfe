"""pkv_decode_step (append + attention in one launch) against the two separate calls.

The fused step must leave the pool bit-identical to kv_append and produce a bit-identical FP32
output to paged_decode_attention over positions + 1 tokens with the same partition size; both
are also checked against the FP64 oracle.
"""

import os

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, bf16_to_bits, layer_tensors, to_gpu_bf16, to_gpu_i32, upload
from workloads import make_config, make_custom

pytestmark = pytest.mark.gpu
NAN_BITS = np.uint16(0x7FC0)


def two_calls(gpu, q, kp, vp, bt, pos, lens, kn, vn, pp):
    import torch

    gpu.kv_append(kp, vp, bt, pos, kn, vn)
    return gpu.paged_decode_attention(q, kp, vp, bt, lens, out_dtype=torch.float32, partition_pages=pp)


def fused(gpu, q, kp, vp, bt, pos, kn, vn, pp):
    import torch

    return gpu.decode_step(q, kp, vp, bt, pos, kn, vn, out_dtype=torch.float32, partition_pages=pp)


@pytest.mark.parametrize("name", ["tiny", "long", "mixed", "model16", "bw256", "bw256tp8"])
def test_fused_step_equals_two_calls(gpu, name):
    import torch

    w = make_config(name)
    # the launch configuration bench.py times: the plan from the longest context
    pp = gpu.plan_partition_pages(w.batch, w.num_kv_heads, w.max_blocks, max_context=int(w.context_lens.max()))
    print(f"[fused] config={name} B={w.batch} layers={w.layers} partition_pages={pp}", flush=True)
    kp1, vp1 = to_gpu_bf16(w.k_pool), to_gpu_bf16(w.v_pool)
    kp2, vp2 = kp1.clone(), vp1.clone()
    pos, lens = to_gpu_i32(w.positions), to_gpu_i32(w.context_lens)
    ref_k, ref_v = w.k_pool, w.v_pool
    for layer in range(w.layers):
        t = layer_tensors(w, layer)
        a = two_calls(gpu, t["q"], kp1, vp1, t["block_tables"], pos, lens, t["k_new"], t["v_new"], pp)
        b = fused(gpu, t["q"], kp2, vp2, t["block_tables"], pos, t["k_new"], t["v_new"], pp)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"layer {layer}"
        if layer == 0 or layer == w.layers - 1:
            ref_k, ref_v = oracle.kv_append(ref_k, ref_v, w.block_tables[layer], w.positions, w.k_new[layer],
                                            w.v_new[layer])
            if name != "bw256" or layer == 0:
                rows = None if w.batch <= 64 else list(range(0, w.batch, 16))
                ref = oracle.paged_decode_attention(w.q[layer], ref_k, ref_v, w.block_tables[layer], w.context_lens,
                                                    sequences=rows)
                sel = slice(None) if rows is None else rows
                assert_close(b.cpu().numpy()[sel], ref[sel], f"{name} layer {layer}")
        elif w.layers > 1:
            ref_k, ref_v = oracle.kv_append(ref_k, ref_v, w.block_tables[layer], w.positions, w.k_new[layer],
                                            w.v_new[layer])
    assert torch.equal(kp1, kp2) and torch.equal(vp1, vp2)
    assert np.array_equal(bf16_to_bits(kp2), ref_k) and np.array_equal(bf16_to_bits(vp2), ref_v)


@pytest.mark.parametrize("partition_pages", [4, 8, 128])
def test_fused_step_boundaries_and_nan_slots(gpu, partition_pages):
    """Positions 0, 15, 16, 31, 2047 and friends; the target slots hold NaN beforehand."""
    import torch

    lengths = [1, 15, 16, 17, 31, 32, 33, 2048, 1000, 2]
    w = make_custom(seed=70, lengths=lengths)
    kp = w.k_pool.copy()
    vp = w.v_pool.copy()
    for b, p in enumerate(w.positions):
        page = w.block_tables[0, b, p // 16]
        kp[page, :, p % 16] = NAN_BITS
        vp[page, :, p % 16] = NAN_BITS
    d = upload(w)
    k1, v1 = to_gpu_bf16(kp), to_gpu_bf16(vp)
    k2, v2 = k1.clone(), v1.clone()
    a = two_calls(gpu, d["q"], k1, v1, d["block_tables"], d["positions"], d["context_lens"], d["k_new"], d["v_new"],
                  partition_pages)
    b = fused(gpu, d["q"], k2, v2, d["block_tables"], d["positions"], d["k_new"], d["v_new"], partition_pages)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    got = b.cpu().numpy()
    assert np.all(np.isfinite(got))
    rk, rv = oracle.kv_append(kp, vp, w.block_tables[0], w.positions, w.k_new[0], w.v_new[0])
    assert_close(got, oracle.paged_decode_attention(w.q[0], rk, rv, w.block_tables[0], w.context_lens), "boundaries")


@pytest.mark.parametrize("partition_pages", [4, 128])
def test_fused_step_invalid_rows(gpu, partition_pages):
    """Out-of-range positions or table entries: no append for that row and a zero output row,
    exactly as with the two separate calls."""
    import torch

    w = make_custom(seed=71, lengths=[40, 70, 20, 90, 33, 137])
    pos = w.positions.copy()
    pos[0] = -1
    pos[2] = 128 * 16
    bt = w.block_tables[0].copy()
    bt[3, 5] = -7  # position 89 -> block 5
    bt[4, 0] = w.num_pages  # a context page (not the append page) out of range
    # block 4 shares a wavefront with the append page (block 8) when both are in one partition:
    # the row is still appended, as pkv_kv_append does, and the output row is zero
    bt[5, 4] = -3
    d = upload(w)
    k1, v1 = d["k_pool"], d["v_pool"]
    k2, v2 = k1.clone(), v1.clone()
    lens = to_gpu_i32(pos + 1)
    a = two_calls(gpu, d["q"], k1, v1, to_gpu_i32(bt), to_gpu_i32(pos), lens, d["k_new"], d["v_new"], partition_pages)
    b = fused(gpu, d["q"], k2, v2, to_gpu_i32(bt), to_gpu_i32(pos), d["k_new"], d["v_new"], partition_pages)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    got = b.cpu().numpy()
    for row in (0, 2, 3, 4, 5):
        assert np.all(got[row] == 0), row
    assert np.any(got[1] != 0)
    page = int(bt[5, 8])
    assert np.array_equal(bf16_to_bits(k2)[page, :, 136 % 16], w.k_new[0, 5])


def test_fused_step_debug_validation(gpu):
    w = make_custom(seed=72, lengths=[10, 20])
    d = upload(w)
    pos = w.positions.copy()
    pos[1] = -1
    os.environ["PKV_DEBUG_VALIDATE"] = "1"
    try:
        fused(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["positions"], d["k_new"], d["v_new"], 0)
        with pytest.raises(gpu.PagedKVError, match="PKV_ERR_VALIDATION"):
            fused(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], to_gpu_i32(pos), d["k_new"], d["v_new"], 0)
    finally:
        del os.environ["PKV_DEBUG_VALIDATE"]


def test_fused_step_graph_replay(gpu):
    import torch

    w = make_custom(seed=73, lengths=[1, 17, 300, 2048, 999, 64])
    d = upload(w)
    k0, v0 = d["k_pool"].clone(), d["v_pool"].clone()
    out = torch.empty((w.batch, 32, 64), dtype=torch.float32, device="cuda")
    pp = 8
    ws = torch.zeros(max(16, gpu.decode_workspace_bytes(w.batch, 32, w.max_blocks, pp)), dtype=torch.uint8, device="cuda")

    def step():
        gpu.decode_step(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["positions"], d["k_new"], d["v_new"], out,
                        partition_pages=pp, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager, ek, ev = out.clone(), d["k_pool"].clone(), d["v_pool"].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for replay in range(3):
        d["k_pool"].copy_(k0)
        d["v_pool"].copy_(v0)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager) and torch.equal(d["k_pool"], ek) and torch.equal(d["v_pool"], ev), replay
