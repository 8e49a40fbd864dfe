"""pkv_decode_step_static (the entry point that allocates nothing; its split scratch is a static
per-GPU array) against pkv_decode_step with an explicit workspace: the same launches, so pools and
outputs must be identical bit for bit, on two calls in a row, the second with a smaller input;
also replayed from a HIP graph, and checked against the FP64 oracle."""

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, bf16_to_bits, to_gpu_bf16, to_gpu_i32
from workloads import make_custom

pytestmark = pytest.mark.gpu


def _inputs(w):
    return {
        "k_pool": to_gpu_bf16(w.k_pool), "v_pool": to_gpu_bf16(w.v_pool), "bt": to_gpu_i32(w.block_tables[0]),
        "pos": to_gpu_i32(w.positions), "q": to_gpu_bf16(w.q[0]), "k_new": to_gpu_bf16(w.k_new[0]),
        "v_new": to_gpu_bf16(w.v_new[0]),
    }


def _both(gpu, w, pp):
    """The static entry and the workspace entry on separate copies of the same inputs."""
    import torch

    a, b = _inputs(w), _inputs(w)
    out_a = torch.full((w.batch, 32, 64), float("nan"), dtype=torch.float32, device="cuda")
    out_b = torch.full_like(out_a, float("nan"))
    gpu.decode_step_static(a["q"], a["k_pool"], a["v_pool"], a["bt"], a["pos"], a["k_new"], a["v_new"], out_a,
                           partition_pages=pp)
    ws = torch.zeros(max(16, gpu.decode_workspace_bytes(w.batch, 32, w.max_blocks, pp)), dtype=torch.uint8,
                     device="cuda")
    gpu.decode_step(b["q"], b["k_pool"], b["v_pool"], b["bt"], b["pos"], b["k_new"], b["v_new"], out_b,
                    partition_pages=pp, workspace=ws)
    torch.cuda.synchronize()
    return a, out_a, b, out_b


@pytest.mark.parametrize("pp", [0, 16, 8])
def test_static_scratch_step_equals_workspace_step(gpu, pp):
    import torch

    first = make_custom(seed=80, lengths=[2048, 1500, 37, 900, 2048, 1])  # a split, several partitions each
    second = make_custom(seed=81, lengths=[700, 20])  # smaller: fewer sequences and partitions
    for call, w in enumerate((first, second)):
        plan = pp or gpu.plan_partition_pages(w.batch, 8, w.max_blocks, max_context=int(w.context_lens.max()))
        need = gpu.decode_workspace_bytes(w.batch, 32, w.max_blocks, plan)
        print(f"[static scratch] call {call} B={w.batch} partition_pages={plan} scratch bytes={need}", flush=True)
        assert 0 < need <= gpu.STATIC_SCRATCH_BYTES
        a, out_a, b, out_b = _both(gpu, w, plan)
        assert torch.equal(out_a, out_b), f"call {call}: outputs differ"
        assert torch.equal(a["k_pool"], b["k_pool"]) and torch.equal(a["v_pool"], b["v_pool"]), f"call {call}: pools"
        rk, rv = oracle.kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.k_new[0], w.v_new[0])
        assert np.array_equal(bf16_to_bits(a["k_pool"]), rk) and np.array_equal(bf16_to_bits(a["v_pool"]), rv)
        ref = oracle.paged_decode_attention(w.q[0], rk, rv, w.block_tables[0], w.context_lens)
        assert_close(out_a.cpu().numpy(), ref, f"static scratch call {call}")


def test_static_scratch_step_graph_replay(gpu):
    """Captured into a HIP graph (the callers this entry is for) and replayed three times with the
    pools restored: every replay equals the eager call bit for bit."""
    import torch

    w = make_custom(seed=82, lengths=[2048, 333, 1024])
    d = _inputs(w)
    k0, v0 = d["k_pool"].clone(), d["v_pool"].clone()
    out = torch.empty((w.batch, 32, 64), dtype=torch.float32, device="cuda")

    def step():
        gpu.decode_step_static(d["q"], d["k_pool"], d["v_pool"], d["bt"], d["pos"], d["k_new"], d["v_new"], out,
                               partition_pages=16)

    step()
    torch.cuda.synchronize()
    eager, ek, ev = out.clone(), d["k_pool"].clone(), d["v_pool"].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        d["k_pool"].copy_(k0)
        d["v_pool"].copy_(v0)
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


def test_static_scratch_rejects_oversized_split(gpu):
    import torch

    w = make_custom(seed=83, lengths=[64] * 64)
    d = _inputs(w)
    out = torch.empty((w.batch, 32, 64), dtype=torch.float32, device="cuda")
    assert gpu.decode_workspace_bytes(w.batch, 32, w.max_blocks, 4) > gpu.STATIC_SCRATCH_BYTES
    before = bf16_to_bits(d["k_pool"])
    with pytest.raises(gpu.PagedKVError, match="SCRATCH"):
        gpu.decode_step_static(d["q"], d["k_pool"], d["v_pool"], d["bt"], d["pos"], d["k_new"], d["v_new"], out,
                               partition_pages=4)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_bits(d["k_pool"]), before)  # nothing was launched
