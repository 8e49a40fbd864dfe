"""The decode step (append + attention, split and unsplit) captured in a HIP graph and replayed.

Each replay is checked against the eager result, with eager work and synchronisations between
replays, as graph-replay bugs can show only after the first replay.
"""

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, bf16_to_bits, upload
from workloads import make_custom

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("partition_pages", [0, 8, 128])
def test_graph_replay_matches_eager(gpu, partition_pages):
    import torch

    w = make_custom(seed=50, lengths=[1, 17, 300, 2048, 999, 64, 16, 1500])
    d = upload(w)
    k0, v0 = d["k_pool"].clone(), d["v_pool"].clone()
    out_eager = torch.empty((w.batch, 32, 64), dtype=torch.float32, device="cuda")
    out_graph = torch.empty_like(out_eager)
    pp = partition_pages if partition_pages > 0 else gpu.plan_partition_pages(w.batch, 8, w.max_blocks, gpu.cu_count())
    ws = torch.empty(max(16, gpu.decode_workspace_bytes(w.batch, 32, w.max_blocks, pp)), dtype=torch.uint8, device="cuda")

    def step(out):
        gpu.kv_append(d["k_pool"], d["v_pool"], d["block_tables"], d["positions"], d["k_new"], d["v_new"])
        gpu.paged_decode_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"], out,
                                   partition_pages=pp, workspace=ws)

    step(out_eager)
    torch.cuda.synchronize()
    eager = out_eager.cpu().numpy()
    rk, rv = oracle.kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.k_new[0], w.v_new[0])
    assert_close(eager, oracle.paged_decode_attention(w.q[0], rk, rv, w.block_tables[0], w.context_lens), "eager")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out_graph)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(out_graph)
    for replay in range(4):
        # restore the pools and scribble over the output between replays (eager work)
        d["k_pool"].copy_(k0)
        d["v_pool"].copy_(v0)
        out_graph.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_graph.cpu().numpy(), eager), f"replay {replay}"
        assert np.array_equal(bf16_to_bits(d["k_pool"]), rk), f"replay {replay} K pool"
        assert np.array_equal(bf16_to_bits(d["v_pool"]), rv), f"replay {replay} V pool"
