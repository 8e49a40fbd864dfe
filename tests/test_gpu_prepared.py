"""PreparedDecodeStep: the fused step on fixed buffers with cached arguments gives exactly what
decode_step gives, also after the buffers' contents change in place between calls."""

import numpy as np
import pytest

from gpu_helpers import upload
from workloads import make_custom

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("partition_pages", [0, 4])
def test_prepared_step_equals_decode_step(gpu, partition_pages):
    import torch

    w1 = make_custom(seed=81, lengths=[300, 2048, 17, 1], num_pages=200)
    w2 = make_custom(seed=82, lengths=[1000, 5, 640, 33], num_pages=200)
    d = upload(w1)
    ref_pools = (d["k_pool"].clone(), d["v_pool"].clone())
    out = torch.empty((w1.batch, 32, 64), dtype=torch.float32, device="cuda")
    step = gpu.PreparedDecodeStep(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["positions"], d["k_new"],
                                  d["v_new"], out, partition_pages=partition_pages, max_context=2048)
    got1 = step().clone()
    ref1 = gpu.decode_step(d["q"], ref_pools[0], ref_pools[1], d["block_tables"], d["positions"], d["k_new"],
                           d["v_new"], out_dtype=torch.float32, partition_pages=step.partition_pages)
    torch.cuda.synchronize()
    assert torch.equal(got1, ref1)
    assert torch.equal(d["k_pool"], ref_pools[0]) and torch.equal(d["v_pool"], ref_pools[1])
    # new contents in the same buffers (same shapes): the prepared step reads them at launch
    d2 = upload(w2)
    for name in ("k_pool", "v_pool", "block_tables", "positions", "q", "k_new", "v_new"):
        d[name].copy_(d2[name])
    got2 = step().clone()
    ref2 = gpu.decode_step(d2["q"], d2["k_pool"], d2["v_pool"], d2["block_tables"], d2["positions"], d2["k_new"],
                           d2["v_new"], out_dtype=torch.float32, partition_pages=step.partition_pages)
    torch.cuda.synchronize()
    assert torch.equal(got2, ref2)
    assert torch.equal(d["k_pool"], d2["k_pool"]) and torch.equal(d["v_pool"], d2["v_pool"])
    assert not torch.equal(got1, got2)


def test_prepared_step_in_a_graph(gpu):
    """Without an explicit stream the prepared step launches on the stream current at the call,
    so it records into a HIP graph; replays after in-place updates of q match eager calls."""
    import torch

    w = make_custom(seed=83, lengths=[700, 64, 2048], num_pages=200)
    d = upload(w)
    out = torch.empty((w.batch, 32, 64), dtype=torch.float32, device="cuda")
    step = gpu.PreparedDecodeStep(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["positions"], d["k_new"],
                                  d["v_new"], out, partition_pages=8)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    gen = torch.Generator(device="cuda").manual_seed(5)
    for rep in range(4):
        d["q"].copy_(torch.randn(d["q"].shape, device="cuda", generator=gen).to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = gpu.decode_step(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["positions"], d["k_new"],
                              d["v_new"], out_dtype=torch.float32, partition_pages=8)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {rep}"
