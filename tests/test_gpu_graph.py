"""The decode step (append + attention, split and unsplit) and the prefill step (append +
causal attention) captured in a HIP graph and replayed.

Each replay is checked against the eager result, with eager work and synchronisations between
replays, as graph-replay bugs can show only after the first replay.
"""

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, bf16_to_bits, layer_tensors, to_gpu_bf16, to_gpu_i32, upload
from workloads import f32_to_bf16_bits, make_config, make_custom, make_prefill

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
    ws = torch.zeros(max(16, gpu.decode_workspace_bytes(w.batch, 32, w.max_blocks, pp)), dtype=torch.uint8, device="cuda")

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


@pytest.mark.parametrize("form", ["fused", "two-call"])
def test_model16_whole_step_graph(gpu, form):
    """The 16-layer model step (one 128 MiB pool shared by all layers, each layer with its own
    block table, q and new K/V rows, one workspace shared by every layer) captured as ONE HIP graph
    in the launch configuration bench.py times (partition plan from the longest context), then
    replayed three times with the pools restored and the outputs scribbled over in between.  Every
    replay equals the eager step bit for bit; the eager step's pools equal the oracle's appends
    applied layer by layer and every layer's output is within tolerance of the oracle."""
    import torch

    w = make_config("model16")
    pp = gpu.plan_partition_pages(w.batch, 8, w.max_blocks, max_context=int(w.context_lens.max()))
    print(f"[graph] model16 form={form} B={w.batch} layers={w.layers} partition_pages={pp}", flush=True)
    kp, vp = to_gpu_bf16(w.k_pool), to_gpu_bf16(w.v_pool)
    k0, v0 = kp.clone(), vp.clone()
    pos, lens = to_gpu_i32(w.positions), to_gpu_i32(w.context_lens)
    layers = [layer_tensors(w, layer) for layer in range(w.layers)]
    outs = [torch.empty((w.batch, 32, 64), dtype=torch.float32, device="cuda") for _ in layers]
    ws = torch.zeros(max(16, gpu.decode_workspace_bytes(w.batch, 32, w.max_blocks, pp)), dtype=torch.uint8,
                     device="cuda")
    if form == "fused":
        prepared = [gpu.PreparedDecodeStep(t["q"], kp, vp, t["block_tables"], pos, t["k_new"], t["v_new"], o,
                                           partition_pages=pp, workspace=ws) for t, o in zip(layers, outs)]

        def step():
            for s in prepared:
                s()
    else:
        def step():  # as bench.py runs it: every layer's append, then every layer's attention
            for t in layers:
                gpu.kv_append(kp, vp, t["block_tables"], pos, t["k_new"], t["v_new"])
            for t, o in zip(layers, outs):
                gpu.paged_decode_attention(t["q"], kp, vp, t["block_tables"], lens, o, partition_pages=pp,
                                           workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = [o.cpu().numpy() for o in outs]
    ek, ev = bf16_to_bits(kp), bf16_to_bits(vp)
    rk, rv = w.k_pool, w.v_pool
    for layer in range(w.layers):
        rk, rv = oracle.kv_append(rk, rv, w.block_tables[layer], w.positions, w.k_new[layer], w.v_new[layer])
        ref = oracle.paged_decode_attention(w.q[layer], rk, rv, w.block_tables[layer], w.context_lens)
        assert_close(eager[layer], ref, f"model16 {form} layer {layer}")
    assert np.array_equal(ek, rk) and np.array_equal(ev, rv)

    kp.copy_(k0)
    vp.copy_(v0)
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
        kp.copy_(k0)
        vp.copy_(v0)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for layer, o in enumerate(outs):
            assert np.array_equal(o.cpu().numpy(), eager[layer]), f"replay {replay} layer {layer}"
        assert np.array_equal(bf16_to_bits(kp), ek) and np.array_equal(bf16_to_bits(vp), ev), f"replay {replay} pools"


@pytest.mark.parametrize("wide", [False, True])
def test_prefill_graph_replay_matches_eager(gpu, wide):
    """Prefill append + attention captured once and replayed: every replay equals the eager run
    bit for bit (pools and output).  `wide` plants a V value past FP16's range, so the attention
    takes its BF16 second pass inside the graph too."""
    import torch

    lens, starts = [200, 37, 96, 1], [0, 40, 300, 7]
    w = make_prefill(55, lens, starts)
    if wide:
        v_new = w.v_new.copy()
        v_new[int(w.cu_seqlens[2]) + 10, 3, 5] = f32_to_bf16_bits(np.array([3e5], dtype=np.float32))[0]
        w.v_new = v_new
    print(f"[graph] prefill lens={lens} starts={starts} wide={wide}", flush=True)
    kp, vp = to_gpu_bf16(w.k_pool), to_gpu_bf16(w.v_pool)
    k0, v0 = kp.clone(), vp.clone()
    bt, cu, st = to_gpu_i32(w.block_tables), to_gpu_i32(w.cu_seqlens), to_gpu_i32(w.start_pos)
    q, kn, vn = to_gpu_bf16(w.q), to_gpu_bf16(w.k_new), to_gpu_bf16(w.v_new)
    mpl = max(lens)
    out_eager = torch.empty((w.tokens, 32, 64), dtype=torch.float32, device="cuda")
    out_graph = torch.empty_like(out_eager)

    def step(out):
        gpu.prefill_kv_append(kp, vp, bt, cu, st, kn, vn, max_prompt_len=mpl)
        gpu.paged_prefill_attention(q, kp, vp, bt, cu, st, out, max_prompt_len=mpl)

    step(out_eager)
    torch.cuda.synchronize()
    eager = out_eager.cpu().numpy()
    rk, rv = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new,
                                      w.v_new)
    assert_close(eager, oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos),
                 "eager prefill")

    kp.copy_(k0)
    vp.copy_(v0)
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
        kp.copy_(k0)
        vp.copy_(v0)
        out_graph.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_graph.cpu().numpy(), eager), f"replay {replay}"
        assert np.array_equal(bf16_to_bits(kp), rk), f"replay {replay} K pool"
        assert np.array_equal(bf16_to_bits(vp), rv), f"replay {replay} V pool"
