"""GPU parity: the HIP path through the C ABI against the FP64 oracle on the same seeded inputs.

kv_append must be bit-exact over the whole pool.  Attention (FP32 output) must satisfy
|gpu - oracle| <= 2e-3 + 1e-2 |oracle| elementwise, and the BF16 output must be the
round-to-nearest-even of the FP32 output bit for bit.
"""

import os

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, bf16_to_bits, layer_tensors, to_gpu_bf16, to_gpu_i32, upload
from workloads import f32_to_bf16_bits, make_config, make_custom

pytestmark = pytest.mark.gpu

CONFIGS = ["tiny", "long", "mixed", "model16", "bw256", "bw256tp8"]
NAN_BITS = np.uint16(0x7FC0)

_cache = {}


def config(name):
    if name not in _cache:
        _cache.clear()  # keep at most one large workload alive
        _cache[name] = make_config(name)
    return _cache[name]


def sampled_rows(w):
    """All sequences up to 256 (the oracle takes ~20 ms per 2048-token sequence); beyond that 24
    spread-out rows."""
    if w.batch <= 256:
        return None
    rng = np.random.default_rng(1234)
    rows = set([0, w.batch - 1]) | set(rng.choice(w.batch, size=22, replace=False).tolist())
    return sorted(rows)


def attend(gpu, q, kp, vp, bt, lens, **kw):
    import torch

    kw.setdefault("out_dtype", torch.float32)
    return gpu.paged_decode_attention(q, kp, vp, bt, lens, **kw)


@pytest.mark.parametrize("name", CONFIGS)
def test_append_bit_exact(gpu, name):
    import torch

    w = config(name)
    print(f"[append] config={name} B={w.batch} layers={w.layers} pages={w.num_pages}", flush=True)
    kp, vp = to_gpu_bf16(w.k_pool), to_gpu_bf16(w.v_pool)
    pos = to_gpu_i32(w.positions)
    ref_k, ref_v = w.k_pool, w.v_pool
    for layer in range(w.layers):
        t = layer_tensors(w, layer)
        gpu.kv_append(kp, vp, t["block_tables"], pos, t["k_new"], t["v_new"])
        ref_k, ref_v = oracle.kv_append(ref_k, ref_v, w.block_tables[layer], w.positions, w.k_new[layer], w.v_new[layer])
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_bits(kp), ref_k)
    assert np.array_equal(bf16_to_bits(vp), ref_v)


@pytest.mark.parametrize("name", CONFIGS)
def test_attention_parity(gpu, name):
    """Append, then attend over L = pos + 1 (the new token included), every layer."""
    import torch

    w = config(name)
    rows = sampled_rows(w)
    print(f"[attention] config={name} B={w.batch} layers={w.layers} rows={rows}", flush=True)
    kp, vp = to_gpu_bf16(w.k_pool), to_gpu_bf16(w.v_pool)
    pos, lens = to_gpu_i32(w.positions), to_gpu_i32(w.context_lens)
    ref_k, ref_v = w.k_pool, w.v_pool
    for layer in range(w.layers):
        t = layer_tensors(w, layer)
        gpu.kv_append(kp, vp, t["block_tables"], pos, t["k_new"], t["v_new"])
        out32 = attend(gpu, t["q"], kp, vp, t["block_tables"], lens)
        out16 = attend(gpu, t["q"], kp, vp, t["block_tables"], lens, out_dtype=torch.bfloat16)
        # the plan bench.py times: from the longest context, which the host knows
        out_bench = attend(gpu, t["q"], kp, vp, t["block_tables"], lens, max_context=int(w.context_lens.max()))
        torch.cuda.synchronize()
        ref_k, ref_v = oracle.kv_append(ref_k, ref_v, w.block_tables[layer], w.positions, w.k_new[layer], w.v_new[layer])
        ref = oracle.paged_decode_attention(w.q[layer], ref_k, ref_v, w.block_tables[layer], w.context_lens, 0.125,
                                            sequences=rows)
        got = out32.cpu().numpy()
        sel = slice(None) if rows is None else rows
        abs_err, rel_err = assert_close(got[sel], ref[sel], f"{name} layer {layer}")
        print(f"  layer {layer}: max abs {abs_err:.3e}, max rel {rel_err:.3e}", flush=True)
        assert_close(out_bench.cpu().numpy()[sel], ref[sel], f"{name} layer {layer}, bench plan")
        assert np.array_equal(bf16_to_bits(out16), oracle.bf16_round_nearest_even(got))


RAGGED = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000, 2047, 2048]


@pytest.mark.parametrize("partition_pages", [0, 4, 8, 12, 128])
def test_ragged_lengths_and_splits(gpu, partition_pages):
    w = make_custom(seed=21, lengths=RAGGED)
    d = upload(w)
    print(f"[ragged] partition_pages={partition_pages}", flush=True)
    out = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                 partition_pages=partition_pages)
    ref = oracle.paged_decode_attention(w.q[0], w.k_pool, w.v_pool, w.block_tables[0], w.context_lens)
    assert_close(out.cpu().numpy(), ref, f"ragged pp={partition_pages}")


def test_known_longest_context_plans_no_split(gpu):
    """With the longest context known on the host, a batch that fits one partition runs unsplit:
    the result is the unsplit kernel's bit for bit, and a context longer than the bound is still
    attended correctly through partitions."""
    w = make_custom(seed=23, lengths=[37, 5, 100, 128])
    d = upload(w)
    args = (gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"])
    assert gpu.plan_partition_pages(w.batch, 8, w.max_blocks, max_context=128) == w.max_blocks
    planned = attend(*args, max_context=128)
    unsplit = attend(*args, partition_pages=w.max_blocks)
    assert np.array_equal(planned.cpu().numpy(), unsplit.cpu().numpy())
    ref = oracle.paged_decode_attention(w.q[0], w.k_pool, w.v_pool, w.block_tables[0], w.context_lens)
    assert_close(planned.cpu().numpy(), ref, "planned with max_context")
    low = attend(*args, max_context=1)  # a wrong (too small) bound changes only the launch shape
    assert_close(low.cpu().numpy(), ref, "bound below the real context")


@pytest.mark.parametrize("partition_pages", [0, 2])
def test_large_batch_of_short_contexts(gpu, partition_pages):
    """4096 sequences of 1..64 tokens: a grid of 32768 (sequence, KV head) workgroups unsplit, or
    twice that with 2-page partitions and the merge, against the oracle on every sequence."""
    import torch

    rng = np.random.default_rng(55)
    lengths = rng.integers(1, 65, size=4096).tolist()
    w = make_custom(seed=56, lengths=lengths, max_blocks=4)
    print(f"[large batch] B={w.batch} pages={w.num_pages} partition_pages={partition_pages}", flush=True)
    d = upload(w)
    gpu.kv_append(d["k_pool"], d["v_pool"], d["block_tables"], d["positions"], d["k_new"], d["v_new"])
    out = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                 partition_pages=partition_pages)
    torch.cuda.synchronize()
    rk, rv = oracle.kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.k_new[0], w.v_new[0])
    assert np.array_equal(bf16_to_bits(d["k_pool"]), rk) and np.array_equal(bf16_to_bits(d["v_pool"]), rv)
    ref = oracle.paged_decode_attention(w.q[0], rk, rv, w.block_tables[0], w.context_lens)
    assert_close(out.cpu().numpy(), ref, f"large batch pp={partition_pages}")


def test_split_matches_unsplit(gpu):
    w = make_custom(seed=22, lengths=[3, 100, 700, 2048, 1500, 64])
    d = upload(w)
    base = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"], partition_pages=128)
    for pp in (4, 16, 20, 64):
        other = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"], partition_pages=pp)
        diff = (base - other).abs().max().item()
        assert diff <= 1e-5, f"partition_pages={pp}: {diff}"


def test_single_token_returns_v_row_exactly(gpu):
    """L = 1: the only probability is exactly 1, so the FP32 output is the appended V row."""
    import torch

    w = make_custom(seed=23, lengths=[1, 1, 1])
    d = upload(w)
    gpu.kv_append(d["k_pool"], d["v_pool"], d["block_tables"], d["positions"], d["k_new"], d["v_new"])
    out = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"])
    torch.cuda.synchronize()
    expect = oracle.bf16_bits_to_f64(w.v_new[0]).astype(np.float32)  # [B][Hkv][D]
    got = out.cpu().numpy()
    for h in range(32):
        assert np.array_equal(got[:, h], expect[:, h // 4]), f"head {h}"


def test_equal_scores_give_mean_of_values(gpu):
    """q = 0: every probability is equal and the output is the plain mean of the V rows."""
    w = make_custom(seed=24, lengths=[5, 77, 300])
    w.q[:] = 0
    d = upload(w)
    out = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"]).cpu().numpy()
    for b, L in enumerate(w.context_lens):
        vals = oracle.bf16_bits_to_f64(oracle.gather_context(w.v_pool, w.block_tables[0, b], int(L)))
        mean = vals.mean(axis=0)  # [Hkv][D]
        for h in range(32):
            assert np.max(np.abs(out[b, h] - mean[h // 4])) <= 1e-5


@pytest.mark.parametrize("batch,partition_pages", [(24, 128), (24, 4), (24, 0), (48, 0)])
@pytest.mark.parametrize("offset", [0, 8, 40, 72])
def test_one_key_far_above_the_rest(gpu, batch, partition_pages, offset):
    """Sequence b's key at token offset + b (in every KV head) is 100 e_0 and every query is
    100 e_0, so that key scores (100 * 100 / 8) log2(e) ~ 1803 in log2 units while every other key
    scores |100 k_0 / 8| log2(e) ~ 18 |k_0| (k_0 ~ N(0, 1)): the output is that key's V row. The
    planted keys sit at every token slot of a two-page step (offset 0 and 8: the first step, 40: the
    second, 72: the third, which 4-page partitions put in the second partition, so the merge has to
    drop the first partition's sum by 2^-1700), so a running maximum that missed any slot's score
    would put 2^1700 into an FP32 weight. batch 24 runs the matrix-core kernel (unsplit, split in
    4-page partitions, the planner's choice), batch 48 the VALU kernel. Contexts are 128 tokens."""
    w = make_custom(seed=60 + offset + batch, lengths=[128] * batch)
    hundred = f32_to_bf16_bits(np.array([100.0], dtype=np.float32))[0]
    w.q[:] = 0
    w.q[..., 0] = hundred
    planted = [offset + b for b in range(batch)]
    for b, t in enumerate(planted):
        page, slot = int(w.block_tables[0, b, t // 16]), t % 16
        w.k_pool[page, :, slot, :] = 0
        w.k_pool[page, :, slot, 0] = hundred
    print(f"[attention] one key far above the rest: B={batch} pp={partition_pages} offset={offset}", flush=True)
    d = upload(w)
    out = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                 partition_pages=partition_pages).cpu().numpy()
    ref = oracle.paged_decode_attention(w.q[0], w.k_pool, w.v_pool, w.block_tables[0], w.context_lens, 0.125)
    for b, t in enumerate(planted):  # the oracle's output is the planted key's V row
        v_row = oracle.bf16_bits_to_f64(w.v_pool[int(w.block_tables[0, b, t // 16]), :, t % 16, :])
        assert np.allclose(ref[b], np.repeat(v_row, 4, axis=0), rtol=0, atol=1e-12)
    assert_close(out, ref, f"one dominant key, B={batch} pp={partition_pages} offset={offset}")


def test_page_permutation_bit_identical(gpu):
    """Renaming physical pages (moving their contents along) leaves the output bit-identical."""
    w = make_custom(seed=25, lengths=[9, 160, 600, 33], num_pages=64)
    d = upload(w)
    base = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"])
    perm = np.random.default_rng(3).permutation(w.num_pages)
    k2 = np.empty_like(w.k_pool)
    v2 = np.empty_like(w.v_pool)
    k2[perm] = w.k_pool
    v2[perm] = w.v_pool
    bt2 = np.where(w.block_tables[0] >= 0, perm[np.maximum(w.block_tables[0], 0)], -1)
    moved = attend(gpu, d["q"], to_gpu_bf16(k2), to_gpu_bf16(v2), to_gpu_i32(bt2), d["context_lens"])
    assert np.array_equal(base.cpu().numpy(), moved.cpu().numpy())


def poison_outside_context(w, layer=0):
    keep = np.zeros((w.num_pages, 16), dtype=bool)
    for b in range(w.batch):
        for t in range(int(w.context_lens[b])):
            keep[w.block_tables[layer, b, t // 16], t % 16] = True
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    kp.transpose(0, 2, 1, 3)[~keep] = NAN_BITS
    vp.transpose(0, 2, 1, 3)[~keep] = NAN_BITS
    return kp, vp


@pytest.mark.parametrize("partition_pages", [0, 128])
def test_nan_outside_context_changes_nothing(gpu, partition_pages):
    w = make_custom(seed=26, lengths=[1, 7, 16, 17, 250, 1023], num_pages=120)
    d = upload(w)
    clean = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                   partition_pages=partition_pages).cpu().numpy()
    kp, vp = poison_outside_context(w)
    dirty = attend(gpu, d["q"], to_gpu_bf16(kp), to_gpu_bf16(vp), d["block_tables"], d["context_lens"],
                   partition_pages=partition_pages).cpu().numpy()
    assert np.all(np.isfinite(dirty))
    assert np.array_equal(clean, dirty)


def test_append_into_nan_pool_touches_only_targets(gpu):
    import torch

    w = make_custom(seed=27, lengths=[1, 16, 17, 40, 33, 2048], num_pages=200)
    kp = np.full_like(w.k_pool, NAN_BITS)
    vp = np.full_like(w.v_pool, NAN_BITS)
    dk, dv = to_gpu_bf16(kp), to_gpu_bf16(vp)
    gpu.kv_append(dk, dv, to_gpu_i32(w.block_tables[0]), to_gpu_i32(w.positions), to_gpu_bf16(w.k_new[0]),
                  to_gpu_bf16(w.v_new[0]))
    torch.cuda.synchronize()
    rk, rv = oracle.kv_append(kp, vp, w.block_tables[0], w.positions, w.k_new[0], w.v_new[0])
    assert np.array_equal(bf16_to_bits(dk), rk)
    assert np.array_equal(bf16_to_bits(dv), rv)


def test_zero_length_rows_are_zero(gpu):
    w = make_custom(seed=28, lengths=[0, 5, 0, 40])
    d = upload(w)
    for pp in (0, 4, 128):
        out = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                     partition_pages=pp).cpu().numpy()
        assert np.all(out[0] == 0) and np.all(out[2] == 0)
        ref = oracle.paged_decode_attention(w.q[0], w.k_pool, w.v_pool, w.block_tables[0], w.context_lens)
        assert_close(out, ref, f"zero-length pp={pp}")


@pytest.mark.parametrize("partition_pages", [4, 128])
@pytest.mark.parametrize("bad_entry", [-1, "num_pages", 1 << 30])
def test_invalid_page_id_zeroes_only_that_sequence(gpu, partition_pages, bad_entry):
    """An out-of-range table entry inside a context is never dereferenced: that sequence's output
    is zero and the other sequences are unchanged."""
    w = make_custom(seed=29, lengths=[70, 300, 45])
    d = upload(w)
    good = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                  partition_pages=partition_pages).cpu().numpy()
    bt = w.block_tables[0].copy()
    bt[1, 13] = w.num_pages if bad_entry == "num_pages" else bad_entry
    out = attend(gpu, d["q"], d["k_pool"], d["v_pool"], to_gpu_i32(bt), d["context_lens"],
                 partition_pages=partition_pages).cpu().numpy()
    assert np.all(out[1] == 0)
    assert np.array_equal(out[0], good[0]) and np.array_equal(out[2], good[2])


@pytest.mark.parametrize("partition_pages", [0, 4, 128])
def test_table_entries_past_the_context_are_ignored(gpu, partition_pages):
    """The kernel reads each wavefront's table entries before it knows the context length (every
    read stays inside the row of max_blocks entries); entries past a sequence's own pages must
    change nothing, whatever they hold: out-of-range values give bit-identical outputs and pools,
    for the attention call and for the fused step."""
    import torch

    w = make_custom(seed=37, lengths=[1, 16, 17, 300, 2047, 0])
    junk = np.array([-1, w.num_pages, 1 << 30, -(1 << 31), (1 << 31) - 1], dtype=np.int64)
    bt = w.block_tables[0].astype(np.int64)
    dirty_bt = bt.copy()
    for b, n in enumerate(w.context_lens):
        used = (int(n) + 15) // 16
        tail = dirty_bt[b, used:]
        tail[:] = junk[np.arange(tail.size) % junk.size]
    print(f"[parity] junk past the context, partition_pages={partition_pages}", flush=True)
    d = upload(w)
    clean = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                   partition_pages=partition_pages)
    dirty = attend(gpu, d["q"], d["k_pool"], d["v_pool"], to_gpu_i32(dirty_bt), d["context_lens"],
                   partition_pages=partition_pages)
    torch.cuda.synchronize()
    assert torch.equal(clean, dirty)
    # fused step: its context is positions + 1 = context_lens (the workloads' convention), so the
    # same entries lie past it
    assert np.array_equal(w.positions + 1, w.context_lens)
    d1, d2 = upload(w), upload(w)
    a = gpu.decode_step(d1["q"], d1["k_pool"], d1["v_pool"], d1["block_tables"], d1["positions"], d1["k_new"],
                        d1["v_new"], out_dtype=torch.float32, partition_pages=partition_pages)
    b = gpu.decode_step(d2["q"], d2["k_pool"], d2["v_pool"], to_gpu_i32(dirty_bt), d2["positions"], d2["k_new"],
                        d2["v_new"], out_dtype=torch.float32, partition_pages=partition_pages)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(d1["k_pool"], d2["k_pool"]) and torch.equal(d1["v_pool"], d2["v_pool"])


def test_invalid_context_length_zeroes_sequence(gpu):
    w = make_custom(seed=30, lengths=[20, 50])
    d = upload(w)
    for bad_len in (-3, 128 * 16 + 1):
        lens = w.context_lens.copy()
        lens[0] = bad_len
        for pp in (4, 128):
            out = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], to_gpu_i32(lens),
                         partition_pages=pp).cpu().numpy()
            assert np.all(out[0] == 0)
            assert np.all(np.isfinite(out[1])) and np.any(out[1] != 0)


def test_append_skips_out_of_range_rows(gpu):
    import torch

    w = make_custom(seed=31, lengths=[10, 20, 30])
    pos = w.positions.copy()
    pos[0] = -1
    pos[2] = 128 * 16
    bt = w.block_tables[0].copy()
    bt[1, 1] = -1  # position 19 -> block 1 unassigned
    d = upload(w)
    gpu.kv_append(d["k_pool"], d["v_pool"], to_gpu_i32(bt), to_gpu_i32(pos), d["k_new"], d["v_new"])
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_bits(d["k_pool"]), w.k_pool)
    assert np.array_equal(bf16_to_bits(d["v_pool"]), w.v_pool)


def test_out_of_range_rows_match_the_oracle(gpu):
    """A batch mixing valid rows with every kind of out-of-range row (negative position, position
    past the table, entry -1, entry past the pool, empty sequence): the append, the attention on
    both paths and the fused step all equal the oracle, which skips such rows and zeroes such
    sequences."""
    import torch

    w = make_custom(seed=33, lengths=[10, 20, 30, 0, 40, 50, 17])
    pos = w.positions.copy()
    bt = w.block_tables[0].copy()
    pos[1] = -5
    pos[2] = 128 * 16
    bt[4, 2] = -1  # position 39 -> block 2 unassigned
    bt[5, 3] = w.num_pages  # position 49 -> block 3 past the pool
    lens = np.where(pos >= 0, pos + 1, 0)
    lens[2] = 128 * 16 + 1  # past the table's span
    print(f"[out of range] positions={pos.tolist()} lens={lens.tolist()}", flush=True)
    rk, rv = oracle.kv_append(w.k_pool, w.v_pool, bt, pos, w.k_new[0], w.v_new[0])
    ref = oracle.paged_decode_attention(w.q[0], rk, rv, bt, lens)
    assert np.all(ref[[1, 2, 3, 4, 5]] == 0) and np.all(ref[[0, 6]] != 0)
    d = upload(w)
    gpu.kv_append(d["k_pool"], d["v_pool"], to_gpu_i32(bt), to_gpu_i32(pos), d["k_new"], d["v_new"])
    outs = [attend(gpu, d["q"], d["k_pool"], d["v_pool"], to_gpu_i32(bt), to_gpu_i32(lens), partition_pages=pp)
            for pp in (4, 128)]
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_bits(d["k_pool"]), rk) and np.array_equal(bf16_to_bits(d["v_pool"]), rv)
    for pp, out in zip((4, 128), outs):
        assert_close(out.cpu().numpy(), ref, f"out of range pp={pp}")
    f = upload(w)
    fused = gpu.decode_step(f["q"], f["k_pool"], f["v_pool"], to_gpu_i32(bt), to_gpu_i32(pos), f["k_new"], f["v_new"],
                            out_dtype=torch.float32, partition_pages=4)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_bits(f["k_pool"]), rk) and np.array_equal(bf16_to_bits(f["v_pool"]), rv)
    # the fused step attends over positions + 1 tokens: the same contexts as `lens`
    assert_close(fused.cpu().numpy(), ref, "fused out of range")


def test_debug_validation_rejects_bad_data(gpu):
    import torch

    w = make_custom(seed=32, lengths=[10, 20])
    d = upload(w)
    bt = w.block_tables[0].copy()
    bt[1, 0] = -1
    os.environ["PKV_DEBUG_VALIDATE"] = "1"
    try:
        gpu.kv_append(d["k_pool"], d["v_pool"], d["block_tables"], d["positions"], d["k_new"], d["v_new"])
        attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"])
        with pytest.raises(gpu.PagedKVError, match="PKV_ERR_VALIDATION"):
            attend(gpu, d["q"], d["k_pool"], d["v_pool"], to_gpu_i32(bt), d["context_lens"])
        same = w.positions.copy()
        same[1] = same[0]
        bt2 = w.block_tables[0].copy()
        bt2[1, 0] = bt2[0, 0]
        with pytest.raises(gpu.PagedKVError, match="PKV_ERR_VALIDATION"):
            gpu.kv_append(d["k_pool"], d["v_pool"], to_gpu_i32(bt2), to_gpu_i32(same), d["k_new"], d["v_new"])
    finally:
        del os.environ["PKV_DEBUG_VALIDATE"]
    torch.cuda.synchronize()


def test_table_wider_than_one_partition(gpu):
    """A 300-entry table with partition_pages=300: a partition holds at most 256 pages (four
    wavefronts with one table entry per lane), so the request is capped and the 282-page context
    runs as two partitions plus the merge."""
    w = make_custom(seed=33, lengths=[4500, 1100], max_blocks=300)
    d = upload(w)
    out = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"], partition_pages=300)
    ref = oracle.paged_decode_attention(w.q[0], w.k_pool, w.v_pool, w.block_tables[0], w.context_lens)
    assert_close(out.cpu().numpy(), ref, "table wider than one partition")
    split = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"], partition_pages=256)
    assert np.array_equal(split.cpu().numpy(), out.cpu().numpy())  # the same launch


@pytest.mark.parametrize("fused", [False, True])
def test_unsplit_partition_of_256_pages(gpu, fused):
    """The largest unsplit launch: a 256-entry table attended with partition_pages=256, so one
    workgroup per (sequence, KV head) covers the whole table, each wavefront streams up to 64 pages
    (one table entry per lane) and no merge runs.  Contexts fill the table exactly, stop one token
    and one page short of it, and are short."""
    import torch

    lengths = [4096, 4095, 4081, 2000, 17, 1]
    w = make_custom(seed=36, lengths=lengths, max_blocks=256)
    print(f"[parity] unsplit 256-page partition, fused={fused}", flush=True)
    assert gpu.decode_workspace_bytes(w.batch, 32, 256, 256) == 0  # one partition: no workspace
    d = upload(w)
    rk, rv = oracle.kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.k_new[0], w.v_new[0])
    if fused:
        out = gpu.decode_step(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["positions"], d["k_new"],
                              d["v_new"], out_dtype=torch.float32, partition_pages=256)
    else:
        gpu.kv_append(d["k_pool"], d["v_pool"], d["block_tables"], d["positions"], d["k_new"], d["v_new"])
        out = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"], partition_pages=256)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_bits(d["k_pool"]), rk) and np.array_equal(bf16_to_bits(d["v_pool"]), rv)
    ref = oracle.paged_decode_attention(w.q[0], rk, rv, w.block_tables[0], w.context_lens)
    assert_close(out.cpu().numpy(), ref, "unsplit 256 pages")


def test_other_kv_head_counts(gpu):
    """The group of four query heads per KV head is fixed; the number of KV heads is not."""
    for hkv in (1, 2, 5):
        w = make_custom(seed=34 + hkv, lengths=[33, 400, 1], num_kv_heads=hkv)
        d = upload(w)
        gpu.kv_append(d["k_pool"], d["v_pool"], d["block_tables"], d["positions"], d["k_new"], d["v_new"])
        out = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"])
        rk, rv = oracle.kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.k_new[0], w.v_new[0])
        ref = oracle.paged_decode_attention(w.q[0], rk, rv, w.block_tables[0], w.context_lens)
        assert_close(out.cpu().numpy(), ref, f"hkv={hkv}")


def test_runs_on_the_callers_stream(gpu):
    import torch

    w = make_custom(seed=40, lengths=[500, 37])
    d = upload(w)
    ref = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"])
    s.synchronize()
    assert torch.equal(out, ref)


def test_concurrent_streams_do_not_interfere(gpu):
    """The library keeps no per-call state: two streams running split decode steps on different
    data at the same time, each with its own workspace, give what each gives alone."""
    import torch

    wa, wb = make_custom(seed=41, lengths=[2048, 900, 33]), make_custom(seed=42, lengths=[1500, 1, 700, 2048, 64])
    da, db = upload(wa), upload(wb)
    alone = [attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"], partition_pages=8)
             for d in (da, db)]
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = {0: [], 1: []}
    for s in (sa, sb):
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(10):
        for i, (s, d, w) in enumerate(((sa, da, wa), (sb, db, wb))):
            with torch.cuda.stream(s):
                ws = torch.zeros(gpu.decode_workspace_bytes(w.batch, 32, w.max_blocks, 8), dtype=torch.uint8,
                                 device="cuda") if rep == 0 else None
                if rep == 0:
                    outs[i].append(ws)
                outs[i].append(attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                                      partition_pages=8, workspace=outs[i][0]))
    torch.cuda.synchronize()
    for i in (0, 1):
        for out in outs[i][1:]:
            assert torch.equal(out, alone[i])


def test_batch_zero_is_a_no_op(gpu):
    import torch

    e = torch.empty
    kp = e((4, 8, 16, 64), dtype=torch.bfloat16, device="cuda")
    gpu.kv_append(kp, kp.clone(), e((0, 8), dtype=torch.int32, device="cuda"), e((0,), dtype=torch.int32, device="cuda"),
                  e((0, 8, 64), dtype=torch.bfloat16, device="cuda"), e((0, 8, 64), dtype=torch.bfloat16, device="cuda"))
    out = gpu.paged_decode_attention(e((0, 32, 64), dtype=torch.bfloat16, device="cuda"), kp, kp,
                                     e((0, 8), dtype=torch.int32, device="cuda"), e((0,), dtype=torch.int32, device="cuda"))
    assert out.shape == (0, 32, 64)


def test_one_workspace_serves_every_shape(gpu):
    """Calls of different shapes and split sizes share one workspace (as the binding's per-stream
    cache does), twice over: zero-filled once, with garbage (NaN-ish bytes) in the partials area,
    every result matches the oracle and every call leaves the counters at zero for the next."""
    import torch

    cases = [(make_custom(seed=32, lengths=[2048] * 3 + [40]), 8), (make_custom(seed=33, lengths=[1500]), 4),
             (make_custom(seed=34, lengths=[700, 1, 2000, 64, 900]), 12), (make_custom(seed=35, lengths=[2048]), 4)]
    nbytes = max(gpu.decode_workspace_bytes(w.batch, 32, w.max_blocks, pp) for w, pp in cases)
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda")
    for rnd in range(2):
        for w, pp in cases:
            d = upload(w)
            out = gpu.paged_decode_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                                             out_dtype=torch.float32, partition_pages=pp, workspace=ws)
            torch.cuda.synchronize()
            ref = oracle.paged_decode_attention(w.q[0], w.k_pool, w.v_pool, w.block_tables[0], w.context_lens)
            assert_close(out.cpu().numpy(), ref, f"round {rnd} B={w.batch} pp={pp}")
            assert int(torch.count_nonzero(ws)) == 0, f"round {rnd} B={w.batch} pp={pp} left workspace bytes set"


def test_split_workspace_must_start_zeroed(gpu, monkeypatch):
    """Debug validation rejects a split call whose workspace counters are not zero (a workspace
    that was never zero-filled); after a call the workspace is all-zero again."""
    import torch

    w = make_custom(seed=37, lengths=[1500, 700])
    d = upload(w)
    nbytes = gpu.decode_workspace_bytes(w.batch, 32, w.max_blocks, 8)
    ws = torch.full((nbytes,), 0x11, dtype=torch.uint8, device="cuda")
    monkeypatch.setenv("PKV_DEBUG_VALIDATE", "1")
    with pytest.raises(gpu.PagedKVError, match="VALIDATION"):
        gpu.paged_decode_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                                   out_dtype=torch.float32, partition_pages=8, workspace=ws)
    ws.zero_()
    out = gpu.paged_decode_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                                     out_dtype=torch.float32, partition_pages=8, workspace=ws)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws)) == 0
    ref = oracle.paged_decode_attention(w.q[0], w.k_pool, w.v_pool, w.block_tables[0], w.context_lens)
    assert_close(out.cpu().numpy(), ref, "zeroed workspace")


@pytest.mark.parametrize("partition_pages", [0, 4, 8, 128])
@pytest.mark.parametrize("row", ["k", "v"])
def test_nan_inside_the_context_reaches_only_its_kv_group(gpu, partition_pages, row):
    """A NaN K (or V) row at token 100 of sequence 4 (250 tokens, 16 pages), KV head 3: the
    definition makes out[4, 12:16, :] NaN (every score of the group is NaN, or every weighted V row
    is) and leaves every other row finite. Split into 4- or 8-page partitions the NaN K row leaves a
    NaN denominator in one partition, which the merge must carry to the output instead of treating
    the partition as one that met an invalid table entry (zeros); the planner's size (24 pages for
    this 128-entry table) and 128 keep the sequence in one partition."""
    w = make_custom(seed=27, lengths=[1, 7, 16, 17, 250, 1023], num_pages=120)
    b, t, g = 4, 100, 3
    page = int(w.block_tables[0, b, t // 16])
    pool = w.k_pool if row == "k" else w.v_pool
    pool[page, g, t % 16, :] = NAN_BITS
    print(f"[attention] NaN {row} row inside the context, pp={partition_pages}", flush=True)
    d = upload(w)
    out = attend(gpu, d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                 partition_pages=partition_pages).cpu().numpy()
    ref = oracle.paged_decode_attention(w.q[0], w.k_pool, w.v_pool, w.block_tables[0], w.context_lens, 0.125)
    expect = np.zeros(ref.shape, dtype=bool)
    expect[b, 4 * g:4 * g + 4, :] = True
    assert np.array_equal(np.isnan(ref), expect)  # the oracle's own reading of the definition
    assert np.array_equal(np.isnan(out), expect)
    keep = ~expect
    assert_close(np.where(keep, out, 0.0), np.where(keep, ref, 0.0), f"NaN {row} row, pp={partition_pages}")
