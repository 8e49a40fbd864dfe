"""Paged prefill through the C ABI against the FP64 prefill oracle: the append bit for bit, the
causal attention within the decode tolerance on every output row, in each launch shape the
library picks (including the 16 x 512 launch the bench times), plus ragged lengths, cached
prefixes and the error behaviour."""

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, bf16_to_bits, to_gpu_bf16, to_gpu_i32
from workloads import f32_to_bf16_bits, make_prefill, make_prefill_config

pytestmark = pytest.mark.gpu
NAN = np.uint16(0x7FC0)


def upload(w):
    return {
        "k_pool": to_gpu_bf16(w.k_pool),
        "v_pool": to_gpu_bf16(w.v_pool),
        "block_tables": to_gpu_i32(w.block_tables),
        "cu_seqlens": to_gpu_i32(w.cu_seqlens),
        "start_pos": to_gpu_i32(w.start_pos),
        "q": to_gpu_bf16(w.q),
        "k_new": to_gpu_bf16(w.k_new),
        "v_new": to_gpu_bf16(w.v_new),
    }


def run(gpu, d, out_dtype, max_prompt_len=None):
    gpu.prefill_kv_append(d["k_pool"], d["v_pool"], d["block_tables"], d["cu_seqlens"], d["start_pos"], d["k_new"],
                          d["v_new"], max_prompt_len=max_prompt_len)
    return gpu.paged_prefill_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["cu_seqlens"],
                                       d["start_pos"], out_dtype=out_dtype, max_prompt_len=max_prompt_len)


def launch_shape(cus, batch, max_prompt_len, kv_heads=8):
    """The attention launch the library picks (its documented rule): with G groups of 32 query
    rows, 32-row tiles in 32-key steps from 4 groups per compute unit, 32-row tiles in 64-key steps
    from 2, else 16-row tiles in 64-key steps."""
    groups = (max_prompt_len + 31) // 32 * batch * kv_heads
    if groups >= 4 * cus:
        return "32 rows, 32-key steps"
    return "32 rows, 64-key steps" if groups >= 2 * cus else "16 rows, 64-key steps"


@pytest.mark.parametrize("name", ["prefill_tiny", "prefill512", "prefill_chunked", "prefill16x512"])
def test_prefill_matches_oracle(gpu, name):
    """Every output row of every named workload, in the launch shape the library picks for it
    (on a 256-CU part: prefill16x512, the bench's workload, takes 32-row tiles in 32-key steps,
    prefill_chunked 32-row tiles in 64-key steps, the two single prompts 16-row tiles)."""
    import torch

    w = make_prefill_config(name)
    mpl = int(w.prompt_lens.max())
    shape = launch_shape(gpu.cu_count(), w.batch, mpl)
    print(f"[prefill] config={name} B={w.batch} tokens={w.tokens} launch={shape}", flush=True)
    d = upload(w)
    out = run(gpu, d, torch.float32, max_prompt_len=mpl)
    torch.cuda.synchronize()
    rk, rv = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new, w.v_new)
    assert np.array_equal(bf16_to_bits(d["k_pool"]), rk) and np.array_equal(bf16_to_bits(d["v_pool"]), rv)
    ref = oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos)
    assert not np.isnan(ref).any()
    got = out.cpu().numpy()
    assert_close(got, ref, name)
    # BF16 output is the round-to-nearest-even of the FP32 output
    out_bf = gpu.paged_prefill_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["cu_seqlens"],
                                         d["start_pos"], out_dtype=torch.bfloat16, max_prompt_len=mpl)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_bits(out_bf), bf16_to_bits(out.to(torch.bfloat16)))


def test_prefill_ragged_lengths_and_prefixes(gpu):
    import torch

    lens = [1, 15, 16, 17, 31, 32, 33, 47, 64, 100]
    starts = [0, 5, 16, 3, 0, 31, 32, 200, 1, 0]
    w = make_prefill(21, lens, starts)
    print(f"[prefill] ragged lens={lens} starts={starts}", flush=True)
    d = upload(w)
    out = run(gpu, d, torch.float32, max_prompt_len=128)  # a bound above every length
    torch.cuda.synchronize()
    rk, rv = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new, w.v_new)
    assert np.array_equal(bf16_to_bits(d["k_pool"]), rk) and np.array_equal(bf16_to_bits(d["v_pool"]), rv)
    ref = oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos)
    assert_close(out.cpu().numpy(), ref, "ragged")


def test_prefill_many_ragged_prompts(gpu):
    """Enough prompts that the launch takes two 16-query blocks per wavefront (at least two
    workgroups per compute unit), with ragged lengths so the second block is often partial."""
    import torch

    rng = np.random.default_rng(40)
    lens = [int(x) for x in rng.integers(1, 200, size=24)] + [1, 16, 17, 32, 33]
    starts = [int(x) for x in rng.integers(0, 600, size=len(lens))]
    w = make_prefill(41, lens, starts)
    print(f"[prefill] many ragged prompts B={w.batch} tokens={w.tokens}", flush=True)
    d = upload(w)
    out = run(gpu, d, torch.float32)
    torch.cuda.synchronize()
    rk, rv = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new, w.v_new)
    assert np.array_equal(bf16_to_bits(d["k_pool"]), rk) and np.array_equal(bf16_to_bits(d["v_pool"]), rv)
    ref = oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos)
    assert_close(out.cpu().numpy(), ref, "many ragged")


def test_prefill_rows_equal_decode_kernel(gpu):
    """Row i of a prefill is the decode attention at position start + i: both kernels agree
    within twice the tolerance (each is within it of the same oracle value)."""
    import torch

    w = make_prefill(22, [70], [9])
    d = upload(w)
    out = run(gpu, d, torch.float32)
    rows = np.arange(w.tokens)
    bt = d["block_tables"].expand(len(rows), -1).contiguous()
    lens = to_gpu_i32(9 + rows + 1)
    dec = gpu.paged_decode_attention(d["q"], d["k_pool"], d["v_pool"], bt, lens, out_dtype=torch.float32)
    torch.cuda.synchronize()
    a, b = out.cpu().numpy(), dec.cpu().numpy()
    assert np.all(np.abs(a - b) <= 4e-3 + 2e-2 * np.abs(b))


@pytest.mark.parametrize("width", [300, 600])
def test_prefill_behind_prefixes_longer_than_the_staged_table(gpu, width):
    """Prompt chunks behind cached prefixes of 4050 to 4200 tokens (past 256 table entries) match
    the oracle in both table forms: a 300-entry table is copied to LDS whole; with a 600-entry
    table the kernel keeps the first 256 entries in LDS and reads the rest from HBM."""
    import torch

    lens, starts = [48, 30, 5], [4200, 4050, 4090]
    w = make_prefill(27, lens, starts, max_blocks=width)
    print(f"[prefill] long prefixes lens={lens} starts={starts} table width={width}", flush=True)
    d = upload(w)
    out = run(gpu, d, torch.float32)
    torch.cuda.synchronize()
    rk, rv = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new, w.v_new)
    assert np.array_equal(bf16_to_bits(d["k_pool"]), rk) and np.array_equal(bf16_to_bits(d["v_pool"]), rv)
    ref = oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos)
    assert_close(out.cpu().numpy(), ref, "long prefixes")


def test_prefill_ignores_stale_slots_and_unused_pages(gpu):
    import torch

    w = make_prefill(23, [40, 25], [10, 0])
    k_pool, v_pool = w.k_pool.copy(), w.v_pool.copy()
    used = set(int(p) for p in w.block_tables.ravel() if p >= 0)
    for p in range(w.num_pages):
        if p not in used:
            k_pool[p] = NAN
            v_pool[p] = NAN
    for b in range(w.batch):  # NaN in every slot past each sequence's last position
        last = int(w.start_pos[b]) + int(w.cu_seqlens[b + 1] - w.cu_seqlens[b]) - 1
        page = int(w.block_tables[b, last // 16])
        k_pool[page, :, last % 16 + 1:] = NAN
        v_pool[page, :, last % 16 + 1:] = NAN
    w.k_pool, w.v_pool = k_pool, v_pool
    d = upload(w)
    out = run(gpu, d, torch.float32).cpu().numpy()
    rk, rv = oracle.prefill_kv_append(k_pool, v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new, w.v_new)
    ref = oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos)
    assert_close(out, ref, "stale NaN")


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_prefill_values_past_fp16_range(gpu, out_dtype):
    """The kernel stages V as FP16; a tile whose keys hold a V magnitude past FP16's largest
    finite value runs again with BF16 V and hi + lo BF16 weights.  Planted values: 7e4 and -3e5
    in prompt rows of sequence 0 (appended by the call), -1e30 in a cached prefix slot of
    sequence 2, and 65280 (the largest BF16 value FP16 holds exactly, so the FP16 path) in
    sequence 1.  Every output row must match the oracle."""
    import torch

    w = make_prefill(27, [70, 40, 100], [9, 0, 30])
    v_new, v_pool = w.v_new.copy(), w.v_pool.copy()
    r0 = [int(x) for x in w.cu_seqlens]
    v_new[r0[0] + 5, 0, :4] = f32_to_bf16_bits(np.array([7e4, -3e5, 1.0, 7e4], dtype=np.float32))
    v_new[r0[0] + 60, 1, 10] = f32_to_bf16_bits(np.array([-3e5], dtype=np.float32))[0]
    v_new[r0[1] + 20, 3, 7] = f32_to_bf16_bits(np.array([65280.0], dtype=np.float32))[0]
    pos = 17  # a cached prefix position of sequence 2 (its prompt starts at 30)
    v_pool[int(w.block_tables[2, pos // 16]), 1, pos % 16, 33] = f32_to_bf16_bits(np.array([-1e30], dtype=np.float32))[0]
    w.v_new, w.v_pool = v_new, v_pool
    print(f"[prefill] V past FP16 range, out={out_dtype}", flush=True)
    d = upload(w)
    out = run(gpu, d, torch.float32 if out_dtype == "f32" else torch.bfloat16).float().cpu().numpy()
    rk, rv = oracle.prefill_kv_append(w.k_pool, v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new, v_new)
    ref = oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos)
    if out_dtype == "bf16":  # the tolerance plus the BF16 store's rounding (2^-8 relative)
        assert np.all(np.abs(out - ref) <= 2e-3 + (1e-2 + 2.0 ** -8) * np.abs(ref)), "BF16 output"
    else:
        assert_close(out, ref, "V past FP16 range")
    assert np.abs(ref).max() > 1e20  # the planted prefix value reaches the outputs


def test_prefill_small_weights_behind_a_dominant_first_key(gpu):
    """Rows whose first key dominates by 25.2 in log2 units (q = 16 e_0; that key's K = 8.75 e_0,
    every other K = 0), with V = 0 there and V = 1000 on the other 4095 keys. The anchor is set
    on the first step, so every later weight is 2^-25.2 of it: under FP16's smallest subnormal.
    FP16 weights without the kernel's fixed 2^7 factor would drop them all (output 0 instead of
    about 0.1); with it they are 2^-18.2, subnormal but kept. Every row must match the oracle."""
    import torch

    w = make_prefill(41, [16], [4080], max_blocks=256)
    k_pool = np.zeros_like(w.k_pool)
    v_pool = np.full_like(w.v_pool, f32_to_bf16_bits(np.array([1000.0], dtype=np.float32))[0])
    first = int(w.block_tables[0, 0])
    k_pool[first, :, 0, 0] = f32_to_bf16_bits(np.array([8.75], dtype=np.float32))[0]
    v_pool[first, :, 0, :] = 0
    q = np.zeros_like(w.q)
    q[:, :, 0] = f32_to_bf16_bits(np.array([16.0], dtype=np.float32))[0]
    w.k_pool, w.v_pool, w.q = k_pool, v_pool, q
    w.k_new = np.zeros_like(w.k_new)
    w.v_new = np.full_like(w.v_new, f32_to_bf16_bits(np.array([1000.0], dtype=np.float32))[0])
    print("[prefill] small weights behind a dominant first key, 16 rows behind 4080 cached", flush=True)
    d = upload(w)
    out = run(gpu, d, torch.float32).cpu().numpy()
    rk, rv = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new,
                                      w.v_new)
    ref = oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos)
    assert ref.min() > 0.09  # what the small weights carry
    assert_close(out, ref, "small weights behind a dominant key")


@pytest.mark.parametrize("shape", ["16 rows, 64-key steps", "32 rows, 64-key steps", "32 rows, 32-key steps"])
def test_prefill_late_key_far_above_the_anchor(gpu, shape):
    """A key that arrives after a tile's anchor is set and outscores it by far more than FP16's
    range allows (every query 16 e_0; the planted key 8.75 e_0 scores 25.2 in log2 units, the
    others 2.9 k_0 with k_0 ~ N(0, 1)): its FP16 weight, 2^7 times 2^(25.2 - anchor), overflows, and
    the kernel must see that and move the anchor. Prompt b, KV head g plants its key at token
    64 + (8 b + g) % 64, so over the first 8 prompts the keys sit at every token slot of a 64-key
    step and of two 32-key steps; further prompts (as many as the launch shape needs on this
    device) repeat the pattern. Every row of every prompt must match the oracle."""
    import torch

    cus = gpu.cu_count()
    groups_per_prompt = 5 * 8  # 160-row prompts: 5 groups of 32 rows per KV head
    prompts = {"16 rows, 64-key steps": 8, "32 rows, 64-key steps": -(-2 * cus // groups_per_prompt),
               "32 rows, 32-key steps": -(-4 * cus // groups_per_prompt)}[shape]
    prompts = max(prompts, 8)
    if launch_shape(cus, prompts, 160) != shape:
        pytest.skip(f"{shape} is not reachable with 160-row prompts on {cus} compute units")
    w = make_prefill(70 + prompts, [160] * prompts, [0] * prompts)
    sixteen = f32_to_bf16_bits(np.array([16.0], dtype=np.float32))[0]
    planted = f32_to_bf16_bits(np.array([8.75], dtype=np.float32))[0]
    q = np.zeros_like(w.q)
    q[:, :, 0] = sixteen
    k_new = w.k_new.copy()
    k_new[:, :, 1:] = 0
    r0 = [int(x) for x in w.cu_seqlens]
    for b in range(prompts):
        for g in range(8):
            t = 64 + (8 * b + g) % 64
            k_new[r0[b] + t, g, 0] = planted
    w.q, w.k_new = q, k_new
    print(f"[prefill] late key far above the anchor, {prompts} prompts x 160, launch={shape}", flush=True)
    d = upload(w)
    out = run(gpu, d, torch.float32).cpu().numpy()
    rk, rv = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new,
                                      w.v_new)
    ref = oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos)
    assert_close(out, ref, f"late dominant key, {shape}")


@pytest.mark.parametrize("shape", ["32 rows, 32-key steps", "32 rows, 64-key steps"])
def test_prefill_values_past_fp16_range_every_launch_shape(gpu, shape):
    """The same second pass in the two 32-row launch shapes (the 16-row one is covered above):
    256-token prompts, as many as the shape needs on this device (8 groups of 32 rows per prompt
    and KV head, so 4 * CUs / 64 prompts for 32-key steps and 2 * CUs / 64 for 64-key steps: 16 and
    8 on a 256-CU part).  Half of the prompts carry a V value past FP16's range; every row of every
    prompt must match the oracle."""
    import torch

    cus = gpu.cu_count()
    per = 4 if shape.startswith("32 rows, 32") else 2
    prompts = -(-per * cus // 64)
    assert launch_shape(cus, prompts, 256) == shape
    w = make_prefill(28 + prompts, [256] * prompts, [0] * prompts)
    v_new = w.v_new.copy()
    r0 = [int(x) for x in w.cu_seqlens]
    rng = np.random.default_rng(prompts)
    for b in range(0, prompts, 2):
        row, g, dim = int(rng.integers(0, 256)), int(rng.integers(0, 8)), int(rng.integers(0, 64))
        v_new[r0[b] + row, g, dim] = f32_to_bf16_bits(np.array([-2.5e6 if b % 4 else 9e4], dtype=np.float32))[0]
    w.v_new = v_new
    print(f"[prefill] V past FP16 range, {prompts} prompts x 256, launch={shape}", flush=True)
    d = upload(w)
    out = run(gpu, d, torch.float32).cpu().numpy()
    rk, rv = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new, v_new)
    ref = oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos)
    assert_close(out, ref, f"V past FP16 range, {shape}")
    assert np.abs(ref).max() > 1e3  # the planted values reach the outputs


@pytest.mark.parametrize("bad", ["entry", "start", "past_table"])
def test_prefill_invalid_sequence_gets_zeros(gpu, bad):
    import torch

    w = make_prefill(24, [20, 30, 18], [0, 4, 0], max_blocks=8)
    bt, sp = w.block_tables.copy(), w.start_pos.copy()
    if bad == "entry":
        bt[1, 1] = w.num_pages  # needed by rows of sequence 1
    elif bad == "start":
        sp[1] = -1
    else:
        sp[1] = 8 * 16 - 29  # start + length runs one past the 8-entry table
    d = upload(w)
    d["block_tables"], d["start_pos"] = to_gpu_i32(bt), to_gpu_i32(sp)
    out = gpu.paged_prefill_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["cu_seqlens"],
                                      d["start_pos"], out_dtype=torch.float32).cpu().numpy()
    lo, hi = int(w.cu_seqlens[1]), int(w.cu_seqlens[2])
    assert np.all(out[lo:hi] == 0.0)
    keep = np.r_[0:lo, hi:w.tokens]
    ref = oracle.paged_prefill_attention(w.q, w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos,
                                         rows=keep.tolist())
    assert_close(out[keep], ref[keep], bad)


def test_prefill_append_skips_rows_outside_the_table(gpu):
    import torch

    w = make_prefill(25, [20, 10], [0, 0], max_blocks=4)
    bt = w.block_tables.copy()
    bt[0, 1] = -1  # rows 16..19 of sequence 0 have no page
    d = upload(w)
    d["block_tables"] = to_gpu_i32(bt)
    gpu.prefill_kv_append(d["k_pool"], d["v_pool"], d["block_tables"], d["cu_seqlens"], d["start_pos"], d["k_new"],
                          d["v_new"])
    torch.cuda.synchronize()
    # the oracle on the rows that do have a page
    cu = np.array([0, 16, 26], dtype=np.int32)
    keep = np.r_[0:16, 20:30]
    rk, rv = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, cu, w.start_pos, w.k_new[keep],
                                      w.v_new[keep])
    assert np.array_equal(bf16_to_bits(d["k_pool"]), rk) and np.array_equal(bf16_to_bits(d["v_pool"]), rv)


def test_prefill_sequences_outside_the_bounds_are_untouched(gpu):
    import torch

    w = make_prefill(26, [20, 40, 8], [0, 0, 0])
    d = upload(w)
    sentinel = torch.full((w.tokens, 32, 64), 7.0, dtype=torch.float32, device=d["q"].device)
    gpu.prefill_kv_append(d["k_pool"], d["v_pool"], d["block_tables"], d["cu_seqlens"], d["start_pos"], d["k_new"],
                          d["v_new"], max_prompt_len=32)  # sequence 1 (40 rows) exceeds the bound
    gpu.paged_prefill_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["cu_seqlens"], d["start_pos"],
                                sentinel, max_prompt_len=32)
    torch.cuda.synchronize()
    out = sentinel.cpu().numpy()
    assert np.all(out[20:60] == 7.0)
    rk, rv = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables[[0, 2]], np.array([0, 20, 28]),
                                      w.start_pos[[0, 2]], w.k_new[np.r_[0:20, 60:68]], w.v_new[np.r_[0:20, 60:68]])
    assert np.array_equal(bf16_to_bits(d["k_pool"]), rk)
    keep = np.r_[0:20, 60:68]
    ref = oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos, rows=keep.tolist())
    assert_close(out[keep], ref[keep], "bounded")


def test_prefill_empty_inputs_are_no_ops(gpu):
    import torch

    w = make_prefill(27, [0, 5, 0], [0, 0, 3])
    d = upload(w)
    out = run(gpu, d, torch.float32)
    torch.cuda.synchronize()
    rk, rv = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new, w.v_new)
    ref = oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos)
    assert_close(out.cpu().numpy(), ref, "empty rows")
    e = make_prefill(28, [0], [0])
    de = upload(e)
    out = run(gpu, de, torch.float32)
    assert out.shape[0] == 0


def test_prefill_debug_validation(gpu, monkeypatch):
    import torch

    w = make_prefill(29, [20, 20], [0, 0])
    bt = w.block_tables.copy()
    bt[1, 0] = bt[0, 0]  # both sequences write page bt[0, 0]
    d = upload(w)
    d["block_tables"] = to_gpu_i32(bt)
    monkeypatch.setenv("PKV_DEBUG_VALIDATE", "1")
    with pytest.raises(gpu.PagedKVError, match="VALIDATION"):
        gpu.prefill_kv_append(d["k_pool"], d["v_pool"], d["block_tables"], d["cu_seqlens"], d["start_pos"],
                              d["k_new"], d["v_new"])
    d["block_tables"] = to_gpu_i32(w.block_tables)
    out = run(gpu, d, torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("where", ["k_new", "v_new", "pool_k", "pool_v"])
def test_prefill_debug_validation_rejects_non_finite_prompt_rows(gpu, monkeypatch, where):
    """The prompt's own K/V rows must be finite (a masked later key enters the PV product with
    weight 0).  Under PKV_DEBUG_VALIDATE the append rejects an infinity or NaN in k_new / v_new,
    and the attention one in the prompt rows' pool slots, before launching; a NaN in the cached
    prefix (positions before the chunk's start) is not a precondition violation."""
    import torch

    w = make_prefill(31, [20, 35], [0, 10])
    d = upload(w)
    r1 = int(w.cu_seqlens[1])
    inf, nan = np.uint16(0x7F80), np.uint16(0xFFC0)
    monkeypatch.setenv("PKV_DEBUG_VALIDATE", "1")
    if where in ("k_new", "v_new"):
        rows = (w.k_new if where == "k_new" else w.v_new).copy()
        rows[r1 + 7, 3, 40] = inf
        d[where] = to_gpu_bf16(rows)
        before = bf16_to_bits(d["k_pool"]), bf16_to_bits(d["v_pool"])
        with pytest.raises(gpu.PagedKVError, match="VALIDATION"):
            gpu.prefill_kv_append(d["k_pool"], d["v_pool"], d["block_tables"], d["cu_seqlens"], d["start_pos"],
                                  d["k_new"], d["v_new"])
        torch.cuda.synchronize()
        assert np.array_equal(bf16_to_bits(d["k_pool"]), before[0])  # nothing was launched
        assert np.array_equal(bf16_to_bits(d["v_pool"]), before[1])
        return
    gpu.prefill_kv_append(d["k_pool"], d["v_pool"], d["block_tables"], d["cu_seqlens"], d["start_pos"], d["k_new"],
                          d["v_new"])
    torch.cuda.synchronize()
    pool = bf16_to_bits(d["k_pool" if where == "pool_k" else "v_pool"]).copy()
    clean = pool.copy()
    pos = 10 + 30  # prompt row 30 of sequence 1
    pool[int(w.block_tables[1, pos // 16]), 5, pos % 16, 0] = nan
    d["k_pool" if where == "pool_k" else "v_pool"] = to_gpu_bf16(pool)
    with pytest.raises(gpu.PagedKVError, match="VALIDATION"):
        gpu.paged_prefill_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["cu_seqlens"],
                                    d["start_pos"], out_dtype=torch.float32)
    # the same NaN in sequence 1's cached prefix (position 4 < start 10) is accepted
    pool = clean.copy()
    pool[int(w.block_tables[1, 0]), 5, 4, 0] = nan
    d["k_pool" if where == "pool_k" else "v_pool"] = to_gpu_bf16(pool)
    out = gpu.paged_prefill_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["cu_seqlens"],
                                      d["start_pos"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(out[:r1]).all()  # sequence 0 does not see it
