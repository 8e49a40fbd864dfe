"""Pools past the 32-bit range: every kernel addresses pages with 64-bit offsets.

A pool of 270,336 pages is 4.4 GB per K or V pool (2.2e9 BF16 elements, past both 2^31 elements
and 2^32 bytes). A small seeded workload is placed in the pool's top pages, the block tables are
renumbered to match, and the rest of the pool holds NaN. Each call must give exactly what it gives
on the small pool (the arithmetic does not depend on where a page lives), match the oracle, and
leave every page below the placed ones untouched.
"""

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, bf16_to_bits, to_gpu_bf16, to_gpu_i32
from workloads import llama3_rope_tables, make_custom, make_prefill

pytestmark = pytest.mark.gpu

BIG_PAGES = (1 << 18) + (1 << 13)  # 270,336 pages x 16 KiB = 4.43 GB per pool
LENGTHS = [2048, 1000, 513, 37, 16, 1, 0]


class HighPool:
    """K and V pools of BIG_PAGES pages, NaN everywhere except the placed small pool."""

    def __init__(self, small_pages):
        import torch

        self.n = small_pages
        self.lo = BIG_PAGES - small_pages  # first placed page
        assert self.lo * 8 * 16 * 64 > (1 << 31)  # every placed page lies past 2^31 elements
        self.k = torch.full((BIG_PAGES, 8, 16, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
        self.v = torch.full_like(self.k, float("nan"))

    def place(self, k_bits, v_bits):
        self.k[self.lo:] = to_gpu_bf16(k_bits)
        self.v[self.lo:] = to_gpu_bf16(v_bits)

    def table(self, small_table):
        t = np.asarray(small_table, dtype=np.int64)
        return to_gpu_i32(np.where(t >= 0, t + self.lo, -1))

    def placed(self):
        return bf16_to_bits(self.k[self.lo:]), bf16_to_bits(self.v[self.lo:])

    def low_untouched(self):
        import torch

        return bool(torch.isnan(self.k[:self.lo]).all().item()) and bool(torch.isnan(self.v[:self.lo]).all().item())


@pytest.fixture(scope="module")
def decode_case():
    w = make_custom(seed=95, lengths=LENGTHS)
    return w


def test_decode_in_a_pool_past_4_gib(gpu, decode_case):
    import torch

    w = decode_case
    print(f"[large pool] decode B={w.batch} small pages={w.num_pages} big pages={BIG_PAGES}", flush=True)
    pool = HighPool(w.num_pages)
    pool.place(w.k_pool, w.v_pool)
    bt_big, bt_small = pool.table(w.block_tables[0]), to_gpu_i32(w.block_tables[0])
    pos, lens = to_gpu_i32(w.positions), to_gpu_i32(w.context_lens)
    q, kn, vn = to_gpu_bf16(w.q[0]), to_gpu_bf16(w.k_new[0]), to_gpu_bf16(w.v_new[0])
    ks, vs = to_gpu_bf16(w.k_pool), to_gpu_bf16(w.v_pool)

    gpu.kv_append(pool.k, pool.v, bt_big, pos, kn, vn)
    gpu.kv_append(ks, vs, bt_small, pos, kn, vn)
    outs = {}
    for pp in (0, 8, 128):  # planned split, 8-page partitions, one partition
        big = gpu.paged_decode_attention(q, pool.k, pool.v, bt_big, lens, out_dtype=torch.float32, partition_pages=pp)
        small = gpu.paged_decode_attention(q, ks, vs, bt_small, lens, out_dtype=torch.float32, partition_pages=pp)
        outs[pp] = (big.cpu().numpy(), small.cpu().numpy())
    torch.cuda.synchronize()

    rk, rv = oracle.kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.k_new[0], w.v_new[0])
    pk, pv = pool.placed()
    assert np.array_equal(pk, rk) and np.array_equal(pv, rv)
    assert pool.low_untouched()
    ref = oracle.paged_decode_attention(w.q[0], rk, rv, w.block_tables[0], w.context_lens)
    for pp, (big, small) in outs.items():
        assert np.array_equal(big, small), f"partition_pages={pp}: result depends on where the pages live"
        assert_close(big, ref, f"large pool pp={pp}")

    # The fused step on a fresh placement equals the two calls bit for bit.
    pool.place(w.k_pool, w.v_pool)
    fused = gpu.decode_step(q, pool.k, pool.v, bt_big, pos, kn, vn, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(fused.cpu().numpy(), outs[0][0])
    pk, pv = pool.placed()
    assert np.array_equal(pk, rk) and np.array_equal(pv, rv)
    assert pool.low_untouched()

    # RoPE + append on a fresh placement: bit-exact against the RoPE oracle.
    pool.place(w.k_pool, w.v_pool)
    cos, sin = llama3_rope_tables(2048)
    q_rot = q.clone()  # a skipped sequence (length 0) leaves its rows as they were
    gpu.rope_kv_append(pool.k, pool.v, bt_big, pos, q, kn, vn, torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda(),
                       q_out=q_rot)
    torch.cuda.synchronize()
    rq, rk2, rv2 = oracle.rope_kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.q[0], w.k_new[0],
                                         w.v_new[0], cos, sin)
    pk, pv = pool.placed()
    assert np.array_equal(bf16_to_bits(q_rot), rq)
    assert np.array_equal(pk, rk2) and np.array_equal(pv, rv2)
    assert pool.low_untouched()
    del pool
    torch.cuda.empty_cache()


def test_prefill_in_a_pool_past_4_gib(gpu):
    import torch

    lens, starts = [300, 17, 64, 1], [100, 0, 1000, 2047]
    w = make_prefill(96, lens, starts)
    print(f"[large pool] prefill lens={lens} starts={starts} small pages={w.k_pool.shape[0]}", flush=True)
    pool = HighPool(w.k_pool.shape[0])
    pool.place(w.k_pool, w.v_pool)
    bt = pool.table(w.block_tables)
    cu, st = to_gpu_i32(w.cu_seqlens), to_gpu_i32(w.start_pos)
    gpu.prefill_kv_append(pool.k, pool.v, bt, cu, st, to_gpu_bf16(w.k_new), to_gpu_bf16(w.v_new))
    out = gpu.paged_prefill_attention(to_gpu_bf16(w.q), pool.k, pool.v, bt, cu, st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rk, rv = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new, w.v_new)
    pk, pv = pool.placed()
    assert np.array_equal(pk, rk) and np.array_equal(pv, rv)
    assert pool.low_untouched()
    ref = oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos)
    assert_close(out.cpu().numpy(), ref, "large pool prefill")
    del pool
    torch.cuda.empty_cache()
