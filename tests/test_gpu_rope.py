"""GPU parity of rope_kv_append: bit-exact rotated q, K pool and V pool against the RoPE oracle."""

import os

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close, bf16_to_bits, to_gpu_bf16, to_gpu_i32
from workloads import f32_to_bf16_bits, llama3_rope_tables, make_config, make_custom

pytestmark = pytest.mark.gpu


def tables_gpu(rows):
    import torch

    cos, sin = llama3_rope_tables(rows)
    return cos, sin, torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()


def run(gpu, w, cos_d, sin_d, in_place=False, layer=0):
    import torch

    kp, vp = to_gpu_bf16(w.k_pool), to_gpu_bf16(w.v_pool)
    q = to_gpu_bf16(w.q[layer])
    q_out = q if in_place else torch.empty_like(q)
    gpu.rope_kv_append(kp, vp, to_gpu_i32(w.block_tables[layer]), to_gpu_i32(w.positions), q, to_gpu_bf16(w.k_new[layer]),
                       to_gpu_bf16(w.v_new[layer]), cos_d, sin_d, q_out=q_out)
    torch.cuda.synchronize()
    return bf16_to_bits(q_out), bf16_to_bits(kp), bf16_to_bits(vp), kp, vp, q_out


@pytest.mark.parametrize("name", ["tiny", "mixed", "bw256"])
def test_rope_append_bit_exact(gpu, name):
    w = make_config(name)
    cos, sin, cos_d, sin_d = tables_gpu(2048)
    print(f"[rope] config={name} B={w.batch}", flush=True)
    q2, k2, v2, *_ = run(gpu, w, cos_d, sin_d)
    rq, rk, rv = oracle.rope_kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.q[0], w.k_new[0],
                                       w.v_new[0], cos, sin)
    assert np.array_equal(q2, rq)
    assert np.array_equal(k2, rk)
    assert np.array_equal(v2, rv)


def test_rope_in_place_and_position_zero(gpu):
    w = make_custom(seed=60, lengths=[1, 1, 33, 16, 17])
    cos, sin, cos_d, sin_d = tables_gpu(64)
    q2, k2, v2, *_ = run(gpu, w, cos_d, sin_d, in_place=True)
    rq, rk, rv = oracle.rope_kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.q[0], w.k_new[0],
                                       w.v_new[0], cos, sin)
    assert np.array_equal(q2, rq) and np.array_equal(k2, rk) and np.array_equal(v2, rv)
    # position 0 (lengths 1) rotates by angle 0: the rows come back unchanged
    assert np.array_equal(q2[0], w.q[0, 0]) and np.array_equal(q2[1], w.q[0, 1])


def test_rope_rounding_order_tie_on_gpu(gpu):
    """x_0 = 3, x_32 = 1, c = 1 + 3*2^-23, s = 1.99609375 + 2^-20: with each FP32 operation rounded
    on its own, y_0 is exactly the BF16 tie 1 + 2^-8, which rounds to even (0x3F80)."""
    import torch

    w = make_custom(seed=61, lengths=[2])
    w.q[:] = 0
    w.q[0, 0, :, 0] = f32_to_bf16_bits(np.float32([3.0]))[0]
    w.q[0, 0, :, 32] = f32_to_bf16_bits(np.float32([1.0]))[0]
    cos = np.ones((4, 64), dtype=np.float32)
    sin = np.zeros((4, 64), dtype=np.float32)
    cos[1, :] = np.float32(1.0 + 3 * 2.0**-23)
    sin[1, :] = np.float32(1.99609375 + 2.0**-20)
    q2, *_ = run(gpu, w, torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda())
    assert np.all(q2[0, :, 0] == 0x3F80)
    rq, _, _ = oracle.rope_kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.q[0], w.k_new[0],
                                     w.v_new[0], cos, sin)
    assert np.array_equal(q2, rq)


def test_rope_skips_rows_outside_the_tables(gpu):
    import torch

    w = make_custom(seed=62, lengths=[10, 40, 20])
    cos, sin, cos_d, sin_d = tables_gpu(32)  # position 39 is past the 32-row tables
    kp, vp = to_gpu_bf16(w.k_pool), to_gpu_bf16(w.v_pool)
    q = to_gpu_bf16(w.q[0])
    q_out = torch.full_like(q, 7.0)
    gpu.rope_kv_append(kp, vp, to_gpu_i32(w.block_tables[0]), to_gpu_i32(w.positions), q, to_gpu_bf16(w.k_new[0]),
                       to_gpu_bf16(w.v_new[0]), cos_d, sin_d, q_out=q_out)
    torch.cuda.synchronize()
    got = bf16_to_bits(q_out)
    assert np.all(got[1] == f32_to_bf16_bits(np.float32([7.0]))[0])
    keep = [0, 2]
    rq, rk, rv = oracle.rope_kv_append(w.k_pool, w.v_pool, w.block_tables[0][keep], w.positions[keep], w.q[0][keep],
                                       w.k_new[0][keep], w.v_new[0][keep], cos, sin)
    assert np.array_equal(got[keep], rq)
    assert np.array_equal(bf16_to_bits(kp), rk) and np.array_equal(bf16_to_bits(vp), rv)
    os.environ["PKV_DEBUG_VALIDATE"] = "1"
    try:
        with pytest.raises(gpu.PagedKVError, match="PKV_ERR_VALIDATION"):
            gpu.rope_kv_append(kp, vp, to_gpu_i32(w.block_tables[0]), to_gpu_i32(w.positions), q,
                               to_gpu_bf16(w.k_new[0]), to_gpu_bf16(w.v_new[0]), cos_d, sin_d, q_out=q_out)
    finally:
        del os.environ["PKV_DEBUG_VALIDATE"]


def test_decode_step_with_rope_matches_oracle(gpu):
    """rope_kv_append then paged_decode_attention == the oracle's rotate, append, attend."""
    import torch

    w = make_custom(seed=63, lengths=[5, 130, 700, 2048])
    cos, sin, cos_d, sin_d = tables_gpu(2048)
    q2, k2, v2, kp, vp, q_out = run(gpu, w, cos_d, sin_d)
    out = gpu.paged_decode_attention(q_out, kp, vp, to_gpu_i32(w.block_tables[0]), to_gpu_i32(w.context_lens),
                                     out_dtype=torch.float32)
    rq, rk, rv = oracle.rope_kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.q[0], w.k_new[0],
                                       w.v_new[0], cos, sin)
    ref = oracle.paged_decode_attention(rq, rk, rv, w.block_tables[0], w.context_lens)
    assert_close(out.cpu().numpy(), ref, "rope + attention")
