"""Pins for the RoPE oracle (rotation of pair (i, i + 32) by the table angle of slot 2i)."""

import math

import numpy as np
import pytest

import oracle
from oracle import rope_oracle as RO
from workloads import f32_to_bf16_bits, llama3_rope_tables, make_custom, normal_bf16

bits = lambda x: f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
bit1 = lambda x: f32_to_bf16_bits(np.asarray([x], dtype=np.float32))[0]


def f32(b):
    return oracle.bf16_bits_to_f32(b)


def angle_tables(angles_per_pair, rows=4):
    """Tables whose row r rotates pair i by r * angles_per_pair[i] (slot 2i and 2i+1 equal)."""
    a = np.asarray(angles_per_pair, dtype=np.float64)
    full = np.arange(rows, dtype=np.float64)[:, None] * np.repeat(a, 2)[None, :]
    return np.cos(full).astype(np.float32), np.sin(full).astype(np.float32)


def exact_tables(c, s, rows=2):
    cos = np.full((rows, 64), c, dtype=np.float32)
    sin = np.full((rows, 64), s, dtype=np.float32)
    return cos, sin


def check_position_zero_identity():
    cos, sin = llama3_rope_tables(4)
    x = normal_bf16(np.random.default_rng(200), (8, 64))
    assert np.array_equal(oracle.rope_rotate(x, 0, cos, sin), x)


def check_quarter_and_half_turns():
    x = normal_bf16(np.random.default_rng(201), (8, 64))
    xf = f32(x)
    cos, sin = exact_tables(0.0, 1.0)
    y = f32(oracle.rope_rotate(x, 1, cos, sin))
    assert np.array_equal(y[:, :32], -xf[:, 32:]) and np.array_equal(y[:, 32:], xf[:, :32])
    cos, sin = exact_tables(-1.0, 0.0)
    y = f32(oracle.rope_rotate(x, 1, cos, sin))
    assert np.array_equal(y, -xf)


def check_pairing_and_sign():
    """A unit vector on element i lands on (cos, sin) of pair i at elements i and i + 32."""
    for i in (0, 5, 31):
        angles = np.zeros(32)
        angles[i] = 0.75
        cos, sin = angle_tables(angles)
        x = np.zeros((1, 64), dtype=np.uint16)
        x[0, i] = bit1(1.0)
        y = f32(oracle.rope_rotate(x, 1, cos, sin))[0]
        expect = np.zeros(64, dtype=np.float32)
        expect[i] = f32(bit1(math.cos(0.75)))
        expect[i + 32] = f32(bit1(math.sin(0.75)))
        assert np.array_equal(y, expect), i
        # the partner element rotates the other way round: (0, 1) -> (-sin, cos)
        x = np.zeros((1, 64), dtype=np.uint16)
        x[0, i + 32] = bit1(1.0)
        y = f32(oracle.rope_rotate(x, 1, cos, sin))[0]
        assert y[i] == -f32(bit1(math.sin(0.75))) and y[i + 32] == f32(bit1(math.cos(0.75)))


def check_complex_formulation():
    """Against (x_i + j x_{i+32}) e^{j theta} in complex128, rounded to BF16: equal except where the
    FP32 rounding of the two-product form lands on the other side of a BF16 rounding boundary."""
    rng = np.random.default_rng(202)
    cos, sin = llama3_rope_tables(2048)
    x = normal_bf16(rng, (40, 64))
    for pos in (1, 17, 511, 2047):
        got = oracle.rope_rotate(x, pos, cos, sin)
        xf = f32(x).astype(np.float64)
        z = (xf[:, :32] + 1j * xf[:, 32:]) * (cos[pos, 0::2].astype(np.float64) + 1j * sin[pos, 0::2].astype(np.float64))
        ref = bits(np.concatenate([z.real, z.imag], axis=1).astype(np.float32))
        diff = np.abs(got.astype(np.int32) - ref.astype(np.int32))
        assert diff.max() <= 1 and (diff == 0).mean() >= 0.98, pos


def check_norm_and_inverse():
    rng = np.random.default_rng(203)
    angles = rng.uniform(-3, 3, 32)
    cos, sin = angle_tables(angles, rows=2)
    cosn, sinn = angle_tables(-angles, rows=2)
    x = normal_bf16(rng, (16, 64))
    y = oracle.rope_rotate(x, 1, cos, sin)
    xf, yf = f32(x).astype(np.float64), f32(y).astype(np.float64)
    n0 = xf[:, :32] ** 2 + xf[:, 32:] ** 2
    n1 = yf[:, :32] ** 2 + yf[:, 32:] ** 2
    assert np.allclose(n1, n0, rtol=2e-2, atol=1e-3)
    back = f32(oracle.rope_rotate(y, 1, cosn, sinn))
    assert np.allclose(back, f32(x), rtol=2e-2, atol=2e-2)


def check_relative_position():
    """<R(m) q, R(n) k> depends on m - n only (up to BF16 rounding of the rotated vectors)."""
    rng = np.random.default_rng(204)
    cos, sin = llama3_rope_tables(600)
    q = normal_bf16(rng, (1, 64))
    k = normal_bf16(rng, (1, 64))
    dots = []
    for m, n in ((10, 3), (110, 103), (510, 503)):
        a = f32(oracle.rope_rotate(q, m, cos, sin)).astype(np.float64)
        b = f32(oracle.rope_rotate(k, n, cos, sin)).astype(np.float64)
        dots.append(float((a * b).sum()))
    scale = float(np.abs(f32(q)).sum() * np.abs(f32(k)).max())
    assert max(dots) - min(dots) <= 2e-2 * scale


def check_fp32_rounding_order():
    """Each product and the sum/difference are separately rounded FP32 operations (torch CPU
    elementwise ops in float32 follow that order), then BF16 round-to-nearest-even."""
    import torch

    rng = np.random.default_rng(205)
    cos, sin = llama3_rope_tables(1024)
    x = normal_bf16(rng, (64, 64))
    for pos in (3, 999):
        got = oracle.rope_rotate(x, pos, cos, sin)
        t = torch.from_numpy(f32(x))
        c = torch.from_numpy(cos[pos, 0::2])
        s = torch.from_numpy(sin[pos, 0::2])
        y1 = t[:, :32] * c - t[:, 32:] * s
        y2 = t[:, :32] * s + t[:, 32:] * c
        ref = torch.cat([y1, y2], dim=1).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, ref), pos


def check_rounding_order_tie():
    """Hand-worked: x_0 = 3, x_32 = 1, c = 1 + 3*2^-23, s = 1.99609375 + 2^-20.  fl(3c) rounds the
    tie 3 + 2^-20 + 2^-23 down to 3 + 2^-20, so fl(3c) - 1*s = 1 + 2^-8 exactly, a BF16 tie that
    rounds to even: 1.0 (0x3F80).  A fused multiply-add would keep the 2^-23 and give 1 + 2^-7."""
    c = np.float32(1.0 + 3 * 2.0**-23)
    s = np.float32(1.99609375 + 2.0**-20)
    assert float(c) == 1.0 + 3 * 2.0**-23 and float(s) == 1.99609375 + 2.0**-20
    cos = np.ones((2, 64), dtype=np.float32)
    sin = np.zeros((2, 64), dtype=np.float32)
    cos[1, 0:2] = c
    sin[1, 0:2] = s
    x = np.zeros((1, 64), dtype=np.uint16)
    x[0, 0] = bit1(3.0)
    x[0, 32] = bit1(1.0)
    y = oracle.rope_rotate(x, 1, cos, sin)
    assert y[0, 0] == 0x3F80


def check_rope_append():
    w = make_custom(seed=206, lengths=[1, 17, 40])
    cos, sin = llama3_rope_tables(64)
    q2, k2, v2 = oracle.rope_kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.q[0], w.k_new[0],
                                       w.v_new[0], cos, sin)
    for b, pos in enumerate(w.positions):
        page = w.block_tables[0, b, pos // 16]
        assert np.array_equal(q2[b], oracle.rope_rotate(w.q[0, b], int(pos), cos, sin))
        assert np.array_equal(k2[page, :, pos % 16], oracle.rope_rotate(w.k_new[0, b], int(pos), cos, sin))
        assert np.array_equal(v2[page, :, pos % 16], w.v_new[0, b])
    changed = np.argwhere(np.any(k2 != w.k_pool, axis=-1))
    assert len(changed) <= w.batch * w.num_kv_heads


def check_out_of_range_skipped():
    """A sequence whose position has no table row, lies outside the block table, or maps to no
    page of the pool is skipped entirely: its q rows come back unchanged and the pool is not
    written; the valid sequence in the same batch is rotated and appended."""
    rng = np.random.default_rng(316)
    P = 4
    k_pool = normal_bf16(rng, (P, 2, 16, 64))
    v_pool = normal_bf16(rng, (P, 2, 16, 64))
    q = normal_bf16(rng, (5, 8, 64))
    k_new = normal_bf16(rng, (5, 2, 64))
    v_new = normal_bf16(rng, (5, 2, 64))
    cos, sin = angle_tables(np.linspace(0.1, 1.0, 32), rows=20)
    tables = np.array([[1, 2], [1, 2], [1, 2], [-1, 2], [P, 2]], dtype=np.int32)
    positions = np.array([3, -1, 20, 5, 6])  # rows 20.. are past the tables (20 rows)
    q2, k2, v2 = oracle.rope_kv_append(k_pool, v_pool, tables, positions, q, k_new, v_new, cos, sin)
    assert np.array_equal(q2[1:], q[1:])
    k_ref, v_ref = k_pool.copy(), v_pool.copy()
    k_ref[1, :, 3] = oracle.rope_rotate(k_new[0], 3, cos, sin)
    v_ref[1, :, 3] = v_new[0]
    assert np.array_equal(k2, k_ref) and np.array_equal(v2, v_ref)
    assert np.array_equal(q2[0], oracle.rope_rotate(q[0], 3, cos, sin)) and not np.array_equal(q2[0], q[0])


PINS = {
    "position_zero_identity": check_position_zero_identity,
    "quarter_and_half_turns": check_quarter_and_half_turns,
    "pairing_and_sign": check_pairing_and_sign,
    "complex_formulation": check_complex_formulation,
    "norm_and_inverse": check_norm_and_inverse,
    "relative_position": check_relative_position,
    "fp32_rounding_order": check_fp32_rounding_order,
    "rounding_order_tie": check_rounding_order_tie,
    "rope_append": check_rope_append,
    "out_of_range_skipped": check_out_of_range_skipped,
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_rope_pin(name):
    PINS[name]()


def _rotate_adjacent_pairs(x_bits, pos, cos_table, sin_table):
    x = RO.bf16_bits_to_f32(x_bits)
    out = np.empty_like(x)
    for i in range(32):
        c, s = np.float32(cos_table[pos, 2 * i]), np.float32(sin_table[pos, 2 * i])
        x1, x2 = x[..., 2 * i], x[..., 2 * i + 1]
        out[..., 2 * i] = np.float32(x1 * c) - np.float32(x2 * s)
        out[..., 2 * i + 1] = np.float32(x1 * s) + np.float32(x2 * c)
    return oracle.bf16_round_nearest_even(out)


def _rotate_fused(x_bits, pos, cos_table, sin_table):
    x = RO.bf16_bits_to_f32(x_bits).astype(np.float64)
    out = np.empty_like(x)
    for i in range(32):
        c, s = float(cos_table[pos, 2 * i]), float(sin_table[pos, 2 * i])
        out[..., i] = (x[..., i] * c - np.float32(x[..., i + 32] * s)).astype(np.float32)  # one rounding fewer
        out[..., i + 32] = (x[..., i] * s + np.float32(x[..., i + 32] * c)).astype(np.float32)
    return oracle.bf16_round_nearest_even(out.astype(np.float32))


def _rotate_wrong_sign(x_bits, pos, cos_table, sin_table):
    x = RO.bf16_bits_to_f32(x_bits)
    out = np.empty_like(x)
    for i in range(32):
        c, s = np.float32(cos_table[pos, 2 * i]), np.float32(sin_table[pos, 2 * i])
        out[..., i] = np.float32(x[..., i] * c) + np.float32(x[..., i + 32] * s)
        out[..., i + 32] = np.float32(x[..., i] * s) + np.float32(x[..., i + 32] * c)
    return oracle.bf16_round_nearest_even(out)


def _rotate_wrong_slot(x_bits, pos, cos_table, sin_table):
    x = RO.bf16_bits_to_f32(x_bits)
    out = np.empty_like(x)
    for i in range(32):
        c, s = np.float32(cos_table[pos, i]), np.float32(sin_table[pos, i])  # slot i instead of 2i
        out[..., i] = np.float32(x[..., i] * c) - np.float32(x[..., i + 32] * s)
        out[..., i + 32] = np.float32(x[..., i] * s) + np.float32(x[..., i + 32] * c)
    return oracle.bf16_round_nearest_even(out)


MUTATIONS = {
    "adjacent_pairs": (_rotate_adjacent_pairs, ["pairing_and_sign", "complex_formulation"]),
    "fused_multiply_add": (_rotate_fused, ["fp32_rounding_order", "rounding_order_tie"]),
    "wrong_sign": (_rotate_wrong_sign, ["pairing_and_sign", "quarter_and_half_turns"]),
    "wrong_table_slot": (_rotate_wrong_slot, ["complex_formulation", "pairing_and_sign"]),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_rope_planted_mistake_is_caught(mutation, monkeypatch):
    bad, pins = MUTATIONS[mutation]
    monkeypatch.setattr(RO, "rope_rotate", bad)
    monkeypatch.setattr(oracle, "rope_rotate", bad)
    caught = []
    for name in pins:
        try:
            PINS[name]()
        except (AssertionError, IndexError):
            caught.append(name)
    assert caught, f"planted mistake {mutation!r} passed every pin in {pins}"
