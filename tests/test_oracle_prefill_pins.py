"""Pins for the paged prefill oracle: each check would fail for a plausible mistake (a mask off by
one, a wrong KV head, a missing scale, rows written at the wrong position)."""

import math

import numpy as np
import pytest

import oracle
from workloads import make_prefill, make_prefill_config


def _appended(w):
    return oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new, w.v_new)


def _contiguous(pool, table, L):
    return oracle.bf16_bits_to_f64(oracle.gather_context(pool, table, L))


def test_append_writes_each_row_at_its_position():
    w = make_prefill(1, [5, 20, 0, 33], [0, 7, 3, 16])
    kp = np.full_like(w.k_pool, 0x7FC0)  # NaN everywhere before the append
    vp = np.full_like(w.v_pool, 0x7FC0)
    k2, v2 = oracle.prefill_kv_append(kp, vp, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new, w.v_new)
    written = 0
    for b in range(w.batch):
        for i in range(int(w.cu_seqlens[b + 1] - w.cu_seqlens[b])):
            pos = int(w.start_pos[b]) + i
            page, slot = int(w.block_tables[b, pos // 16]), pos % 16
            row = int(w.cu_seqlens[b]) + i
            assert np.array_equal(k2[page, :, slot], w.k_new[row]) and np.array_equal(v2[page, :, slot], w.v_new[row])
            written += 1
    # nothing else changed: exactly `written` (page, slot) rows left NaN-free
    assert int((k2 != 0x7FC0).any(axis=(1, 3)).sum()) == written == w.tokens
    assert int((v2 != 0x7FC0).any(axis=(1, 3)).sum()) == written


def test_append_equals_per_token_decode_appends():
    w = make_prefill(2, [17, 40], [5, 0])
    k2, v2 = _appended(w)
    kd, vd = w.k_pool, w.v_pool
    for b in range(w.batch):
        for i in range(int(w.cu_seqlens[b + 1] - w.cu_seqlens[b])):
            row = int(w.cu_seqlens[b]) + i
            kd, vd = oracle.kv_append(kd, vd, w.block_tables[b:b + 1], [int(w.start_pos[b]) + i], w.k_new[row:row + 1],
                                      w.v_new[row:row + 1])
    assert np.array_equal(k2, kd) and np.array_equal(v2, vd)


@pytest.mark.parametrize("name", ["prefill_tiny", "prefill_chunked"])
def test_rows_equal_decode_attention_at_their_position(name):
    """Prefill row i is the decode step of its sequence at position start + i (the decode oracle
    is pinned separately)."""
    w = make_prefill_config(name)
    k2, v2 = _appended(w)
    rng = np.random.default_rng(0)
    rows = sorted(set(rng.integers(0, w.tokens, size=12).tolist()) | {0, w.tokens - 1})
    out = oracle.paged_prefill_attention(w.q, k2, v2, w.block_tables, w.cu_seqlens, w.start_pos, rows=rows)
    seq_of = np.searchsorted(w.cu_seqlens, np.arange(w.tokens), side="right") - 1
    for r in rows:
        b = int(seq_of[r])
        L = int(w.start_pos[b]) + r - int(w.cu_seqlens[b]) + 1
        ref = oracle.paged_decode_attention(w.q[r:r + 1], k2, v2, w.block_tables[b:b + 1], [L])
        assert np.max(np.abs(out[r] - ref[0])) <= 1e-13


def test_torch_sdpa_causal_float64():
    torch = pytest.importorskip("torch")
    w = make_prefill(3, [70], [0])
    k2, v2 = _appended(w)
    out = oracle.paged_prefill_attention(w.q, k2, v2, w.block_tables, w.cu_seqlens, w.start_pos)
    K = torch.from_numpy(_contiguous(k2, w.block_tables[0], 70)).permute(1, 0, 2)  # [Hkv][L][D]
    V = torch.from_numpy(_contiguous(v2, w.block_tables[0], 70)).permute(1, 0, 2)
    Q = torch.from_numpy(oracle.bf16_bits_to_f64(w.q)).permute(1, 0, 2)  # [Hq][L][D]
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q, K.repeat_interleave(4, dim=0), V.repeat_interleave(4, dim=0), is_causal=True, scale=0.125)
    assert np.max(np.abs(out - ref.permute(1, 0, 2).numpy())) <= 1e-12


def test_torch_sdpa_with_cached_prefix():
    torch = pytest.importorskip("torch")
    start, n = 45, 30
    w = make_prefill(4, [n], [start])
    k2, v2 = _appended(w)
    out = oracle.paged_prefill_attention(w.q, k2, v2, w.block_tables, w.cu_seqlens, w.start_pos)
    L = start + n
    K = torch.from_numpy(_contiguous(k2, w.block_tables[0], L)).permute(1, 0, 2)
    V = torch.from_numpy(_contiguous(v2, w.block_tables[0], L)).permute(1, 0, 2)
    Q = torch.from_numpy(oracle.bf16_bits_to_f64(w.q)).permute(1, 0, 2)
    mask = torch.arange(L)[None, :] <= (start + torch.arange(n))[:, None]  # True = visible
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q, K.repeat_interleave(4, dim=0), V.repeat_interleave(4, dim=0), attn_mask=mask, scale=0.125)
    assert np.max(np.abs(out - ref.permute(1, 0, 2).numpy())) <= 1e-12


def test_brute_force_rows():
    """Scalar loops with math.fsum over contiguous rows taken straight from the prompt inputs
    and the pool's cached prefix."""
    start, n = 19, 24
    w = make_prefill(5, [n], [start])
    k2, v2 = _appended(w)
    out = oracle.paged_prefill_attention(w.q, k2, v2, w.block_tables, w.cu_seqlens, w.start_pos)

    def row_of(pool, new, pos):
        if pos >= start:
            return oracle.bf16_bits_to_f64(new[pos - start])
        page = int(w.block_tables[0, pos // 16])
        return oracle.bf16_bits_to_f64(pool[page, :, pos % 16])

    for i in (0, 5, n - 1):
        for h in (0, 7, 31):
            g = h // 4
            q = oracle.bf16_bits_to_f64(w.q[i, h])
            keys = [row_of(w.k_pool, w.k_new, t)[g] for t in range(start + i + 1)]
            vals = [row_of(w.v_pool, w.v_new, t)[g] for t in range(start + i + 1)]
            s = [math.fsum(q * k) / 8.0 for k in keys]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            den = math.fsum(e)
            ref = np.array([math.fsum(e[t] * vals[t][d] for t in range(len(e))) / den for d in range(64)])
            assert np.max(np.abs(out[i, h] - ref)) <= 1e-12


def test_first_row_of_a_fresh_prompt_is_its_own_value_row():
    w = make_prefill(6, [9, 4], [0, 0])
    k2, v2 = _appended(w)
    out = oracle.paged_prefill_attention(w.q, k2, v2, w.block_tables, w.cu_seqlens, w.start_pos)
    for b in range(2):
        r = int(w.cu_seqlens[b])
        expect = np.repeat(oracle.bf16_bits_to_f64(w.v_new[r]), 4, axis=0)  # head h -> KV head h // 4
        assert np.array_equal(out[r], expect)


def test_future_rows_and_stale_slots_do_not_matter():
    w = make_prefill(7, [40], [10])
    k2, v2 = _appended(w)
    base = oracle.paged_prefill_attention(w.q, k2, v2, w.block_tables, w.cu_seqlens, w.start_pos)
    # NaN into every slot after the last prompt position, and into unassigned pages
    k3, v3 = k2.copy(), v2.copy()
    last = 10 + 40 - 1
    page = int(w.block_tables[0, last // 16])
    k3[page, :, last % 16 + 1:] = 0x7FC0
    v3[page, :, last % 16 + 1:] = 0x7FC0
    used = set(int(p) for p in w.block_tables[0] if p >= 0)
    for p in range(w.num_pages):
        if p not in used:
            k3[p] = 0x7FC0
            v3[p] = 0x7FC0
    assert np.array_equal(base, oracle.paged_prefill_attention(w.q, k3, v3, w.block_tables, w.cu_seqlens, w.start_pos))
    # changing the K/V of prompt row j changes rows >= j only
    j = 17
    k_new = w.k_new.copy()
    k_new[j] ^= 0x0100
    k4, v4 = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, k_new, w.v_new)
    out = oracle.paged_prefill_attention(w.q, k4, v4, w.block_tables, w.cu_seqlens, w.start_pos)
    assert np.array_equal(out[:j], base[:j])
    assert np.all(np.any(out[j:] != base[j:], axis=(1, 2)))


def test_gqa_mapping_with_constant_values_per_kv_head():
    w = make_prefill(8, [20], [0])
    v_new = np.zeros_like(w.v_new)
    for g in range(8):
        v_new[:, g, :] = np.uint16(0x3F80 + 16 * g)  # 1.0, then distinct values per KV head
    k2, v2 = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new, v_new)
    out = oracle.paged_prefill_attention(w.q, k2, v2, w.block_tables, w.cu_seqlens, w.start_pos)
    for h in range(32):
        expect = oracle.bf16_bits_to_f64(np.uint16(0x3F80 + 16 * (h // 4)))
        assert np.allclose(out[:, h, :], expect, rtol=0, atol=1e-15)


def test_out_of_range_prompts_follow_the_error_rule():
    """A negative start writes nothing; a row whose position has no page of the pool is not
    written while the prompt's other rows are; a prompt that cannot be read through its table
    gets all-zero rows; a valid prompt in the same batch is unaffected."""
    w = make_prefill(3, [5, 6, 4, 3], [0, 0, 0, 0], max_blocks=2)
    w.start_pos[:] = [0, -2, 14, 30]  # prompt 2 crosses into block 1, prompt 3 runs past the span
    P = w.k_pool.shape[0]
    spare = sorted(set(range(P)) - set(int(x) for x in w.block_tables.ravel() if x >= 0))
    w.block_tables[2, 1] = -1  # prompt 2's second page is missing
    w.block_tables[3, 1] = spare[0]  # prompt 3's positions 30, 31 have a page; 32 is past the span
    kp = np.full_like(w.k_pool, 0x7FC0)
    vp = np.full_like(w.v_pool, 0x7FC0)
    k2, v2 = oracle.prefill_kv_append(kp, vp, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new, w.v_new)
    expect_k, expect_v = kp.copy(), vp.copy()
    def put(b, i):
        pos = int(w.start_pos[b]) + i
        page, slot = int(w.block_tables[b, pos // 16]), pos % 16
        row = int(w.cu_seqlens[b]) + i
        expect_k[page, :, slot] = w.k_new[row]
        expect_v[page, :, slot] = w.v_new[row]
    for i in range(5):
        put(0, i)  # valid prompt: every row
    put(2, 0), put(2, 1)  # positions 14, 15 have a page; 16, 17 do not
    put(3, 0), put(3, 1)  # positions 30, 31 are inside the span; 32 is not
    assert np.array_equal(k2, expect_k) and np.array_equal(v2, expect_v)
    out = oracle.paged_prefill_attention(w.q, k2, v2, w.block_tables, w.cu_seqlens, w.start_pos)
    lo = int(w.cu_seqlens[1])
    assert np.array_equal(out[lo:], np.zeros_like(out[lo:]))
    first = oracle.paged_prefill_attention(w.q, k2, v2, w.block_tables[:1], w.cu_seqlens[:2], w.start_pos[:1])
    assert np.array_equal(out[:lo], first[:lo]) and np.all(np.isfinite(out[:lo])) and np.any(out[:lo] != 0)


@pytest.mark.parametrize("mistake", ["mask_off_by_one", "wrong_kv_head", "no_scale", "append_shift", "append_unchecked",
                                     "attention_unchecked"])
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    """Each plausible mistake, planted in the oracle, fails one of the pins above."""
    import oracle.prefill_oracle as po

    if mistake == "mask_off_by_one":
        real = po.causal_attention_rows
        # every row also sees the next (future) position
        monkeypatch.setattr(po, "causal_attention_rows", lambda q, k, v, s, scale: real(q, k, v, s + 1, scale))
        with pytest.raises(AssertionError):
            test_torch_sdpa_causal_float64()
    elif mistake == "wrong_kv_head":
        monkeypatch.setattr(po, "kv_head_of", lambda h, group: h % 8)
        with pytest.raises(AssertionError):
            test_gqa_mapping_with_constant_values_per_kv_head()
    elif mistake == "no_scale":
        real = po.causal_attention_rows
        monkeypatch.setattr(po, "causal_attention_rows", lambda q, k, v, s, scale: real(q, k, v, s, 1.0))
        with pytest.raises(AssertionError):
            test_brute_force_rows()
    elif mistake == "append_unchecked":
        monkeypatch.setattr(po, "slot_in_pool", lambda row, pos, n: True)
        with pytest.raises((AssertionError, IndexError, ValueError)):
            test_out_of_range_prompts_follow_the_error_rule()
    elif mistake == "attention_unchecked":
        monkeypatch.setattr(po, "context_in_pool", lambda row, length, n: True)
        with pytest.raises((AssertionError, IndexError, ValueError)):
            test_out_of_range_prompts_follow_the_error_rule()
    elif mistake == "append_shift":
        real = po.locate_slot
        monkeypatch.setattr(po, "locate_slot", lambda row, pos: real(row, pos + 1))
        with pytest.raises(AssertionError):
            test_append_writes_each_row_at_its_position()
