"""The seeded input generators: reproducible, correctly shaped, and consistent paging."""

import numpy as np
import pytest

from workloads import BLOCK_SIZE, MAX_BLOCKS, f32_to_bf16_bits, make_config, make_custom


def test_bf16_conversion_matches_torch():
    import torch

    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    x = np.concatenate([x, np.float32([0.0, -0.0, 1.0 + 2.0**-8, np.inf, -np.inf])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)
    assert f32_to_bf16_bits(np.float32([np.nan]))[0] == 0x7FC0


@pytest.mark.parametrize("name", ["tiny", "long", "mixed", "model16"])
def test_config_shapes_and_tables(name):
    w = make_config(name)
    assert w.k_pool.shape == (w.num_pages, 8, BLOCK_SIZE, 64) and w.k_pool.dtype == np.uint16
    assert w.v_pool.shape == w.k_pool.shape
    assert w.block_tables.shape == (w.layers, w.batch, MAX_BLOCKS) and w.block_tables.dtype == np.int32
    assert w.q.shape == (w.layers, w.batch, 32, 64)
    assert w.k_new.shape == (w.layers, w.batch, 8, 64)
    assert np.array_equal(w.context_lens, w.positions + 1)
    used = []
    for layer in range(w.layers):
        for b in range(w.batch):
            n = (int(w.context_lens[b]) + 15) // 16
            row = w.block_tables[layer, b]
            assert np.all(row[:n] >= 0) and np.all(row[:n] < w.num_pages)
            assert np.all(row[n:] == -1)
            used.extend(row[:n].tolist())
    assert len(used) == len(set(used)), "a physical page is shared"


def test_config_values():
    tiny = make_config("tiny")
    assert tiny.batch == 1 and int(tiny.context_lens[0]) == 37 and tiny.num_pages == 8
    assert int(tiny.positions[0]) // 16 == 2 and int(tiny.positions[0]) % 16 == 4
    mixed = make_config("mixed")
    assert mixed.batch == 16 and mixed.num_pages == 2048
    assert 1 <= mixed.context_lens.min() and mixed.context_lens.max() <= 2048
    m16 = make_config("model16")
    assert m16.layers == 16 and m16.num_pages == 4096
    # FIFO admission under the 4096-page budget with seed 3 admits 17 of the 64 requests
    assert m16.meta["admitted"] == 17 and m16.meta["pages_budgeted"] == 4016
    assert m16.meta["sum_context"] == 3870
    assert m16.meta["pages_budgeted"] <= 4096


def test_generators_are_reproducible():
    a = make_custom(seed=5, lengths=[3, 40, 17])
    b = make_custom(seed=5, lengths=[3, 40, 17])
    for f in ("k_pool", "v_pool", "block_tables", "q", "k_new", "v_new"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = make_custom(seed=6, lengths=[3, 40, 17])
    assert not np.array_equal(a.k_pool, c.k_pool)


def test_fresh_page_only_when_position_opens_a_page():
    w = make_custom(seed=9, lengths=[1, 16, 17, 33, 32], num_pages=12)
    for b, L in enumerate(w.context_lens):
        pos = int(L) - 1
        assert w.block_tables[0, b, pos // 16] >= 0
        assert np.all(w.block_tables[0, b, (pos // 16) + 1 :] == -1)


def test_empty_sequence_allowed():
    w = make_custom(seed=2, lengths=[0, 5])
    assert int(w.positions[0]) == -1 and np.all(w.block_tables[0, 0] == -1)
