"""Property tests of the oracle on random small decode steps (hypothesis, derandomized)."""

import math

import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from workloads import make_custom

SETTINGS = settings(max_examples=30, deadline=None, derandomize=True)


@SETTINGS
@given(lengths=st.lists(st.integers(1, 70), min_size=1, max_size=4), hkv=st.integers(1, 3), seed=st.integers(0, 2**16))
def test_oracle_matches_brute_force_and_page_renaming(lengths, hkv, seed):
    w = make_custom(seed=seed, lengths=lengths, num_kv_heads=hkv)
    out = oracle.paged_decode_attention(w.q[0], w.k_pool, w.v_pool, w.block_tables[0], w.context_lens)
    rng = np.random.default_rng(seed)
    perm = rng.permutation(w.num_pages)
    k2 = np.empty_like(w.k_pool)
    v2 = np.empty_like(w.v_pool)
    k2[perm] = w.k_pool
    v2[perm] = w.v_pool
    bt2 = np.where(w.block_tables[0] >= 0, perm[np.maximum(w.block_tables[0], 0)], -1)
    assert np.array_equal(out, oracle.paged_decode_attention(w.q[0], k2, v2, bt2, w.context_lens))
    # brute force on one random head of one random sequence
    b = int(rng.integers(len(lengths)))
    h = int(rng.integers(4 * hkv))
    L = int(w.context_lens[b])
    g = h // 4
    q = oracle.bf16_bits_to_f64(w.q[0, b, h])
    kk = [oracle.bf16_bits_to_f64(w.k_pool[w.block_tables[0, b, t // 16], g, t % 16]) for t in range(L)]
    vv = [oracle.bf16_bits_to_f64(w.v_pool[w.block_tables[0, b, t // 16], g, t % 16]) for t in range(L)]
    s = [math.fsum(q * k) / 8.0 for k in kk]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    den = math.fsum(e)
    ref = np.array([math.fsum(e[t] * vv[t][d] for t in range(L)) / den for d in range(64)])
    assert np.max(np.abs(out[b, h] - ref)) <= 1e-12


@SETTINGS
@given(length=st.integers(2, 300), cuts=st.lists(st.integers(1, 299), max_size=6), seed=st.integers(0, 2**16))
def test_online_merge_any_cut_points(length, cuts, seed):
    w = make_custom(seed=seed, lengths=[length], num_kv_heads=1)
    keys = oracle.bf16_bits_to_f64(oracle.gather_context(w.k_pool, w.block_tables[0, 0], length))
    vals = oracle.bf16_bits_to_f64(oracle.gather_context(w.v_pool, w.block_tables[0, 0], length))
    q = oracle.bf16_bits_to_f64(w.q[0, 0])
    two = oracle.attend_one(q, keys, vals, 0.125)
    online = oracle.attend_one_online(q, keys, vals, 0.125, sorted(set(c for c in cuts if c < length)))
    assert np.max(np.abs(two - online)) <= 1e-12
