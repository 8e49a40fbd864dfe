"""Pins for the FP64 oracle: each check ties it to something other than itself.

The pages print no attention output for any input, so the pins are closed forms, invariants,
an independent brute-force implementation on contiguous K/V, and torch's scaled-dot-product
attention.  The second half plants plausible mistakes in the oracle (on the CPU, via
monkeypatch) and asserts that some pin fails for each of them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import paged_oracle as PO
from workloads import f32_to_bf16_bits, make_custom, normal_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NAN_BITS = np.uint16(0x7FC0)


def bits(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def as_f64(b):
    """BF16 bits -> float64 through torch's bfloat16 type (an independent decoder)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def page_contiguous(rng, k_rows, v_rows, extra_pages=3, table_width=8):
    """Scatter contiguous per-sequence rows [L][Hkv][D] into a shuffled page pool.

    Written independently of the oracle: token t of sequence b goes to slot t % 16 of the
    (t // 16)-th page handed to b.  Pages not used by any sequence hold random values.
    """
    hkv, d = k_rows[0].shape[1], k_rows[0].shape[2]
    need = [(r.shape[0] + 15) // 16 for r in k_rows]
    num_pages = sum(need) + extra_pages
    k_pool = normal_bf16(rng, (num_pages, hkv, 16, d))
    v_pool = normal_bf16(rng, (num_pages, hkv, 16, d))
    order = rng.permutation(num_pages)
    tables = np.full((len(k_rows), table_width), -1, dtype=np.int32)
    cursor = 0
    for b, (kr, vr) in enumerate(zip(k_rows, v_rows)):
        for j in range(need[b]):
            tables[b, j] = order[cursor]
            cursor += 1
        for t in range(kr.shape[0]):
            page = tables[b, t // 16]
            k_pool[page, :, t % 16, :] = kr[t]
            v_pool[page, :, t % 16, :] = vr[t]
    return k_pool, v_pool, tables


def brute_force(q_bits, k_rows, v_rows, scale):
    """Naive loops with math.fsum / math.exp on the contiguous rows of one sequence."""
    q = as_f64(q_bits)
    k = as_f64(k_rows)
    v = as_f64(v_rows)
    hq, d = q.shape
    L, hkv, _ = k.shape
    group = hq // hkv
    out = np.zeros((hq, d))
    for h in range(hq):
        g = h // group
        s = [math.fsum(q[h, i] * k[t, g, i] for i in range(d)) * scale for t in range(L)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        den = math.fsum(w)
        for i in range(d):
            out[h, i] = math.fsum(w[t] * v[t, g, i] for t in range(L)) / den
    return out


def one_sequence(rng, L, hkv=2, group=4, d=64):
    q = normal_bf16(rng, (hkv * group, d))
    k = normal_bf16(rng, (L, hkv, d))
    v = normal_bf16(rng, (L, hkv, d))
    return q, k, v


def run_paged(q, k, v, rng, scale=0.125):
    kp, vp, tb = page_contiguous(rng, [k], [v])
    out = oracle.paged_decode_attention(q[None], kp, vp, tb, np.array([k.shape[0]]), scale)
    return out[0]


# ------------------------------------------------------------------------------------------
# Pin checks (each raises AssertionError when the oracle is wrong)
# ------------------------------------------------------------------------------------------

def check_brute_force():
    """O1: paged oracle == brute force on contiguous rows, several sequences and lengths."""
    rng = np.random.default_rng(100)
    lengths = [1, 16, 17, 37]
    seqs = [one_sequence(rng, L) for L in lengths]
    qs = np.stack([s[0] for s in seqs])
    kp, vp, tb = page_contiguous(rng, [s[1] for s in seqs], [s[2] for s in seqs])
    got = oracle.paged_decode_attention(qs, kp, vp, tb, np.array(lengths), 0.125)
    for b, (q, k, v) in enumerate(seqs):
        ref = brute_force(q, k, v, 0.125)
        assert np.max(np.abs(got[b] - ref)) <= 1e-12, f"sequence {b} (L={lengths[b]})"


def check_single_token():
    """O2: a context of one token returns that token's V row exactly."""
    rng = np.random.default_rng(101)
    q, k, v = one_sequence(rng, 1)
    out = run_paged(q, k, v, rng)
    for h in range(q.shape[0]):
        assert np.array_equal(out[h], as_f64(v[0, h // 4])), f"head {h}"


def check_uniform_scores():
    """O3: q = 0 makes every score equal, so the output is the plain mean of the V rows."""
    rng = np.random.default_rng(102)
    L = 29
    _, k, v = one_sequence(rng, L)
    q = np.zeros((8, 64), dtype=np.uint16)
    out = run_paged(q, k, v, rng)
    vv = as_f64(v)
    for h in range(8):
        mean = np.array([math.fsum(vv[:, h // 4, i]) / L for i in range(64)])
        assert np.max(np.abs(out[h] - mean)) <= 1e-14, f"head {h}"


def check_page_permutation():
    """O4: renaming physical pages (and moving their contents) leaves the output bit-identical."""
    w = make_custom(seed=103, lengths=[5, 33, 48, 70], num_pages=24)
    tb = w.block_tables[0]
    base = oracle.paged_decode_attention(w.q[0], w.k_pool, w.v_pool, tb, w.context_lens)
    perm = np.random.default_rng(7).permutation(w.num_pages)
    k2 = np.empty_like(w.k_pool)
    v2 = np.empty_like(w.v_pool)
    k2[perm] = w.k_pool
    v2[perm] = w.v_pool
    tb2 = np.where(tb >= 0, perm[np.maximum(tb, 0)], -1).astype(np.int32)
    moved = oracle.paged_decode_attention(w.q[0], k2, v2, tb2, w.context_lens)
    assert np.array_equal(base, moved)


def check_online_equals_two_pass():
    """O5: chunked online softmax folded with the pairwise merge rule == two-pass softmax."""
    rng = np.random.default_rng(104)
    for L in (2, 31, 100, 257):
        q, k, v = one_sequence(rng, L)
        qq, kk, vv = as_f64(q), as_f64(k), as_f64(v)
        two = oracle.attend_one(qq, kk, vv, 0.125)
        cuts = sorted(rng.choice(np.arange(1, L), size=min(L - 1, 5), replace=False)) if L > 1 else []
        online = oracle.attend_one_online(qq, kk, vv, 0.125, cuts)
        assert np.max(np.abs(two - online)) <= 1e-12, f"L={L}"
        # one chunk per token: the merge rule alone does all the work
        per_token = oracle.attend_one_online(qq, kk, vv, 0.125, list(range(1, L)))
        assert np.max(np.abs(two - per_token)) <= 1e-12, f"L={L} per-token"


def softmax_probe(xs):
    """q = 8 e0, K[t] = x_t e0, V[t] = e_t: the scores are exactly x_t and out[h] = softmax(x)."""
    L = len(xs)
    assert L <= 64
    q = np.zeros((8, 64), dtype=np.uint16)
    q[:, 0] = bits(8.0)
    k = np.zeros((L, 2, 64), dtype=np.uint16)
    k[:, :, 0] = bits(np.asarray(xs, dtype=np.float32))[:, None]
    v = np.zeros((L, 2, 64), dtype=np.uint16)
    for t in range(L):
        v[t, :, t] = bits(1.0)
    return q, k, v


def check_softmax_rows():
    """O6: stress rows through the public attention; compared to math.exp and the row-sum
    criterion of the pages' softmax test."""
    with open(os.path.join(GOLDEN, "softmax_rows.json")) as f:
        golden = json.load(f)
    tol = golden["row_sum_tolerance"]
    rng = np.random.default_rng(105)
    for name, xs in golden["rows"].items():
        q, k, v = softmax_probe(xs)
        out = run_paged(q, k, v, rng)
        m = max(xs)
        den = math.fsum(math.exp(x - m) for x in xs)
        expect = np.array([math.exp(x - m) / den for x in xs])
        for h in range(8):
            p = out[h, : len(xs)]
            assert np.all(np.isfinite(out[h])), name
            assert abs(p.sum() - 1.0) <= tol, name
            assert np.max(np.abs(p - expect)) <= 1e-15, name
            assert np.all(out[h, len(xs):] == 0.0), name


def check_spike():
    """O7: one score 50 above the rest returns that token's V row up to e^-50 terms."""
    rng = np.random.default_rng(106)
    L = 12
    xs = [0.0] * L
    xs[5] = 50.0
    q, k, _ = softmax_probe(xs)
    v = normal_bf16(rng, (L, 2, 64))
    out = run_paged(q, k, v, rng)
    vv = as_f64(v)
    bound = (L - 1) * math.exp(-50.0) * 2 * np.abs(vv).max()
    for h in range(8):
        assert np.max(np.abs(out[h] - vv[5, h // 4])) <= bound


def check_gqa_mapping():
    """O8: V rows constant g + 1 on KV head g give out[h] = h // 4 + 1."""
    rng = np.random.default_rng(107)
    hkv, group, L = 8, 4, 21
    q = normal_bf16(rng, (hkv * group, 64))
    k = normal_bf16(rng, (L, hkv, 64))
    v = np.zeros((L, hkv, 64), dtype=np.uint16)
    for g in range(hkv):
        v[:, g, :] = bits(float(g + 1))
    out = run_paged(q, k, v, rng)
    for h in range(hkv * group):
        assert np.max(np.abs(out[h] - (h // group + 1))) <= 1e-13, f"head {h}"


def check_two_tokens():
    """O9: scores (0, x) give (v0 + e^x v1) / (1 + e^x)."""
    rng = np.random.default_rng(108)
    for x in (-3.5, 0.0, 0.75, 6.0):
        q, k, _ = softmax_probe([0.0, x])
        v = normal_bf16(rng, (2, 2, 64))
        out = run_paged(q, k, v, rng)
        vv = as_f64(v)
        for h in range(8):
            g = h // 4
            expect = (vv[0, g] + math.exp(x) * vv[1, g]) / (1.0 + math.exp(x))
            assert np.max(np.abs(out[h] - expect)) <= 1e-15, f"x={x} head {h}"


def poison_outside_context(w, layer=0):
    """Copies of the pools with NaN in every slot that no sequence's context covers."""
    keep = np.zeros((w.num_pages, 16), dtype=bool)
    for b in range(w.batch):
        L = int(w.context_lens[b])
        for t in range(L):
            keep[w.block_tables[layer, b, t // 16], t % 16] = True
    kp = w.k_pool.copy()
    vp = w.v_pool.copy()
    kp.transpose(0, 2, 1, 3)[~keep] = NAN_BITS
    vp.transpose(0, 2, 1, 3)[~keep] = NAN_BITS
    return kp, vp, int((~keep).sum())


def check_poison():
    """O10: NaN in unused slots of last pages and in unreferenced pages changes nothing."""
    w = make_custom(seed=109, lengths=[3, 16, 17, 45], num_pages=16)
    clean = oracle.paged_decode_attention(w.q[0], w.k_pool, w.v_pool, w.block_tables[0], w.context_lens)
    kp, vp, n = poison_outside_context(w)
    assert n > 0
    dirty = oracle.paged_decode_attention(w.q[0], kp, vp, w.block_tables[0], w.context_lens)
    assert np.all(np.isfinite(dirty))
    assert np.array_equal(clean, dirty)


def check_append():
    """O11: appending into a NaN pool changes exactly the target rows, bit-for-bit."""
    w = make_custom(seed=110, lengths=[1, 16, 17, 40, 33], num_pages=20)
    kp = np.full_like(w.k_pool, NAN_BITS)
    vp = np.full_like(w.v_pool, NAN_BITS)
    k2, v2 = oracle.kv_append(kp, vp, w.block_tables[0], w.positions, w.k_new[0], w.v_new[0])
    changed_k = np.argwhere(np.any(k2 != NAN_BITS, axis=-1))
    assert len(changed_k) == w.batch * w.num_kv_heads
    for b in range(w.batch):
        pos = int(w.positions[b])
        page = w.block_tables[0, b, pos // 16]
        for g in range(w.num_kv_heads):
            assert np.array_equal(k2[page, g, pos % 16], w.k_new[0, b, g])
            assert np.array_equal(v2[page, g, pos % 16], w.v_new[0, b, g])
    assert np.sum(np.any(v2 != NAN_BITS, axis=-1)) == w.batch * w.num_kv_heads


def check_append_then_attend_single():
    """Append at position 0, then attend over L = 1: the output is the appended V row."""
    w = make_custom(seed=111, lengths=[1, 1], num_pages=6)
    k2, v2 = oracle.kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.k_new[0], w.v_new[0])
    out = oracle.paged_decode_attention(w.q[0], k2, v2, w.block_tables[0], w.context_lens)
    for b in range(2):
        for h in range(32):
            assert np.array_equal(out[b, h], as_f64(w.v_new[0, b, h // 4]))


def check_torch_sdpa():
    """O12: torch scaled_dot_product_attention in float64 on the gathered rows."""
    import torch

    w = make_custom(seed=112, lengths=[7, 64, 130], num_pages=20)
    got = oracle.paged_decode_attention(w.q[0], w.k_pool, w.v_pool, w.block_tables[0], w.context_lens)
    for b in range(w.batch):
        L = int(w.context_lens[b])
        pages = w.block_tables[0, b, : (L + 15) // 16]
        k = as_f64(w.k_pool[pages]).transpose(1, 0, 2, 3).reshape(8, -1, 64)[:, :L]
        v = as_f64(w.v_pool[pages]).transpose(1, 0, 2, 3).reshape(8, -1, 64)[:, :L]
        kt = torch.from_numpy(np.ascontiguousarray(k)).repeat_interleave(4, dim=0)
        vt = torch.from_numpy(np.ascontiguousarray(v)).repeat_interleave(4, dim=0)
        qt = torch.from_numpy(as_f64(w.q[0, b])).unsqueeze(1)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.125).squeeze(1).numpy()
        assert np.max(np.abs(got[b] - ref)) <= 1e-12, f"sequence {b}"


def check_bf16_rounding():
    """O13: the BF16 store rule (nearest, ties to even) against torch and hand-worked ties."""
    import torch

    assert oracle.bf16_round_nearest_even(np.float32([1.0 + 2.0**-8]))[0] == 0x3F80  # tie -> even
    assert oracle.bf16_round_nearest_even(np.float32([1.0 + 3 * 2.0**-8]))[0] == 0x3F82  # tie -> even
    assert oracle.bf16_round_nearest_even(np.float32([1.0 + 2.0**-8 + 2.0**-20]))[0] == 0x3F81
    assert oracle.bf16_round_nearest_even(np.float32([-1.0 - 2.0**-8]))[0] == 0xBF80
    x = np.random.default_rng(113).standard_normal(200000).astype(np.float32)
    ties = (np.arange(-2000, 2000, dtype=np.int32).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_round_nearest_even(x), ref)


def check_out_of_range():
    """O14: rows and contexts outside the table or the pool follow the library's error rule
    (append: not written; attention: an all-zero row), never Python's wrap-around indexing."""
    rng = np.random.default_rng(114)
    P = 6
    k_pool = normal_bf16(rng, (P, 2, 16, 64))
    v_pool = normal_bf16(rng, (P, 2, 16, 64))
    # table span = 2 pages = 32 positions
    tables = np.array([[3, 1], [2, 4], [-1, 0], [2, -1], [P, 1], [5, 0]], dtype=np.int32)
    positions = np.array([5, -1, 3, 20, 7, 32])  # only row 0 names a slot of the pool
    k_new = normal_bf16(rng, (6, 2, 64))
    v_new = normal_bf16(rng, (6, 2, 64))
    k2, v2 = oracle.kv_append(k_pool, v_pool, tables, positions, k_new, v_new)
    k_ref, v_ref = k_pool.copy(), v_pool.copy()
    k_ref[3, :, 5, :] = k_new[0]
    v_ref[3, :, 5, :] = v_new[0]
    assert np.array_equal(k2, k_ref) and np.array_equal(v2, v_ref)
    # attention: context 16 with a bad second entry is valid (only page 0 is read); the others
    # ask for a page that is not in the pool or for more than the table spans
    q = normal_bf16(rng, (6, 8, 64))
    tables = np.array([[3, -1], [3, 1], [-1, 2], [3, P], [3, 1], [3, 1]], dtype=np.int32)
    lens = np.array([16, 33, 4, 17, -1, 0])
    out = oracle.paged_decode_attention(q, k_pool, v_pool, tables, lens)
    assert np.array_equal(out[1:], np.zeros_like(out[1:]))
    k_rows = k_pool[3].transpose(1, 0, 2)  # [16][Hkv][D] of page 3
    v_rows = v_pool[3].transpose(1, 0, 2)
    assert np.max(np.abs(out[0] - brute_force(q[0], k_rows, v_rows, 0.125))) <= 1e-12


PINS = {
    "brute_force": check_brute_force,
    "single_token": check_single_token,
    "uniform_scores": check_uniform_scores,
    "page_permutation": check_page_permutation,
    "online_equals_two_pass": check_online_equals_two_pass,
    "softmax_rows": check_softmax_rows,
    "spike": check_spike,
    "gqa_mapping": check_gqa_mapping,
    "two_tokens": check_two_tokens,
    "poison": check_poison,
    "append": check_append,
    "append_then_attend_single": check_append_then_attend_single,
    "torch_sdpa": check_torch_sdpa,
    "bf16_rounding": check_bf16_rounding,
    "out_of_range": check_out_of_range,
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    PINS[name]()


# ------------------------------------------------------------------------------------------
# Planted mistakes: every one of them must make at least one pin fail
# ------------------------------------------------------------------------------------------

def _gather_transposed(pool, row, length):
    n = (length + 15) // 16
    blocks = pool[np.asarray(row[:n], dtype=np.int64)]
    return blocks.reshape(n * 16, pool.shape[1], pool.shape[3])[:length]  # forgot the transpose


def _gather_off_by_one(pool, row, length):
    n = (length + 15) // 16
    blocks = pool[np.asarray(row[:n], dtype=np.int64)]
    tokens = blocks.transpose(0, 2, 1, 3).reshape(n * 16, pool.shape[1], pool.shape[3])
    return tokens[1 : length + 1] if n * 16 > length else tokens[:length]


def _merge_wrong_sign(a, b):
    ma, da, oa = a
    mb, db, ob = b
    if da == 0.0:
        return b
    if db == 0.0:
        return a
    m = max(ma, mb)
    ea, eb = math.exp(m - ma), math.exp(m - mb)
    return m, da * ea + db * eb, oa * ea + ob * eb


MUTATIONS = {
    "gqa_modulo": ("kv_head_of", lambda h, group: h % (32 // group if group else 1), ["gqa_mapping", "brute_force"]),
    "gather_transposed": ("gather_context", _gather_transposed, ["brute_force", "torch_sdpa"]),
    "gather_off_by_one": ("gather_context", _gather_off_by_one, ["brute_force", "softmax_rows"]),
    "softmax_unnormalised": ("softmax_two_pass", lambda s: np.exp(s - s.max(axis=-1, keepdims=True)),
                             ["uniform_scores", "softmax_rows"]),
    "softmax_no_max_shift_sign": ("softmax_two_pass",
                                  lambda s: (lambda w: w / w.sum(axis=-1, keepdims=True))(np.exp(s.max(axis=-1, keepdims=True) - s)),
                                  ["softmax_rows", "two_tokens"]),
    "slot_swapped": ("locate_slot", lambda row, pos: (int(row[pos % 16]), pos // 16), ["append"]),
    "merge_wrong_sign": ("merge_states", _merge_wrong_sign, ["online_equals_two_pass"]),
    "append_unchecked": ("slot_in_pool", lambda row, pos, n: True, ["out_of_range"]),
    "attention_unchecked": ("context_in_pool", lambda row, length, n: True, ["out_of_range"]),
    "bf16_decode_shift": ("bf16_bits_to_f64",
                          lambda b: (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64),
                          ["single_token"]),
    "bf16_round_truncate": ("bf16_round_nearest_even",
                            lambda x: (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16),
                            ["bf16_rounding"]),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation, monkeypatch):
    attr, bad, pins = MUTATIONS[mutation]
    monkeypatch.setattr(PO, attr, bad)
    monkeypatch.setattr(oracle, attr, bad)
    caught = []
    for name in pins:
        try:
            PINS[name]()
        except (AssertionError, IndexError, ValueError):
            caught.append(name)
    assert caught, f"planted mistake {mutation!r} passed every pin in {pins}"
