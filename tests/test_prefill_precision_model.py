"""The precision reading behind the prefill kernel's FP16 second product, as a CPU check.

The kernel rounds each softmax weight (times a fixed 2^7) to FP16 (round to nearest even, 11 significant bits) before
the weights-times-V product, and takes V in FP16 (exact for these N(0, 1) BF16 values); the
denominator is the sum of the same rounded weights. This models that rounding in numpy (no GPU
code involved) on the rows where rounding hurts most, rows with few keys, and compares with the
FP64 oracle under the parity tolerance. FP16 weights must stay well inside it; a single BF16
weight (8 significant bits) must not, which is why the kernel's fallback pass carries BF16
weights as a hi + lo pair.
"""

import numpy as np

import oracle
from workloads import make_prefill

ATOL, RTOL = 2e-3, 1e-2
SHIFT = 7.0  # log2 of the fixed factor the kernel's weights carry (it cancels in the ratio)


def _bf16_round(w):
    u = w.astype(np.float32).view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def _worst_ratio(w, fmt):
    """Largest |model - exact| / (ATOL + RTOL |exact|) over every row and head of prompt set w."""
    rk, rv = oracle.prefill_kv_append(w.k_pool, w.v_pool, w.block_tables, w.cu_seqlens, w.start_pos, w.k_new,
                                      w.v_new)
    K, V = oracle.bf16_bits_to_f64(rk), oracle.bf16_bits_to_f64(rv)
    q = oracle.bf16_bits_to_f64(w.q)
    exact = oracle.paged_prefill_attention(w.q, rk, rv, w.block_tables, w.cu_seqlens, w.start_pos)
    worst = 0.0
    for b in range(len(w.cu_seqlens) - 1):
        r0, r1, st = int(w.cu_seqlens[b]), int(w.cu_seqlens[b + 1]), int(w.start_pos[b])
        for i in range(r1 - r0):
            n = st + i + 1
            keys = [(int(w.block_tables[b, t // 16]), t % 16) for t in range(n)]
            for h in range(q.shape[1]):
                g = h // 4
                kc = np.stack([K[pg, g, s] for pg, s in keys])
                vc = np.stack([V[pg, g, s] for pg, s in keys])
                s_ = kc @ q[r0 + i, h] * 0.125
                wt = np.exp(s_ - s_.max()) * 2.0 ** SHIFT
                wr = wt.astype(np.float16).astype(np.float64) if fmt == "f16" else _bf16_round(wt)
                model = (wr @ vc) / wr.sum()
                ref = exact[r0 + i, h]
                worst = max(worst, float(np.max(np.abs(model - ref) / (ATOL + RTOL * np.abs(ref)))))
    return worst


def test_fp16_weights_stay_well_inside_the_tolerance():
    for w in (make_prefill(22, [3] * 12, [0] * 12), make_prefill(21, [1, 2, 5, 8, 17, 33], [0, 0, 0, 0, 0, 0])):
        assert _worst_ratio(w, "f16") < 0.5


def test_single_bf16_weights_do_not():
    assert _worst_ratio(make_prefill(22, [3] * 40, [0] * 40), "bf16") > 1.0


# Long, peaked rows. The kernel's weights are 2^(x - m + 7) in log2 units: a lazy per-query anchor m
# somewhere between the row's maximum minus 8 and its maximum, and a fixed factor 2^7 that cancels
# in the ratio but keeps small weights out of FP16's subnormal range; then rounded to FP16. Normal
# FP16 weights keep a relative error of at most 2^-11; below 2^-14 (a weight 2^-21 of the
# anchor's) each carries an absolute error of at most 2^-25, and below 2^-25 it becomes 0.


def _fp16_row(scores_log2, v, anchor, shift=SHIFT):
    w = np.exp2(scores_log2 - anchor + shift).astype(np.float16).astype(np.float64)
    return (w @ v) / w.sum(), w


def _exact_row(scores_log2, v):
    e = np.exp2(scores_log2 - scores_log2.max())
    return (e @ v) / e.sum()


def _ratio(model, exact):
    return float(np.max(np.abs(model - exact) / (ATOL + RTOL * np.abs(exact))))


def _long_rows(rng, v_scales):
    """2048- and 4096-key rows of N(0, 1) scores (the N(0, 1) BF16 inputs at scale 1/8) in log2
    units with one key lifted 4 to 30 above the rest, V ~ N(0, v_scale) clipped to 1e3."""
    for n in (2048, 4096):
        for gap in (4.0, 12.0, 20.0, 30.0):
            for v_scale in v_scales:
                s = rng.standard_normal(n) / np.log(2.0)
                s[rng.integers(n)] = s.max() + gap
                yield s, np.clip(rng.standard_normal((n, 64)) * v_scale, -1e3, 1e3)


def test_fp16_weights_on_long_rows_with_one_dominant_key():
    """Up to |V| ~ 1e2 the FP16 weights stay inside half the tolerance, for the anchor at the
    maximum and 8.99 below it (past the lazy limit: the kernel moves the anchor once a scaled score
    lies more than 8 above it, so its weights, times 2^7, stay at most 2^15)."""
    worst = 0.0
    for s, v in _long_rows(np.random.default_rng(5), (1.0, 10.0, 1e2)):
        exact = _exact_row(s, v)
        for lag in (0.0, 8.99):
            worst = max(worst, _ratio(_fp16_row(s, v, s.max() - lag)[0], exact))
    assert worst < 0.5, worst


def test_fp16_weights_error_bound_on_long_rows():
    """For any |V| the error of a row stays under the rounding bound
    (2^-11 sum|w v| + 2^-11 |out| sum w + n 2^-25 max|V| (1 + |out| / max|V|)) / sum w over the
    rounded weights w. That bound exceeds the absolute tolerance once |V| reaches ~1e3 on these
    rows, where some output dims cancel to near 0: the FP16 weights' limit (the row's BF16 output
    rounding, 2^-9 of |out|, is coarser still)."""
    worst = 0.0
    for s, v in _long_rows(np.random.default_rng(6), (1.0, 1e2, 1e3)):
        exact = _exact_row(s, v)
        for lag in (0.0, 8.99):
            model, w = _fp16_row(s, v, s.max() - lag)
            n = len(s)
            bound = (2.0 ** -11 * (np.abs(w) @ np.abs(v)) + 2.0 ** -11 * np.abs(exact) * w.sum()
                     + n * 2.0 ** -25 * (np.abs(v).max() + np.abs(exact))) / w.sum()
            assert np.all(np.abs(model - exact) <= bound * (1 + 1e-9))
            worst = max(worst, _ratio(model, exact))
    assert worst > 0.5  # the |V| ~ 1e3 rows come close to or past the tolerance


def test_weight_shift_keeps_small_weights_out_of_the_subnormal_range():
    """An adversarial row: every non-dominant key 25.3 below the maximum (a weight just under
    FP16's smallest subnormal, 2^-25, without the shift) with V = +1e3 while the dominant key has
    V = 0. Unshifted FP16 weights drop all of it and miss the tolerance; with the factor 2^7 the
    weights are 2^-18.3 and the row is inside it."""
    n = 4096
    s = np.full(n, -25.3)
    s[0] = 0.0
    v = np.full((n, 64), 1e3)
    v[0] = 0.0
    exact = _exact_row(s, v)
    plain, _ = _fp16_row(s, v, 0.0, shift=0.0)
    assert np.all(plain == 0.0) and _ratio(plain, exact) > 1.0
    shifted, _ = _fp16_row(s, v, 0.0)
    assert _ratio(shifted, exact) < 0.5
    # at the largest lag the kernel keeps (8), and at 8.99, the shifted weight is a finite FP16 number
    assert np.isfinite(np.float16(2.0 ** (8.0 + SHIFT))) and np.isfinite(np.float16(2.0 ** (8.99 + SHIFT)))
