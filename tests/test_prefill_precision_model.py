"""The precision reading behind the prefill kernel's FP16 second product, as a CPU check.

The kernel rounds each softmax weight to FP16 (round to nearest even, 11 significant bits) before
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
                wt = np.exp(s_ - s_.max())
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
