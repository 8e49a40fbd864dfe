"""Moving seeded workloads between numpy (BF16 bit patterns) and GPU tensors, and comparing."""

import numpy as np

ATOL = 2e-3
RTOL = 1e-2


def to_gpu_bf16(bits):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).cuda()


def to_gpu_i32(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def bf16_to_bits(t):
    import torch

    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def upload(w, layer=0):
    """Device tensors of one layer of a workload (pools are uploaded fresh each call)."""
    return {
        "k_pool": to_gpu_bf16(w.k_pool),
        "v_pool": to_gpu_bf16(w.v_pool),
        "block_tables": to_gpu_i32(w.block_tables[layer]),
        "positions": to_gpu_i32(w.positions),
        "context_lens": to_gpu_i32(w.context_lens),
        "q": to_gpu_bf16(w.q[layer]),
        "k_new": to_gpu_bf16(w.k_new[layer]),
        "v_new": to_gpu_bf16(w.v_new[layer]),
    }


def layer_tensors(w, layer):
    return {
        "block_tables": to_gpu_i32(w.block_tables[layer]),
        "q": to_gpu_bf16(w.q[layer]),
        "k_new": to_gpu_bf16(w.k_new[layer]),
        "v_new": to_gpu_bf16(w.v_new[layer]),
    }


def assert_close(got, ref, what=""):
    """|got - ref| <= ATOL + RTOL * |ref| elementwise (ref from the FP64 oracle)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} elements out of tolerance; worst at {i}: got {got[i]!r} ref {ref[i]!r}"
        )
    return float(err.max()), float((err / np.maximum(np.abs(ref), 1e-2)).max())
