"""The C ABI from a plain C++ program (no Python, no PyTorch): it owns its device memory and
stream, runs pkv_kv_append + pkv_paged_decode_attention and pkv_decode_step, and writes the
results, which are checked here against the FP64 oracle."""

import os
import subprocess

import numpy as np
import pytest

import oracle
from gpu_helpers import assert_close
from workloads import make_config, make_custom

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "host", "pkv_abi_client")  # built by build()


def run_client(tmp_path, w, partition_pages):
    hq = w.num_q_heads
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([w.batch, w.num_pages, w.num_kv_heads, w.max_blocks, partition_pages], dtype=np.int32).tobytes())
        for a in (w.block_tables[0], w.positions, w.q[0], w.k_new[0], w.v_new[0], w.k_pool, w.v_pool):
            f.write(np.ascontiguousarray(a).tobytes())
    print(f"[abi client] B={w.batch} pages={w.num_pages} pp={partition_pages}", flush=True)
    res = subprocess.run([CLIENT, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    raw = open(out, "rb").read()
    pool_bytes = w.k_pool.nbytes
    out_bytes = w.batch * hq * 64 * 4
    o = 0

    def take(n, dtype, shape):
        nonlocal o
        a = np.frombuffer(raw[o:o + n], dtype=dtype).reshape(shape)
        o += n
        return a

    kp = take(pool_bytes, np.uint16, w.k_pool.shape)
    vp = take(pool_bytes, np.uint16, w.v_pool.shape)
    out1 = take(out_bytes, np.float32, (w.batch, hq, 64))
    out2 = take(out_bytes, np.float32, (w.batch, hq, 64))
    kp2 = take(pool_bytes, np.uint16, w.k_pool.shape)
    vp2 = take(pool_bytes, np.uint16, w.v_pool.shape)
    assert o == len(raw)
    return kp, vp, out1, out2, kp2, vp2


@pytest.mark.parametrize("case", ["tiny", "mixed", "ragged_split"])
def test_c_client_matches_oracle(gpu, tmp_path, case):
    if not os.path.exists(CLIENT):
        pytest.fail(f"{CLIENT} is not built (build() compiles it)")
    if case == "ragged_split":
        w, pp = make_custom(seed=60, lengths=[1, 17, 300, 2048, 999, 64]), 8
    else:
        w, pp = make_config(case), 0
    kp, vp, out1, out2, kp2, vp2 = run_client(tmp_path, w, pp)
    rk, rv = oracle.kv_append(w.k_pool, w.v_pool, w.block_tables[0], w.positions, w.k_new[0], w.v_new[0])
    assert np.array_equal(kp, rk) and np.array_equal(vp, rv)
    assert np.array_equal(kp2, rk) and np.array_equal(vp2, rv)
    ref = oracle.paged_decode_attention(w.q[0], rk, rv, w.block_tables[0], w.context_lens)
    assert_close(out1, ref, f"{case} two calls")
    assert np.array_equal(out1, out2), "pkv_decode_step differs from the two calls"
