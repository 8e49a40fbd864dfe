"""The C ABI without a GPU: the library loads, exports every declared symbol, and its synchronous
host checks return the documented status codes before anything reaches the device."""

import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_cache_pages_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")

OK, NULL, SHAPE, UNSUP, WS, VALID, HIP, ALIGN = range(8)
FAKE = 0x10000  # a 16-byte aligned non-null address that the checks below never dereference


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkv.LIB_PATH):
        pytest.fail("libpagedkv.so is not built (run __graft_entry__.build())")
    return pkv.library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert names, "no declarations parsed"
    assert set(names) == set(pkv.SIGNATURES), "binding signatures and header disagree"
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.pkv_abi_version() == 1
    for code in range(12):
        assert lib.pkv_status_string(code)
    assert b"aligned" in lib.pkv_status_string(ALIGN)


def test_partition_planning():
    plan = lambda b, h, t, c: pkv.plan_partition_pages(b, h, t, num_cus=c)
    assert plan(256, 8, 128, 256) == 128  # 2048 (sequence, head) workgroups: no split
    assert plan(1, 8, 128, 256) == 8  # one long sequence: 16 partitions of 8 pages (the minimum)
    assert plan(4, 8, 128, 256) == 16  # about one workgroup per compute unit
    assert plan(8, 8, 128, 256) == 32
    assert plan(16, 8, 128, 256) == 64 and plan(17, 8, 128, 256) == 64 and plan(23, 8, 128, 256) == 64
    assert plan(24, 8, 128, 256) == 128 and plan(32, 8, 128, 256) == 128  # from 3/4 workgroup per CU
    assert plan(40, 8, 128, 256) == 128 and plan(64, 8, 128, 256) == 128
    assert plan(4, 8, 16, 256) == 16 and plan(4, 8, 24, 256) == 24  # up to 24 pages: never split
    assert plan(4, 8, 25, 256) == 8  # 25 pages: 4 partitions
    assert plan(4, 8, 48, 256) == 8  # 48 pages: 6 partitions
    assert plan(2, 8, 48, 256) == 8 and plan(2, 8, 128, 256) == 8
    for b in range(0, 300, 7):
        p = plan(b, 8, 128, 256)
        assert 8 <= p <= 128 and (p == 128 or p % 4 == 0)
    assert pkv.library().pkv_plan_partition_pages(-1, 8, 128, 256) == -1


def test_partition_planning_with_a_known_longest_context():
    plan = lambda b, t, mc: pkv.plan_partition_pages(b, 8, t, num_cus=256, max_context=mc)
    assert plan(1, 128, 37) == 128  # 3 pages: no split
    assert plan(1, 128, 256) == 128  # 16 pages: no split
    assert plan(1, 128, 384) == 128  # 24 pages: no split
    assert plan(1, 128, 385) == 8  # 25 pages: split
    assert plan(1, 128, 2048) == 8
    assert plan(17, 128, 856) == 28  # 54 pages over 2 partitions
    assert plan(17, 128, 2048) == 64
    assert plan(4, 128, 1024) == 8 and plan(8, 128, 1024) == 16 and plan(16, 128, 1024) == 32
    assert plan(40, 128, 1024) == 128 and plan(40, 128, 2048) == 128
    assert plan(1, 300, 37) == 256  # the 256-page cap
    assert plan(256, 128, 2048) == 128
    for b in (1, 5, 16, 17, 40):
        assert plan(b, 128, None) == pkv.plan_partition_pages(b, 8, 128, num_cus=256)
    lib = pkv.library()
    assert lib.pkv_plan_partition_pages_for_context(1, 8, 128, -1, 256) == 8
    assert lib.pkv_plan_partition_pages_for_context(1, 8, 128, 0, 256) == 128
    assert lib.pkv_plan_partition_pages_for_context(1, 8, 128, 5000, 256) == 8  # clamped to the table
    assert lib.pkv_plan_partition_pages_for_context(-1, 8, 128, 100, 256) == -1


def test_workspace_bytes():
    assert pkv.decode_workspace_bytes(4, 32, 128, 128) == 0
    assert pkv.decode_workspace_bytes(4, 32, 128, 200) == 0
    # partials (64 outputs + max + sum per sequence, query head and partition), 128 bytes of
    # alignment room, then a 128-byte counter per (sequence, KV head)
    assert pkv.decode_workspace_bytes(1, 32, 128, 4) == 1 * 32 * 32 * 66 * 4 + 128 + 1 * 8 * 128
    assert pkv.decode_workspace_bytes(3, 32, 128, 20) == 3 * 32 * 7 * 66 * 4 + 128 + 3 * 8 * 128
    assert pkv.decode_workspace_bytes(5, 4, 300, 300) == 5 * 4 * 2 * 66 * 4 + 128 + 5 * 1 * 128  # 256-page cap


def _append(lib, pool, bt=FAKE, maxb=128, pos=FAKE, k=FAKE, v=FAKE, batch=1):
    return lib.pkv_kv_append(pool, bt, maxb, pos, k, v, batch, None)


def test_append_host_checks(lib):
    good = pkv.Pool(FAKE, FAKE, 8, 8, 64, 16)
    assert _append(lib, None) == NULL
    assert _append(lib, ctypes.byref(pkv.Pool(FAKE, FAKE, 8, 8, 128, 16))) == UNSUP
    assert _append(lib, ctypes.byref(pkv.Pool(FAKE, FAKE, 8, 8, 64, 32))) == UNSUP
    assert _append(lib, ctypes.byref(pkv.Pool(FAKE, FAKE, 0, 8, 64, 16))) == SHAPE
    assert _append(lib, ctypes.byref(good), batch=-1) == SHAPE
    assert _append(lib, ctypes.byref(good), maxb=0) == SHAPE
    assert _append(lib, ctypes.byref(good), batch=0) == OK  # no-op, nothing enqueued
    assert _append(lib, ctypes.byref(good), bt=None) == NULL
    assert _append(lib, ctypes.byref(good), k=None) == NULL
    assert _append(lib, ctypes.byref(good), k=FAKE + 2) == ALIGN
    assert _append(lib, ctypes.byref(pkv.Pool(FAKE + 8, FAKE, 8, 8, 64, 16))) == ALIGN


def _decode(lib, q=FAKE, kp=FAKE, vp=FAKE, pages=8, bt=FAKE, maxb=128, lens=FAKE, out=FAKE, odt=0, batch=1, hq=32,
            hkv=8, d=64, bs=16, scale=0.125, pp=128, ws=None, wsb=0):
    return lib.pkv_paged_decode_attention(q, kp, vp, pages, bt, maxb, lens, out, odt, batch, hq, hkv, d, bs, scale, pp,
                                          ws, wsb, None)


def test_decode_host_checks(lib):
    assert _decode(lib, batch=-1) == SHAPE
    assert _decode(lib, pages=0) == SHAPE
    assert _decode(lib, scale=0.0) == SHAPE
    assert _decode(lib, scale=float("nan")) == SHAPE
    assert _decode(lib, scale=float("inf")) == SHAPE
    assert _decode(lib, odt=7) == SHAPE
    assert _decode(lib, d=128) == UNSUP
    assert _decode(lib, bs=32) == UNSUP
    assert _decode(lib, hq=16) == UNSUP  # group of 2
    assert _decode(lib, batch=0) == OK
    assert _decode(lib, batch=65536) == SHAPE  # one grid dimension per sequence
    assert _decode(lib, q=None) == NULL
    assert _decode(lib, lens=None) == NULL
    assert _decode(lib, out=FAKE + 4) == ALIGN
    # an explicit split needs a workspace of the documented size
    need = pkv.decode_workspace_bytes(1, 32, 128, 4)
    assert _decode(lib, pp=4) == WS
    assert _decode(lib, pp=4, ws=FAKE, wsb=need - 1) == WS
    assert _decode(lib, pp=4, ws=FAKE + 8, wsb=need) == ALIGN


def test_static_scratch_step_host_checks(lib):
    """pkv_decode_step_static rejects a split larger than its static scratch before touching the
    device, and checks its arguments like pkv_decode_step."""
    pool = pkv.Pool(FAKE, FAKE, 64, 8, 64, 16)
    args = lambda batch, maxb, pp, q=FAKE, pos=FAKE: (ctypes.byref(pool), q, FAKE, maxb, pos, FAKE, FAKE, FAKE, 1,
                                                       batch, 32, 0.125, pp, None)
    assert pkv.decode_workspace_bytes(64, 32, 128, 4) > pkv.STATIC_SCRATCH_BYTES
    assert lib.pkv_decode_step_static(*args(64, 128, 4)) == 11  # PKV_ERR_SCRATCH
    assert b"static scratch" in lib.pkv_status_string(11)
    assert lib.pkv_decode_step_static(*args(1, 128, 16, q=None)) == NULL
    assert lib.pkv_decode_step_static(*args(1, 128, 16, pos=None)) == NULL
    assert lib.pkv_decode_step_static(*args(0, 128, 16)) == OK
    assert lib.pkv_decode_step_static(None, *args(1, 128, 16)[1:]) == NULL


def test_rope_append_host_checks(lib):
    good = pkv.Pool(FAKE, FAKE, 8, 8, 64, 16)

    def call(pool=ctypes.byref(good), q=FAKE, q_out=FAKE, hq=32, cos=FAKE, sin=FAKE, rows=16, batch=1):
        return lib.pkv_rope_kv_append(pool, FAKE, 128, FAKE, q, q_out, hq, FAKE, FAKE, cos, sin, rows, batch, None)

    assert call(pool=None) == NULL
    assert call(rows=0) == SHAPE
    assert call(hq=0) == SHAPE
    assert call(batch=-1) == SHAPE
    assert call(pool=ctypes.byref(pkv.Pool(FAKE, FAKE, 8, 8, 32, 16))) == UNSUP
    assert call(batch=0) == OK
    assert call(cos=None) == NULL
    assert call(q_out=None) == NULL
    assert call(sin=FAKE + 4) == ALIGN
    assert call(q=FAKE + 2) == ALIGN


def test_decode_step_host_checks(lib):
    good = pkv.Pool(FAKE, FAKE, 8, 8, 64, 16)

    def call(pool=ctypes.byref(good), q=FAKE, pos=FAKE, kn=FAKE, out=FAKE, batch=1, hq=32, scale=0.125, pp=128, ws=None,
             wsb=0):
        return lib.pkv_decode_step(pool, q, FAKE, 128, pos, kn, FAKE, out, 0, batch, hq, scale, pp, ws, wsb, None)

    assert call(pool=None) == NULL
    assert call(pos=None) == NULL
    assert call(kn=None) == NULL
    assert call(batch=-1) == SHAPE
    assert call(scale=-1.0) == SHAPE
    assert call(hq=8) == UNSUP
    assert call(batch=0) == OK
    assert call(kn=FAKE + 2) == ALIGN
    assert call(pp=4) == WS


def test_host_validators():
    bt = np.full((3, 4), -1, dtype=np.int32)
    bt[0, :2] = [5, 6]
    bt[1, :1] = [2]
    bt[2, :4] = [0, 1, 3, 4]
    assert pkv.validate_decode_host(bt, [20, 16, 64], 8) == (OK, -1)
    assert pkv.validate_decode_host(bt, [20, 17, 64], 8) == (VALID, 1)  # needs block 1 of row 1
    assert pkv.validate_decode_host(bt, [20, 16, 65], 8) == (VALID, 2)  # beyond the table
    assert pkv.validate_decode_host(bt, [-1, 16, 64], 8) == (VALID, 0)
    assert pkv.validate_decode_host(bt, [0, 0, 0], 8) == (OK, -1)
    assert pkv.validate_decode_host(bt, [20, 16, 64], 6) == (VALID, 0)  # row 0 holds page 6 of a 6-page pool
    assert pkv.validate_append_host(bt, [19, 15, 63], 8) == (OK, -1)
    assert pkv.validate_append_host(bt, [19, 16, 63], 8) == (VALID, 1)  # block 1 unassigned
    assert pkv.validate_append_host(bt, [19, 15, 64], 8) == (VALID, 2)  # position past the table
    bt2 = bt.copy()
    bt2[1, 0] = 6
    assert pkv.validate_append_host(bt2, [19, 3, 63], 8) == (VALID, 1)  # same (page 6, slot 3) twice
    assert pkv.validate_append_host(bt2, [19, 4, 63], 8) == (OK, -1)


def test_prefill_host_checks(lib):
    good = pkv.Pool(FAKE, FAKE, 8, 8, 64, 16)

    def app(pool=ctypes.byref(good), bt=FAKE, maxb=128, cu=FAKE, sp=FAKE, k=FAKE, v=FAKE, batch=1, tokens=4, mpl=4):
        return lib.pkv_prefill_kv_append(pool, bt, maxb, cu, sp, k, v, batch, tokens, mpl, None)

    def att(pool=ctypes.byref(good), q=FAKE, cu=FAKE, out=FAKE, odt=0, batch=1, tokens=4, mpl=4, hq=32, scale=0.125):
        return lib.pkv_paged_prefill_attention(pool, q, FAKE, 128, cu, FAKE, out, odt, batch, tokens, mpl, hq, scale,
                                               None)

    assert app(pool=None) == NULL
    assert app(batch=-1) == SHAPE and app(tokens=-1) == SHAPE and app(mpl=-1) == SHAPE and app(maxb=0) == SHAPE
    assert app(batch=70000) == SHAPE
    assert app(pool=ctypes.byref(pkv.Pool(FAKE, FAKE, 8, 8, 128, 16))) == UNSUP
    assert app(batch=0) == OK and app(tokens=0) == OK and app(mpl=0) == OK
    assert app(cu=None) == NULL and app(k=None) == NULL and app(sp=None) == NULL
    assert app(k=FAKE + 2) == ALIGN
    assert app(pool=ctypes.byref(pkv.Pool(FAKE + 4, FAKE, 8, 8, 64, 16))) == ALIGN
    assert att(pool=None) == NULL
    assert att(scale=0.0) == SHAPE and att(scale=float("nan")) == SHAPE and att(odt=5) == SHAPE
    assert att(hq=0) == SHAPE and att(hq=16) == UNSUP
    assert att(batch=0) == OK
    assert att(q=None) == NULL and att(cu=None) == NULL and att(out=None) == NULL
    assert att(out=FAKE + 8) == ALIGN


def test_prefill_validator():
    bt = np.full((3, 4), -1, dtype=np.int32)
    bt[0, :2] = [5, 6]
    bt[1, :1] = [2]
    bt[2, :4] = [0, 1, 3, 4]
    cu, sp = [0, 20, 36, 100], [0, 0, 0]
    assert pkv.validate_prefill_host(bt, cu, sp, 100, 64, 8) == (OK, -1)
    assert pkv.validate_prefill_host(bt, cu, sp, 99, 64, 8) == (VALID, 2)  # rows past num_tokens
    assert pkv.validate_prefill_host(bt, cu, sp, 100, 63, 8) == (VALID, 2)  # longer than the bound
    assert pkv.validate_prefill_host(bt, [0, 20, 37, 100], sp, 100, 64, 8) == (VALID, 1)  # needs block 1 of row 1
    assert pkv.validate_prefill_host(bt, cu, [0, 0, 1], 100, 64, 8) == (VALID, 2)  # runs past the table
    assert pkv.validate_prefill_host(bt, cu, [-1, 0, 0], 100, 64, 8) == (VALID, 0)
    assert pkv.validate_prefill_host(bt, [0, 20, 19, 100], sp, 100, 81, 8) == (VALID, 1)  # negative length
    assert pkv.validate_prefill_host(bt, [0, 10, 26, 90], [10, 0, 0], 100, 64, 8) == (OK, -1)  # chunk behind 10
    bt2 = bt.copy()
    bt2[1, 0] = 6
    # row 0 fills page 6 slots 0..3 (positions 16..19); row 1 writes one token into page 6
    assert pkv.validate_prefill_host(bt2, [0, 20, 21, 22], [0, 4, 0], 22, 64, 8) == (OK, -1)
    assert pkv.validate_prefill_host(bt2, [0, 20, 21, 22], [0, 3, 0], 22, 64, 8) == (VALID, 1)  # (page 6, slot 3) twice


def test_finite_rows_validator():
    """Every BF16 pattern whose exponent field is all ones (infinities and NaNs) is rejected; the
    largest finite values, zeros of both signs and subnormals pass."""
    from workloads import f32_to_bf16_bits

    rows = f32_to_bf16_bits(np.random.default_rng(0).standard_normal((6, 8, 64)).astype(np.float32))
    rows[0, 0, :4] = [0x7F7F, 0xFF7F, 0x8000, 0x0001]  # +-max finite, -0, smallest subnormal
    assert pkv.validate_finite_rows_host(rows) == (OK, -1)
    for bits in (0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F81):  # +inf, -inf, NaNs of both signs
        bad = rows.copy()
        bad[4, 7, 63] = bits
        bad[5, 0, 0] = bits
        assert pkv.validate_finite_rows_host(bad) == (VALID, 4), hex(bits)
    assert pkv.validate_finite_rows_host(rows[:0]) == (OK, -1)
    lib = pkv.library()
    bad = ctypes.c_int32(-2)
    assert lib.pkv_validate_finite_rows_host(rows.ctypes.data, -1, 64, ctypes.byref(bad)) == SHAPE
    assert lib.pkv_validate_finite_rows_host(rows.ctypes.data, 1, 0, ctypes.byref(bad)) == SHAPE
    assert lib.pkv_validate_finite_rows_host(None, 1, 64, ctypes.byref(bad)) == NULL


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from paged_kv_cache_pages_amd import _binding

    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "libpagedkv.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        _binding.library()
