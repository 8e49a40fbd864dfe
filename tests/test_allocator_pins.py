"""Pins for the allocator reference model: hand-worked scenarios from the admission rules."""

import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import AllocatorModel


def test_budget_formula():
    m = AllocatorModel(num_pages=100000, layers=16, max_blocks=128)
    assert m.budget(17, 16) == 16 * 2  # prefix 17 + 16 - 1 = 32 tokens -> 2 pages per layer
    assert m.budget(17, 17) == 16 * 3  # 33 tokens -> 3 pages
    assert m.budget(1, 0) == 16 * 1  # at least the prompt
    assert m.budget(1, 1) == 16 * 1
    assert m.budget(2048, 5) == 16 * 128  # no room to generate: allowed output clamps to 0
    assert m.budget(2000, 100) == 16 * 128  # allowed 48 -> prefix 2047
    assert m.budget(16, 1) == 16 * 1 and m.budget(16, 2) == 16 * 2


def test_fifo_blocks_without_skipping():
    m = AllocatorModel(num_pages=64, layers=1, max_blocks=128)
    assert m.submit(1, 40 * 16, 1)  # 40 pages
    assert m.submit(2, 30 * 16, 1)  # 30 pages
    assert m.submit(3, 10 * 16, 1)  # 10 pages: would fit, but waits behind request 2
    assert m.admit() == [1]
    assert m.snapshot()["admission_waits"] == 1
    assert m.admit() == []
    assert m.release(1)
    assert m.admit() == [2, 3]
    assert m.snapshot()["credits_reserved"] == 40


def test_oversize_request_is_rejected():
    m = AllocatorModel(num_pages=100, layers=16, max_blocks=128)
    assert not m.submit(1, 7 * 16, 1)  # 16 layers x 7 pages = 112 > 100
    assert m.submit(2, 6 * 16, 1)  # 96 fits
    assert m.snapshot()["rejected"] == 1
    assert not m.submit(3, 3000, 1)  # longer than the context
    assert not m.submit(4, 0, 1)


def test_lazy_pages_from_the_back_and_reuse_after_release():
    m = AllocatorModel(num_pages=10, layers=2, max_blocks=4, free_order=list(range(100, 110)))
    assert m.submit(7, 20, 20)  # prefix 20 + 20 - 1 = 39 tokens -> 3 pages per layer -> 6 credits
    assert m.admit() == [7]
    assert m.table(7) == [[-1] * 4, [-1] * 4]
    assert m.ensure(7, 0)
    assert m.table(7) == [[109, -1, -1, -1], [108, -1, -1, -1]]  # popped from the back, layer order
    assert m.ensure(7, 15)  # same block: nothing new
    assert m.snapshot()["free_pages"] == 8
    assert m.ensure(7, 16)
    assert m.ensure(7, 32)
    assert m.table(7) == [[109, 107, 105, -1], [108, 106, 104, -1]]
    assert not m.ensure(7, 48)  # a fourth page per layer would exceed the 6 credits
    assert m.snapshot()["peak_assigned"] == 6
    assert m.release(7)
    # pages go back to the end of the free list, layer by layer in block order
    assert m.free == [100, 101, 102, 103, 109, 107, 105, 108, 106, 104]
    assert m.snapshot()["credits_reserved"] == 0 and not m.release(7)


@settings(max_examples=60, deadline=None, derandomize=True)
@given(ops=st.lists(st.tuples(st.sampled_from(["submit", "admit", "ensure", "release"]), st.integers(0, 9),
                              st.integers(1, 300), st.integers(0, 200)), max_size=60))
def test_invariants_under_random_operations(ops):
    m = AllocatorModel(num_pages=48, layers=3, max_blocks=20)
    next_pos = {}
    for op, rid, a, b in ops:
        if op == "submit" and rid not in m.active and all(r.rid != rid for r in m.waiting):
            m.submit(rid, a, b)
        elif op == "admit":
            for r in m.admit():
                next_pos[r] = 0
        elif op == "ensure" and rid in m.active:
            pos = next_pos[rid]
            if m.ensure(rid, pos):
                next_pos[rid] = pos + 1 + b % 20
        elif op == "release":
            m.release(rid)
        # invariants
        held = [p for r in m.active.values() for row in r.tables for p in row if p != -1]
        assert len(held) == len(set(held))
        assert len(held) + len(m.free) == m.num_pages
        assert sorted(held + m.free) == list(range(m.num_pages))
        assert m.credits_reserved == sum(r.credits for r in m.active.values()) <= m.num_pages
        assert all(r.assigned <= r.credits for r in m.active.values())
        # every admitted request can still take all of its remaining credits as pages
        assert sum(r.credits - r.assigned for r in m.active.values()) <= len(m.free)


def test_static_batching_waits_for_the_whole_group():
    m = AllocatorModel(num_pages=100, layers=1, max_blocks=128, static=True)
    for rid in (1, 2, 3):
        assert m.submit(rid, 16, 1)
    assert m.admit() == [1, 2, 3]
    assert m.submit(4, 16, 1)
    assert m.admit() == [] and m.snapshot()["admission_waits"] == 1
    m.release(1)
    m.release(2)
    assert m.admit() == []  # request 3 still runs
    m.release(3)
    assert m.admit() == [4]


def test_admission_limit_and_duplicates():
    m = AllocatorModel(num_pages=100, layers=1, max_blocks=128)
    for rid in (1, 2, 3):
        assert m.submit(rid, 16, 1)
    assert not m.submit(2, 16, 1)  # already queued
    assert m.admit(limit=2) == [1, 2]
    assert m.snapshot()["admission_waits"] == 0  # a capped pass is not a wait
    assert not m.submit(1, 16, 1)  # already active
    assert m.snapshot()["rejected"] == 0
    assert m.admit() == [3]


def test_prepare_step_tables_and_first_failure():
    m = AllocatorModel(num_pages=8, layers=2, max_blocks=3, free_order=list(range(8)))
    assert m.submit(5, 16, 1) and m.submit(6, 17, 1)  # 2 and 4 credits
    assert m.admit() == [5, 6]
    tables, bad = m.prepare_step([5, 6], [15, 16])
    assert bad == -1 and tables.shape == (2, 2, 3)
    assert tables[:, 0].tolist() == [[7, -1, -1], [6, -1, -1]]
    assert tables[:, 1].tolist() == [[-1, 5, -1], [-1, 4, -1]]  # only the block holding position 16
    assert m.snapshot()["largest_batch"] == 2
    tables, bad = m.prepare_step([6, 5], [0, 16])  # request 5 has no credit for a second page
    assert tables is None and bad == 1
    assert m.table(6)[0][:2] == [3, 5]
