"""Reference model of the host page allocator with admission credits.

TEST INFRASTRUCTURE ONLY (imported by ``tests/``; the C++ allocator in the library never uses it).

The rules, from "6 Hours of YouTube and 85 handtyped pages of notes on LLM Inference", section
"Current scope", and "The prefill path: flowing the entire prompt at once", section "Distributing
K/V into paged blocks":

* Admission reserves room for a request's largest processed prefix, ``prompt + allowed_new - 1``
  tokens, rounded up to 16-token pages, in every layer.  The output budget is clamped to the
  context limit.  These credits are separate from physical pages.
* Physical pages are assigned lazily: a block-table entry of -1 means "unassigned", and the page
  comes from the back of the free list.
* Requests wait first-in-first-out when their budget cannot fit beside the active requests; a
  waiting request blocks the ones behind it.  A request whose budget exceeds the whole pool is
  rejected.
* Completion returns the request's pages (to the back of the free list) and its remaining credits.
* Static batching admits the next group only once every active request has finished; continuous
  batching admits whenever credits allow.
* A request never holds more physical pages than its credits, so with the sum of credits of the
  active requests within the pool, no lazy assignment of an admitted request can fail.

Readings where the page is silent: the allowed output is ``min(max_new, context - prompt)`` (prompt
plus output fit in the context); a request processes at least its prompt, so the prefix is
``max(prompt, prompt + allowed_new - 1)``; "admission waits" counts admission passes that stopped
at a request that did not fit; released pages go back layer by layer in block order; a request id
may not be queued twice; one admission pass may be capped at ``limit`` requests (a cap is not a
wait).
"""

from __future__ import annotations

from dataclasses import dataclass, field

BLOCK = 16


def pages_for(tokens: int) -> int:
    return (tokens + BLOCK - 1) // BLOCK


@dataclass
class Request:
    rid: int
    prompt: int
    max_new: int
    credits: int = 0
    assigned: int = 0
    tables: list = field(default_factory=list)  # [layer][block] page or -1


class AllocatorModel:
    def __init__(self, num_pages: int, layers: int, max_blocks: int, free_order=None, static: bool = False):
        self.static = static
        self.num_pages = num_pages
        self.layers = layers
        self.max_blocks = max_blocks
        self.context = max_blocks * BLOCK
        self.free = list(range(num_pages)) if free_order is None else [int(p) for p in free_order]
        self.waiting: list[Request] = []
        self.active: dict[int, Request] = {}
        self.credits_reserved = 0
        self.stats = {"peak_active": 0, "peak_assigned": 0, "largest_batch": 0, "admission_waits": 0,
                      "rejected": 0}

    # -- admission ------------------------------------------------------------------------
    def budget(self, prompt: int, max_new: int) -> int:
        allowed = max(0, min(max_new, self.context - prompt))
        prefix = max(prompt, prompt + allowed - 1)
        return self.layers * pages_for(prefix)

    def submit(self, rid: int, prompt: int, max_new: int) -> bool:
        """Queue a request; False (and counted as rejected) when it can never fit."""
        if rid in self.active or any(r.rid == rid for r in self.waiting):
            return False  # duplicate id: refused, not counted
        if prompt <= 0 or prompt > self.context or max_new < 0:
            self.stats["rejected"] += 1
            return False
        need = self.budget(prompt, max_new)
        if need > self.num_pages:
            self.stats["rejected"] += 1
            return False
        self.waiting.append(Request(rid, prompt, max_new, credits=need))
        return True

    def admit(self, limit: int | None = None) -> list[int]:
        admitted = []
        if self.static and self.active:
            if self.waiting:
                self.stats["admission_waits"] += 1
            return admitted
        while self.waiting and (limit is None or len(admitted) < limit) \
                and self.credits_reserved + self.waiting[0].credits <= self.num_pages:
            r = self.waiting.pop(0)
            r.tables = [[-1] * self.max_blocks for _ in range(self.layers)]
            self.active[r.rid] = r
            self.credits_reserved += r.credits
            admitted.append(r.rid)
        if self.waiting and (limit is None or len(admitted) < limit):
            self.stats["admission_waits"] += 1
        self.stats["peak_active"] = max(self.stats["peak_active"], len(self.active))
        return admitted

    # -- step a0: lazy page assignment ----------------------------------------------------
    def ensure(self, rid: int, pos: int) -> bool:
        """Make the page holding token ``pos`` present in every layer of request ``rid``."""
        r = self.active.get(rid)
        if r is None or pos < 0 or pos >= self.context:
            return False
        blk = pos // BLOCK
        missing = sum(1 for layer in range(self.layers) if r.tables[layer][blk] == -1)
        # Never beyond the request's credits: that is what keeps every admitted request's lazy
        # assignments from running out of pages.
        if r.assigned + missing > r.credits or missing > len(self.free):
            return False
        for layer in range(self.layers):
            if r.tables[layer][blk] == -1:
                r.tables[layer][blk] = self.free.pop()
        r.assigned += missing
        assigned = self.num_pages - len(self.free)
        self.stats["peak_assigned"] = max(self.stats["peak_assigned"], assigned)
        return True

    def note_batch(self, size: int) -> None:
        self.stats["largest_batch"] = max(self.stats["largest_batch"], size)

    def prepare_step(self, rids, positions):
        """One decode step's tables: ensure each row's page in turn (stopping at the first failure,
        whose row index is returned) and return int32 tables [layers][batch][max_blocks]."""
        import numpy as np

        for i, (rid, pos) in enumerate(zip(rids, positions)):
            if not self.ensure(int(rid), int(pos)):
                return None, i
        out = np.full((self.layers, len(rids), self.max_blocks), -1, dtype=np.int32)
        for i, rid in enumerate(rids):
            out[:, i, :] = np.asarray(self.active[int(rid)].tables, dtype=np.int32)
        self.note_batch(len(rids))
        return out, -1

    def table(self, rid: int):
        return [list(row) for row in self.active[rid].tables]

    def release(self, rid: int) -> bool:
        r = self.active.pop(rid, None)
        if r is None:
            return False
        for layer in range(self.layers):
            for blk in range(self.max_blocks):
                if r.tables[layer][blk] != -1:
                    self.free.append(r.tables[layer][blk])
        self.credits_reserved -= r.credits
        return True

    def snapshot(self) -> dict:
        return dict(self.stats, free_pages=len(self.free), credits_reserved=self.credits_reserved,
                    pool_pages=self.num_pages, active=len(self.active), waiting=len(self.waiting))
