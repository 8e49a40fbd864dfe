"""The synthetic decode-step configurations and a generic builder.

Every array is produced from ``numpy.random.default_rng(seed)`` (PCG64) in a fixed draw order:
context lengths, then the physical page permutation, then the K pool, the V pool, the queries,
the new K rows and the new V rows (layer-major where there are several layers).  Values are
standard normal FP32 rounded to BF16 with round-to-nearest-even; they stand in for post-RoPE
projections, since the pages measure on no public dataset.

Pages are handed out the way the pages' host code does it: a free list of physical page ids
is consumed from its back, and a block-table entry of -1 means "not assigned"
("The prefill path: flowing the entire prompt at once", section "Distributing K/V into paged blocks").  A decode step
appends the token at absolute position ``pos`` ("6 Hours of YouTube and 85 handtyped pages of notes on LLM Inference", section "What works so far": decode
appends one new token at its absolute position), so a fresh page is taken only when
``pos % 16 == 0``; attention then covers ``L = pos + 1`` tokens.

Nothing here computes attention or writes a pool slot from a new row: that is the method, and
it lives in ``oracle/`` (CPU reference) and ``paged_kv_cache_pages_amd`` (HIP) separately.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
HEAD_DIM = 64
NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
MAX_BLOCKS = 128  # 2048-token context / 16 tokens per page

CONFIG_NAMES = ("tiny", "long", "mixed", "model16", "bw256", "bw256tp8")

_CHUNK = 1 << 24


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round FP32 values to BF16 (round-to-nearest-even) and return the 16-bit patterns.

    Input construction only.  NaN inputs become the canonical quiet NaN 0x7FC0.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))
    out = ((bits + bias) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """Standard-normal FP32 draws rounded to BF16 bit patterns, generated in chunks."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.uint16)
    for start in range(0, n, _CHUNK):
        stop = min(n, start + _CHUNK)
        out[start:stop] = f32_to_bf16_bits(rng.standard_normal(stop - start, dtype=np.float32))
    return out.reshape(shape)


@dataclass
class Workload:
    """Inputs of one decode step (append, then attend) for ``layers`` layers.

    Shapes (P pages, B sequences, Hq/Hkv heads, D head_dim, T table width):

    * ``k_pool``, ``v_pool``: uint16 [P][Hkv][16][D] BF16 bits, shared by all layers.
    * ``block_tables``: int32 [layers][B][T]; -1 marks an unassigned entry.
    * ``positions``: int32 [B], absolute position of the appended token.
    * ``context_lens``: int32 [B], tokens attended after the append (``positions + 1``).
    * ``q``: uint16 [layers][B][Hq][D]; ``k_new``, ``v_new``: uint16 [layers][B][Hkv][D].
    """

    name: str
    seed: int
    k_pool: np.ndarray
    v_pool: np.ndarray
    block_tables: np.ndarray
    positions: np.ndarray
    context_lens: np.ndarray
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def layers(self) -> int:
        return int(self.block_tables.shape[0])

    @property
    def batch(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[2])

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_pool.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.k_pool.shape[3])


def _pages(n_tokens: int) -> int:
    return (int(n_tokens) + BLOCK_SIZE - 1) // BLOCK_SIZE


def _fill_tables_lifo(perm: np.ndarray, lengths: np.ndarray, layers: int, max_blocks: int):
    """Assign pages from the back of a shuffled free list.

    The ``pos // 16`` pages that already hold the prefix come first (layer-major, then sequence
    order); then, per layer, a fresh page for every sequence whose new token opens a page.
    Returns the tables and a boolean [layers][B] mask of the fresh (step a0) assignments.
    """
    free = [int(p) for p in perm]
    batch = len(lengths)
    tables = np.full((layers, batch, max_blocks), -1, dtype=np.int32)
    fresh = np.zeros((layers, batch), dtype=bool)
    for layer in range(layers):
        for b, L in enumerate(lengths):
            for j in range(_pages(int(L) - 1)):
                tables[layer, b, j] = free.pop()
    for layer in range(layers):
        for b, L in enumerate(lengths):
            pos = int(L) - 1
            if pos % BLOCK_SIZE == 0:
                if not free:
                    raise RuntimeError("page pool exhausted")
                tables[layer, b, pos // BLOCK_SIZE] = free.pop()
                fresh[layer, b] = True
    return tables, fresh, len(free)


def _draw_rows(rng, layers, batch, num_pages, hq, hkv, d):
    k_pool = normal_bf16(rng, (num_pages, hkv, BLOCK_SIZE, d))
    v_pool = normal_bf16(rng, (num_pages, hkv, BLOCK_SIZE, d))
    q = normal_bf16(rng, (layers, batch, hq, d))
    k_new = normal_bf16(rng, (layers, batch, hkv, d))
    v_new = normal_bf16(rng, (layers, batch, hkv, d))
    return k_pool, v_pool, q, k_new, v_new


def _finish(name, seed, tables, lengths, pools_and_rows, meta):
    k_pool, v_pool, q, k_new, v_new = pools_and_rows
    lengths = np.asarray(lengths, dtype=np.int32)
    return Workload(
        name=name,
        seed=seed,
        k_pool=k_pool,
        v_pool=v_pool,
        block_tables=tables,
        positions=(lengths - 1).astype(np.int32),
        context_lens=lengths.copy(),
        q=q,
        k_new=k_new,
        v_new=v_new,
        meta=meta,
    )


def make_tiny(seed: int = 0) -> Workload:
    """One sequence, context 37 (three pages, the last one partial), pool of 8 pages."""
    rng = np.random.default_rng(seed)
    num_pages, L = 8, 37
    perm = rng.permutation(num_pages).astype(np.int32)
    tables = np.full((1, 1, MAX_BLOCKS), -1, dtype=np.int32)
    tables[0, 0, : _pages(L)] = perm[: _pages(L)]
    rows = _draw_rows(rng, 1, 1, num_pages, NUM_Q_HEADS, NUM_KV_HEADS, HEAD_DIM)
    return _finish("tiny", seed, tables, [L], rows, {"sum_context": L})


def make_long(seed: int = 1) -> Workload:
    """One sequence at the 2048-token cap over a 512-page pool in random physical order."""
    rng = np.random.default_rng(seed)
    num_pages, L = 512, 2048
    perm = rng.permutation(num_pages).astype(np.int32)
    tables = perm[:MAX_BLOCKS].reshape(1, 1, MAX_BLOCKS).copy()
    rows = _draw_rows(rng, 1, 1, num_pages, NUM_Q_HEADS, NUM_KV_HEADS, HEAD_DIM)
    return _finish("long", seed, tables, [L], rows, {"sum_context": L})


def make_mixed(seed: int = 2) -> Workload:
    """Sixteen sequences with context lengths uniform in [1, 2048] over a 2048-page pool."""
    rng = np.random.default_rng(seed)
    num_pages, batch = 2048, 16
    lengths = rng.integers(1, 2049, size=batch).astype(np.int32)
    perm = rng.permutation(num_pages).astype(np.int32)
    tables, fresh, free_left = _fill_tables_lifo(perm, lengths, 1, MAX_BLOCKS)
    rows = _draw_rows(rng, 1, batch, num_pages, NUM_Q_HEADS, NUM_KV_HEADS, HEAD_DIM)
    meta = {"sum_context": int(lengths.sum()), "fresh_pages": int(fresh.sum()), "free_pages_left": free_left}
    return _finish("mixed", seed, tables, lengths, rows, meta)


def make_model16(seed: int = 3, requests: int = 64, pool_pages: int = 4096, layers: int = 16) -> Workload:
    """Sixteen layers sharing a 128 MiB pool; requests admitted first-in-first-out.

    Sixty-four context lengths are drawn geometric with mean 256 and capped at 2048.  Requests
    are admitted in order while the pages they need over all layers (``layers * ceil(L/16)``)
    still fit in the pool; the first request that does not fit stops admission, mirroring the
    FIFO wait without skipping described on "6 Hours of YouTube and 85 handtyped pages of notes on LLM Inference", section "Current scope".
    """
    rng = np.random.default_rng(seed)
    drawn = np.minimum(rng.geometric(1.0 / 256.0, size=requests), 2048).astype(np.int32)
    admitted, used = [], 0
    for L in drawn:
        need = layers * _pages(int(L))
        if used + need > pool_pages:
            break
        admitted.append(int(L))
        used += need
    lengths = np.asarray(admitted, dtype=np.int32)
    perm = rng.permutation(pool_pages).astype(np.int32)
    tables, fresh, free_left = _fill_tables_lifo(perm, lengths, layers, MAX_BLOCKS)
    rows = _draw_rows(rng, layers, len(lengths), pool_pages, NUM_Q_HEADS, NUM_KV_HEADS, HEAD_DIM)
    meta = {
        "requests_drawn": requests,
        "admitted": int(len(lengths)),
        "pages_budgeted": int(used),
        "sum_context": int(lengths.sum()),
        "fresh_pages": int(fresh.sum()),
        "free_pages_left": free_left,
    }
    return _finish("model16", seed, tables, lengths, rows, meta)


def make_bw256(seed: int = 4) -> Workload:
    """256 sequences at context 2048 over exactly 32768 pages (1 GiB of BF16 K+V)."""
    rng = np.random.default_rng(seed)
    batch, L = 256, 2048
    num_pages = batch * MAX_BLOCKS
    perm = rng.permutation(num_pages).astype(np.int32)
    tables = perm.reshape(1, batch, MAX_BLOCKS).copy()
    rows = _draw_rows(rng, 1, batch, num_pages, NUM_Q_HEADS, NUM_KV_HEADS, HEAD_DIM)
    return _finish("bw256", seed, tables, np.full(batch, L, dtype=np.int32), rows, {"sum_context": batch * L})


def make_bw256_tp8(seed: int = 6) -> Workload:
    """One GPU's share of bw256 under 8-way tensor parallelism over KV heads: 256 sequences at
    context 2048, 1 KV head and its 4 query heads, 32768 pages of one head (128 MiB of BF16 K+V)."""
    rng = np.random.default_rng(seed)
    batch, L, hkv = 256, 2048, 1
    num_pages = batch * MAX_BLOCKS
    perm = rng.permutation(num_pages).astype(np.int32)
    tables = perm.reshape(1, batch, MAX_BLOCKS).copy()
    rows = _draw_rows(rng, 1, batch, num_pages, hkv * (NUM_Q_HEADS // NUM_KV_HEADS), hkv, HEAD_DIM)
    return _finish("bw256tp8", seed, tables, np.full(batch, L, dtype=np.int32), rows, {"sum_context": batch * L})


_MAKERS = {
    "tiny": make_tiny,
    "long": make_long,
    "mixed": make_mixed,
    "model16": make_model16,
    "bw256": make_bw256,
    "bw256tp8": make_bw256_tp8,
}


def make_config(name: str) -> Workload:
    """Build one of the named configurations with its own seed (tiny=0 ... bw256=4, bw256tp8=6)."""
    if name not in _MAKERS:
        raise KeyError(f"unknown config {name!r}; expected one of {CONFIG_NAMES}")
    return _MAKERS[name]()


def make_custom(
    seed: int,
    lengths,
    num_pages: int | None = None,
    layers: int = 1,
    max_blocks: int = MAX_BLOCKS,
    num_kv_heads: int = NUM_KV_HEADS,
    group: int = NUM_Q_HEADS // NUM_KV_HEADS,
    head_dim: int = HEAD_DIM,
) -> Workload:
    """A decode step with the given context lengths (after the append) and a shuffled pool.

    ``num_pages`` defaults to exactly the pages the step needs plus eight spares.  Lengths of 0
    are allowed (empty sequences get no pages and position -1).
    """
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int32).reshape(-1)
    need = layers * sum(_pages(int(L)) for L in lengths)
    if num_pages is None:
        num_pages = need + 8
    if need > num_pages:
        raise ValueError(f"{need} pages needed but the pool has {num_pages}")
    if lengths.size and int(lengths.max()) > max_blocks * BLOCK_SIZE:
        raise ValueError("a context length exceeds the block-table width")
    perm = rng.permutation(num_pages).astype(np.int32)
    nonempty = lengths > 0
    tables = np.full((layers, len(lengths), max_blocks), -1, dtype=np.int32)
    if nonempty.any():
        sub, _, _ = _fill_tables_lifo(perm, lengths[nonempty], layers, max_blocks)
        tables[:, nonempty, :] = sub
    rows = _draw_rows(rng, layers, len(lengths), num_pages, num_kv_heads * group, num_kv_heads, head_dim)
    return _finish("custom", seed, tables, lengths, rows, {"sum_context": int(lengths.sum())})


def llama3_rope_tables(max_pos: int, head_dim: int = HEAD_DIM, theta: float = 500000.0, factor: float = 32.0,
                       low_freq_factor: float = 1.0, high_freq_factor: float = 4.0, original_context: int = 8192):
    """FP32 cos/sin tables [max_pos][head_dim] for the rotary embedding, built the way Llama-3
    checkpoints specify their frequencies (base theta plus the piecewise long-context scaling).

    Input construction only.  The pages do not print how their engine fills these tables (only
    that it fills them once at start-up, and that the two slots of each rotated pair hold the same
    value, "The prefill path: flowing the entire prompt at once", section "RoPE: a rotation that
    references a table"), so the tables are caller inputs of the rotation; this builder gives
    realistic values.  Entry [pos][2i] and [pos][2i+1] both hold the angle of pair i.
    """
    half = head_dim // 2
    inv = 1.0 / theta ** (np.arange(half, dtype=np.float64) * 2.0 / head_dim)
    wavelen = 2.0 * np.pi / inv
    low_wl = original_context / low_freq_factor
    high_wl = original_context / high_freq_factor
    smooth = (original_context / wavelen - low_freq_factor) / (high_freq_factor - low_freq_factor)
    scaled = np.where(wavelen > low_wl, inv / factor, inv)
    mid = (wavelen <= low_wl) & (wavelen >= high_wl)
    scaled = np.where(mid, (1.0 - smooth) * inv / factor + smooth * inv, scaled)
    angles = np.arange(max_pos, dtype=np.float64)[:, None] * scaled[None, :]  # [pos][half]
    full = np.repeat(angles, 2, axis=1)  # slots 2i and 2i+1 share pair i's angle
    return np.cos(full).astype(np.float32), np.sin(full).astype(np.float32)
