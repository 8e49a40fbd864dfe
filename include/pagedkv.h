/*
 * pagedkv.h -- C ABI of libpagedkv: the decode-step hot path of a paged BF16 KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * Two calls carry the method: pkv_kv_append writes each sequence's new K/V row into its page,
 * and pkv_paged_decode_attention streams each sequence's pages with grouped-query attention and
 * an FP32 online softmax.  pkv_rope_kv_append and pkv_decode_step fuse the rotary embedding
 * into the append and the append into the attention launch.  pkv_prefill_kv_append and
 * pkv_paged_prefill_attention are the prompt-side pair (many rows per sequence, causal).  The
 * pkv_alloc_* calls are the host page allocator that fills the block tables.  The rest are
 * helpers (planning, workspace size, host-side validation, status strings).
 *
 * Conventions for every call:
 *   - Pointers documented as "device" must point to GPU memory of the current HIP device;
 *     "host" pointers to ordinary CPU memory.  The caller owns every buffer; the library
 *     allocates no device memory, keeps no per-call state and is reentrant.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is only
 *     enqueued; nothing synchronises with the host unless debug validation is on (below).
 *     Ordering between calls comes from stream order.
 *   - BF16 values travel as their 16-bit patterns (uint16_t storage).  Every device buffer
 *     must be 16-byte aligned (the kernels move 16-byte vectors).
 *   - Return value: PKV_OK, or the first error found by the synchronous host checks.  No
 *     kernel is launched when a check fails.  Kernels never read or write out of bounds: a
 *     block-table entry outside [0, num_pages), a position outside the table, or a context
 *     length outside [0, 16 * max_blocks_per_seq] is never dereferenced; append skips that
 *     row and attention writes zeros for that sequence.
 *   - Environment PKV_DEBUG_VALIDATE=1 makes both calls copy the block tables, positions and
 *     context lengths to the host (synchronously) and return PKV_ERR_VALIDATION instead of
 *     launching when any of them is out of range, when a table entry needed by the step is -1,
 *     or (append) when two sequences target the same (page, slot).
 *
 * Page pool layout ("[page][kv_head][token][dim]"): K and V live in two separate buffers, each
 * bf16[num_pages][num_kv_heads][block_size][head_dim], so the 16 tokens of one KV head in one
 * page are one contiguous 2 KiB run (block_size 16, head_dim 64).
 *
 * Supported geometry (anything else returns PKV_ERR_UNSUPPORTED): block_size 16, head_dim 64,
 * num_q_heads == 4 * num_kv_heads.  These are the Llama-3.2-1B decode constants of the pages:
 * 16-token pages ("Code-Series on Jaehun's Blog", entry 6 "Splitting the KV cache into 16-token
 * blocks"), 32 query heads over 8 KV heads with consecutive groups of four and head_dim 64
 * ("The prefill path: flowing the entire prompt at once", section "Per-head attention scores and GQA").
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 1

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required pointer is NULL                                    */
  PKV_ERR_SHAPE = 2,       /* a size is negative/zero where it must be positive, or scale  */
                           /* is not a positive finite number                               */
  PKV_ERR_UNSUPPORTED = 3, /* geometry outside the compiled kernels (see above)             */
  PKV_ERR_WORKSPACE = 4,   /* the chosen split needs more workspace than was passed         */
  PKV_ERR_VALIDATION = 5,  /* debug validation rejected the data (PKV_DEBUG_VALIDATE=1)     */
  PKV_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed                    */
  PKV_ERR_ALIGNMENT = 7,   /* a device buffer is not 16-byte aligned                        */
  PKV_ERR_REJECTED = 8,    /* allocator: the request can never be served (see pkv_alloc_*)  */
  PKV_ERR_STATE = 9,       /* allocator: unknown request id, or an id already queued/active */
  PKV_ERR_EXHAUSTED = 10,  /* allocator: the page would exceed the request's credits        */
  PKV_ERR_SCRATCH = 11     /* pkv_decode_step_static: the split exceeds the static scratch  */
} pkv_status;

typedef enum {
  PKV_OUT_BF16 = 0, /* output stored as BF16, rounded to nearest even from the FP32 result */
  PKV_OUT_F32 = 1   /* output stored as FP32 (the pre-rounding value, used for parity)     */
} pkv_out_dtype;

/* The shared page pool.  k_pool / v_pool: device, bf16[num_pages][num_kv_heads][block_size]
 * [head_dim] each. */
typedef struct {
  void *k_pool;
  void *v_pool;
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
} pkv_pool;

/* Human-readable name of a status code (static string, never NULL). */
const char *pkv_status_string(pkv_status status);

/* PKV_ABI_VERSION of the built library. */
int32_t pkv_abi_version(void);

/*
 * kv_append(pool, block_tables, positions, k_new, v_new)
 *
 * Decode-side KV write: for every sequence b and KV head g, copy k_new[b][g][:] into
 * K[page][g][slot][:] and v_new[b][g][:] into V[page][g][slot][:], where
 * page = block_tables[b * max_blocks_per_seq + positions[b] / 16] and slot = positions[b] % 16.
 * The pages describe this step as decode appending one new token at its absolute (RoPE)
 * position into the shared BF16 page pool ("6 Hours of YouTube and 85 handtyped pages of notes on LLM Inference", section "What works so far"), with the
 * page found through the per-sequence block table ("The prefill path: flowing the entire prompt at once", section
 * "Distributing K/V into paged blocks").  The copy is bit-exact.
 *
 *   pool                host struct; its k_pool / v_pool are device buffers (modified)
 *   block_tables        device int32[batch][max_blocks_per_seq]; the entry for block
 *                       positions[b] / 16 must already hold a page (the host allocator
 *                       assigns a fresh page when positions[b] % 16 == 0); other entries unused
 *   positions           device int32[batch], absolute position of the new token
 *   k_new, v_new        device bf16[batch][num_kv_heads][head_dim]
 *   batch               >= 0 (0 is a no-op)
 * Preconditions: targets are distinct (page, slot) pairs; otherwise which row lands is
 * unspecified.  Rows with an out-of-range position or page id are skipped.
 */
pkv_status pkv_kv_append(const pkv_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                         const int32_t *positions, const void *k_new, const void *v_new, int32_t batch,
                         void *stream);

/*
 * rope_kv_append: the decode step's rotary embedding fused into kv_append.
 *
 * For every sequence b at absolute position pos = positions[b]: rotate each query head of
 * q[b] and the new key row k_new[b][g] ("The prefill path: flowing the entire prompt at once",
 * section "RoPE: a rotation that references a table": inside each 64-wide head, element i is
 * paired with element i + 32 and rotated by the angle of slot 2i of the position's table row:
 *   y_i = x_i * c - x_{i+32} * s,   y_{i+32} = x_i * s + x_{i+32} * c,
 * with c = cos_table[pos][2i], s = sin_table[pos][2i]; every product and the sum/difference are
 * separate FP32 operations, the result is rounded to BF16 to nearest even).  The rotated query
 * goes to q_out; the rotated key and the unrotated v_new[b][g] are written into the pool exactly
 * as pkv_kv_append writes them.  Values are not rotated.
 *
 *   q, q_out            device bf16[batch][num_q_heads][64]; q_out may equal q (in place)
 *   k_new, v_new        device bf16[batch][num_kv_heads][64]; not modified
 *   cos_table, sin_table device f32[table_rows][64], built by the caller (e.g. with the model's
 *                       RoPE frequencies); slots 2i and 2i+1 conventionally hold the same value
 * A sequence whose position is outside [0, table_rows), outside the block table or whose page
 * entry is out of range is skipped entirely: its q_out rows and its pool slots are not written.
 * With PKV_DEBUG_VALIDATE=1 such a batch is rejected with PKV_ERR_VALIDATION instead.
 */
pkv_status pkv_rope_kv_append(const pkv_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                              const int32_t *positions, const void *q, void *q_out, int32_t num_q_heads,
                              const void *k_new, const void *v_new, const float *cos_table,
                              const float *sin_table, int32_t table_rows, int32_t batch, void *stream);

/*
 * paged_decode_attention(q, k_pool, v_pool, block_tables, context_lens, out)
 *
 * For every sequence b, query head h (KV head g = h / 4) and dim d:
 *   s_t = scale * sum_d q[b][h][d] * K[page(t)][g][t % 16][d]          for t < L = context_lens[b]
 *   out[b][h][:] = sum_t softmax(s)_t * V[page(t)][g][t % 16][:]
 * with page(t) = block_tables[b * max_blocks_per_seq + t / 16].  The pages' decode attention
 * streams each sequence's cached pages per query head and accumulates weighted values with an
 * FP32 online softmax, gathering no contiguous prefix and storing no scores ("6 Hours of YouTube and 85 handtyped pages of notes on LLM Inference",
 * "What works so far"); the online-softmax merge of partial (max, sum) pairs is the rule of
 * "The prefill path: flowing the entire prompt at once", section "causalMask and online softmax".  Inputs are BF16,
 * all arithmetic is FP32, the output is FP32 or BF16 (round to nearest even).  A NaN in a K row
 * inside a sequence's context makes the 4 output rows of that KV group NaN, a NaN in a V row
 * the dims it holds, split or not (as the definition gives); slot contents outside the context
 * are never read into the result.
 *
 *   q                 device bf16[batch][num_q_heads][head_dim]
 *   k_pool, v_pool    device bf16[num_pages][num_kv_heads][block_size][head_dim]
 *   block_tables      device int32[batch][max_blocks_per_seq]; the whole buffer must be
 *                     readable (a workgroup may read entries past its sequence's context
 *                     before it knows the length); entries past the context are ignored
 *   context_lens      device int32[batch]; tokens attended, including the one just appended;
 *                     0 gives an all-zero output row
 *   out               device, bf16 or f32 [batch][num_q_heads][head_dim] per out_dtype
 *   scale             positive finite score scale (1/sqrt(head_dim) = 0.125 for Llama)
 *   batch             0 .. 65535 sequences (PKV_ERR_SHAPE above); a partition size giving more
 *                     than 65535 partitions is PKV_ERR_SHAPE as well
 *   partition_pages   pages per context partition.  <= 0: choose automatically with
 *                     pkv_plan_partition_pages for the current device.  When a sequence's
 *                     pages are cut into several partitions, each partition publishes a
 *                     (max, sum, partial output) triple per query head in `workspace` and the
 *                     partition that finishes last merges them, inside the same launch.  Values
 *                     above 256 are treated as 256 (one workgroup covers at most 256 pages);
 *                     >= max_blocks_per_seq (when that is <= 256) never splits.
 *   workspace         device scratch of at least pkv_decode_workspace_bytes(...) bytes for the
 *                     resolved partition size (may be NULL when that is 0).  It must be
 *                     all-zero before its first use (e.g. hipMemset once at allocation); every
 *                     call leaves it all-zero again, so one workspace, sized for the largest
 *                     shape, serves any sequence of calls of any shape on one stream.  Calls
 *                     that run at the same time (other streams) need workspaces of their own.
 *                     Debug validation rejects a split call whose counters are not zero.
 */
pkv_status pkv_paged_decode_attention(const void *q, const void *k_pool, const void *v_pool, int32_t num_pages,
                                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                                      const int32_t *context_lens, void *out, pkv_out_dtype out_dtype,
                                      int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, float scale, int32_t partition_pages, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * decode_step: kv_append followed by paged_decode_attention over context = positions[b] + 1, in
 * one launch.  The result (pool contents and out) is exactly that of pkv_kv_append(pool,
 * block_tables, positions, k_new, v_new) then pkv_paged_decode_attention(..., context_lens =
 * positions + 1, ...) with the same partition size.  The workgroup that reads a sequence's last
 * page writes the new rows into the pool and uses them from registers, so this also holds when
 * the old slot content is stale or NaN.
 *
 *   pool, block_tables, positions, k_new, v_new   as for pkv_kv_append
 *   q, out, out_dtype, scale, partition_pages, workspace   as for pkv_paged_decode_attention
 *   num_q_heads                                   4 * pool->num_kv_heads
 * Out-of-range data behaves exactly as with the two separate calls: a position outside
 * [0, 16 * max_blocks_per_seq), or an append page entry outside [0, num_pages), appends nothing;
 * any needed table entry outside [0, num_pages) zeroes that sequence's output rows (the row is
 * still appended when its own page entry is valid).
 * Precondition (as for the separate calls): no other sequence of the batch references the page
 * a sequence appends to.
 */
pkv_status pkv_decode_step(const pkv_pool *pool, const void *q, const int32_t *block_tables, int32_t max_blocks_per_seq,
                           const int32_t *positions, const void *k_new, const void *v_new, void *out,
                           pkv_out_dtype out_dtype, int32_t batch, int32_t num_q_heads, float scale,
                           int32_t partition_pages, void *workspace, size_t workspace_bytes, void *stream);

/*
 * decode_step_static: pkv_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, hosts that forbid hipMalloc).  Same arguments, results
 * and out-of-range behaviour as pkv_decode_step, without the workspace: a split uses scratch that
 * the library holds in a static device array of PKV_STATIC_SCRATCH_BYTES per GPU (kept until the
 * process ends, its address resolved once per device on the first call there).  Allocates
 * nothing: no hipMalloc/hipFree and no host buffers (so PKV_DEBUG_VALIDATE does not apply here).
 *   Returns PKV_ERR_SCRATCH when pkv_decode_workspace_bytes(batch, num_q_heads,
 *   max_blocks_per_seq, resolved partition size) exceeds PKV_STATIC_SCRATCH_BYTES (nothing is
 *   launched); an unsplit call needs no scratch.
 *   All calls on one GPU share its array: calls that can run at the same time on one GPU (other
 *   streams, other threads) race and must not overlap.  The array starts zero-filled and every
 *   call leaves it zero-filled, which is what a split needs.
 */
#define PKV_STATIC_SCRATCH_BYTES (4u << 20)
pkv_status pkv_decode_step_static(const pkv_pool *pool, const void *q, const int32_t *block_tables,
                                  int32_t max_blocks_per_seq, const int32_t *positions, const void *k_new,
                                  const void *v_new, void *out, pkv_out_dtype out_dtype, int32_t batch,
                                  int32_t num_q_heads, float scale, int32_t partition_pages, void *stream);

/*
 * Pages per partition chosen when partition_pages <= 0.  Pure function (no GPU needed).  With L
 * the pages of the longest context (here the table width): no split when the batch *
 * num_kv_heads workgroups number at least 3/4 of num_cus, or when L <= 24; otherwise the
 * smallest multiple of 4 pages, at least 8, that gives about one workgroup per compute unit over
 * L, and no split if that is >= L; never more than 256.  Returns min(max_blocks_per_seq, 256)
 * when no split is planned; -1 on bad arguments.
 */
int32_t pkv_plan_partition_pages(int32_t batch, int32_t num_kv_heads, int32_t max_blocks_per_seq, int32_t num_cus);

/*
 * The same plan for a batch whose longest context (tokens attended, the new one included) is
 * max_context_len, a bound the caller's scheduler knows on the host: L is then that context's
 * pages instead of the table width, so short batches run unsplit (no partials to publish and
 * merge) and long ones split by their real length.  max_context_len < 0 means unknown (the plain plan); -1 on bad
 * arguments.  Only the launch shape depends on it: a context longer than the bound is still
 * attended correctly, through partitions of the returned size.
 */
int32_t pkv_plan_partition_pages_for_context(int32_t batch, int32_t num_kv_heads, int32_t max_blocks_per_seq,
                                             int32_t max_context_len, int32_t num_cus);

/* Workspace bytes needed for the given positive partition size (after the same 256-page cap
 * the attention call applies); 0 without a split.  Returns 0 on bad arguments.  Layout (internal):
 * the partial outputs and (max, sum) pairs of every (sequence, query head, partition), then one
 * counter per (sequence, KV head) 128 bytes apart. */
size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                  int32_t partition_pages);

/* Compute units of the current HIP device, or -1 when no device is available. */
int32_t pkv_device_cu_count(void);

/*
 * Host-side data validation (plain C++, no GPU needed; also what PKV_DEBUG_VALIDATE runs).
 * All pointers are host pointers.  On failure *bad_row (if not NULL) receives the offending
 * batch row; on success it receives -1.
 *
 * Append: every position is in [0, 16 * max_blocks_per_seq), the entry for block
 * positions[b] / 16 is in [0, num_pages), and no two rows target the same (page, slot).
 * Decode: every context length is in [0, 16 * max_blocks_per_seq] and the first
 * ceil(L / 16) entries of the row are in [0, num_pages).
 */
pkv_status pkv_validate_append_host(const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *positions,
                                    int32_t batch, int32_t num_pages, int32_t *bad_row);
pkv_status pkv_validate_decode_host(const int32_t *block_tables, int32_t max_blocks_per_seq,
                                    const int32_t *context_lens, int32_t batch, int32_t num_pages, int32_t *bad_row);

/*
 * Paged prefill ("The prefill path: flowing the entire prompt at once", sections "Distributing
 * K/V into paged blocks", "Per-head attention scores and GQA", "causalMask and online softmax").
 *
 * A prefill step covers `batch` sequences packed into num_tokens rows: sequence b owns rows
 * cu_seqlens[b] .. cu_seqlens[b+1]-1 (device int32[batch+1]) of q, k_new, v_new and out, and its
 * prompt token i sits at absolute position start_pos[b] + i (device int32[batch]; 0 = a whole
 * prompt, > 0 = a prompt chunk behind that many tokens already in the cache).  max_prompt_len is a
 * host-side bound on every cu_seqlens[b+1] - cu_seqlens[b]; it sizes the grids.
 *
 * A sequence whose rows are not inside [0, num_tokens), whose length is negative or above
 * max_prompt_len, is left untouched by both calls.
 *
 * pkv_prefill_kv_append writes row i's K and V (device bf16[num_tokens][num_kv_heads][64]) into
 * slot (start + i) % 16 of page table[(start + i) / 16]; a row whose position is outside the table
 * or whose entry is outside [0, num_pages) is skipped.  Rows of one call must target distinct
 * (page, slot) pairs.
 *
 * pkv_paged_prefill_attention computes, for every row and query head h, the causal attention of
 * q (device bf16[num_tokens][num_q_heads][64]) over positions 0 .. start + i of the sequence read
 * through its block table (KV head h / 4, scale, FP32 online softmax), written to out (device,
 * FP32 or BF16 [num_tokens][num_q_heads][64]).  Both products run on the matrix cores with FP32
 * accumulation: q.k on the BF16 inputs (exact products); p.v with V converted to FP16 (exact for
 * every BF16 value up to 65280) and each weight, scaled by 2^7 (it cancels in the ratio), rounded
 * to FP16 (11 significant bits, nearest even), the denominator summing the same rounded weights.
 * The weight of a key stays a normal FP16 number down to 2^-21 of the row's anchor weight; below
 * that it keeps an absolute error of at most 2^-25 (times 2^-7 after the scale cancels), so an
 * output row's error is about 2^-11 of the weighted |V| plus, at worst, n * 2^-32 * max|V| over n
 * keys.  Precision limit: with |V| of order 1e3 on rows of thousands of keys whose output dims
 * cancel to near 0, that can exceed an absolute error of 2e-3 (still below the BF16 output's own
 * rounding).  A query tile whose keys hold a finite V magnitude above 65504 is recomputed with
 * BF16 V and each weight as two BF16 terms (about 16 significant bits, not exact).  The prompt's own rows must already be in the pool (call the
 * append first, on the same stream).  When start < 0, start + length > 16 * max_blocks_per_seq or
 * any of the sequence's first ceil((start + length) / 16) entries is outside [0, num_pages), all
 * its rows get zeros.  Slots past the last prompt position are never read.
 * Precondition: the prompt's own K and V rows are finite.  The kernel multiplies a causally masked
 * (later) key's V row by weight 0, so an infinity or NaN in prompt row i reaches the earlier rows of
 * the same query tile (16 or 32 rows), which the definition would leave finite.  Values in the
 * cached prefix (positions < start) are visible to every row and carry no such caveat.
 *
 * Both calls: NULL, shape (negative sizes, num_tokens < 0, max_prompt_len < 0, bad scale or
 * dtype), unsupported geometry and alignment are reported before launching; nothing is launched
 * when batch, num_tokens or max_prompt_len is 0.  PKV_DEBUG_VALIDATE=1 also runs
 * pkv_validate_prefill_host on copies of the tables, cu_seqlens and start_pos, and checks the
 * finiteness precondition with pkv_validate_finite_rows_host: the append on copies of k_new and
 * v_new, the attention on copies of the prompt rows' pool slots.
 */
pkv_status pkv_prefill_kv_append(const pkv_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                 const int32_t *cu_seqlens, const int32_t *start_pos, const void *k_new,
                                 const void *v_new, int32_t batch, int32_t num_tokens, int32_t max_prompt_len,
                                 void *stream);
pkv_status pkv_paged_prefill_attention(const pkv_pool *pool, const void *q, const int32_t *block_tables,
                                       int32_t max_blocks_per_seq, const int32_t *cu_seqlens,
                                       const int32_t *start_pos, void *out, pkv_out_dtype out_dtype, int32_t batch,
                                       int32_t num_tokens, int32_t max_prompt_len, int32_t num_q_heads, float scale,
                                       void *stream);

/* Host-side prefill validation (host pointers): cu_seqlens non-decreasing from >= 0 up to
 * <= num_tokens, every length <= max_prompt_len, start_pos >= 0, start + length within the table,
 * the first ceil((start + length) / 16) entries in [0, num_pages), and all appended (page, slot)
 * targets distinct.  *bad_row receives the offending sequence (or -1). */
pkv_status pkv_validate_prefill_host(const int32_t *block_tables, int32_t max_blocks_per_seq,
                                     const int32_t *cu_seqlens, const int32_t *start_pos, int32_t batch,
                                     int32_t num_tokens, int32_t max_prompt_len, int32_t num_pages,
                                     int32_t *bad_row);

/* Host-side check (host pointer) that every value of num_rows packed BF16 rows of row_elems
 * values each is finite (exponent field not all ones).  PKV_ERR_VALIDATION with *bad_row = the
 * first row holding an infinity or NaN; PKV_OK and *bad_row = -1 otherwise; PKV_ERR_SHAPE for
 * num_rows < 0 or row_elems <= 0. */
pkv_status pkv_validate_finite_rows_host(const uint16_t *rows, int32_t num_rows, int32_t row_elems, int32_t *bad_row);

/*
 * Host page allocator with admission credits (plain C++, no GPU; step a0 of a decode loop:
 * it produces the block tables the calls above read).
 *
 * Rules ("6 Hours of YouTube and 85 handtyped pages of notes on LLM Inference", section
 * "Current scope"; "The prefill path: flowing the entire prompt at once", section
 * "Distributing K/V into paged blocks"):
 *   - A request of P prompt tokens asking for N new tokens may generate A = min(N, C - P)
 *     tokens (C = 16 * max_blocks_per_seq, the context limit).  Its last generated token is
 *     never appended, so the longest prefix it stores is max(P, P + A - 1) tokens, and
 *     admission reserves that many 16-token pages in every layer as credits.
 *   - Requests are admitted first-in-first-out while their credits fit beside those of the
 *     active requests; the first one that does not fit blocks the queue (no skipping, no
 *     preemption).  Static batching admits only when no request is active.
 *   - Physical pages are taken lazily, from the back of the free list, the first time a
 *     position of a block is needed; a table entry of -1 is "unassigned".  A request never
 *     holds more pages than its credits, so an admitted request always finds its pages.
 *   - Release returns the request's pages to the back of the free list (layer by layer, each
 *     in block order) and its credits to the pool.
 *
 * The allocator is a host object owned by the caller (create/destroy); it is not thread-safe
 * (one caller thread at a time).  All pointers are host pointers.
 */
typedef struct pkv_allocator pkv_allocator;

typedef struct {
  int64_t pool_pages;       /* pages in the pool                                          */
  int64_t free_pages;       /* pages on the free list now                                 */
  int64_t credits_reserved; /* credits held by active requests                            */
  int64_t active;           /* admitted, not yet released                                 */
  int64_t waiting;          /* queued, not yet admitted                                   */
  int64_t peak_active;      /* most requests active at once (checked after each admit)    */
  int64_t peak_assigned;    /* most pages assigned at once                                */
  int64_t largest_batch;    /* largest batch passed to pkv_alloc_prepare_step             */
  int64_t admission_waits;  /* admission passes that stopped at a request that did not fit */
  int64_t rejected;         /* submissions refused with PKV_ERR_REJECTED                  */
} pkv_alloc_stats;

/* Create an allocator over num_pages pages shared by `layers` layers, each request's table
 * holding max_blocks_per_seq entries per layer.  free_order (NULL = 0, 1, ..., num_pages - 1)
 * is the initial free list, a permutation of [0, num_pages); pages are taken from its end.
 * PKV_ERR_SHAPE for non-positive sizes or a free_order that is not a permutation. */
pkv_status pkv_alloc_create(int32_t num_pages, int32_t layers, int32_t max_blocks_per_seq, const int32_t *free_order,
                            int32_t static_batching, pkv_allocator **out);
void pkv_alloc_destroy(pkv_allocator *alloc);

/* Queue a request.  PKV_ERR_REJECTED (counted in `rejected`) when prompt_tokens is outside
 * [1, C], max_new_tokens < 0, or its credits exceed the whole pool; PKV_ERR_STATE when the id
 * is already queued or active. */
pkv_status pkv_alloc_submit(pkv_allocator *alloc, int64_t request_id, int32_t prompt_tokens, int32_t max_new_tokens);

/* One admission pass: admit queued requests in order while their credits fit (at most
 * `capacity` of them), writing their ids to admitted[0 .. *count). */
pkv_status pkv_alloc_admit(pkv_allocator *alloc, int64_t *admitted, int32_t capacity, int32_t *count);

/* Make the page holding token `pos` present in every layer of an active request.
 * PKV_ERR_STATE for an unknown id, PKV_ERR_SHAPE for pos outside [0, C), PKV_ERR_EXHAUSTED
 * when it would exceed the request's credits (nothing is assigned then). */
pkv_status pkv_alloc_ensure(pkv_allocator *alloc, int64_t request_id, int32_t pos);

/* Decode-step tables: for b = 0 .. batch-1 in order, pkv_alloc_ensure(ids[b], positions[b]);
 * then write the block tables of all rows to block_tables, int32[layers][batch][max_blocks],
 * the layout pkv_kv_append / pkv_paged_decode_attention read per layer.  On the first failure
 * *bad_row gets its row, pages ensured for earlier rows stay assigned and nothing is written;
 * on success *bad_row = -1 and `largest_batch` is updated. */
pkv_status pkv_alloc_prepare_step(pkv_allocator *alloc, const int64_t *request_ids, const int32_t *positions,
                                  int32_t batch, int32_t *block_tables, int32_t *bad_row);

/* Copy an active request's table, int32[layers][max_blocks], to dst. */
pkv_status pkv_alloc_table(const pkv_allocator *alloc, int64_t request_id, int32_t *dst);

/* Finish a request: return its pages and credits.  PKV_ERR_STATE for an unknown id. */
pkv_status pkv_alloc_release(pkv_allocator *alloc, int64_t request_id);

pkv_status pkv_alloc_get_stats(const pkv_allocator *alloc, pkv_alloc_stats *out);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
