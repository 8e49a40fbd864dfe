// C ABI of libpagedkv: synchronous host checks, optional debug validation, kernel dispatch.
// The two method calls follow the problem statement of "6 Hours of YouTube and 85 handtyped pages of notes on LLM Inference", section "What works so far":
// decode appends each new token at its absolute position into a shared BF16 page pool through a
// per-sequence block table, and decode attention streams each sequence's pages with an FP32
// online softmax).  Argument meaning, layout and error behaviour are documented in pagedkv.h.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "pagedkv.h"
#include "pkv_internal.h"

namespace {

// Read on every call so that a process can switch validation on and off.
bool debug_validate_enabled() {
  const char *v = getenv("PKV_DEBUG_VALIDATE");
  return v != nullptr && v[0] != '\0' && strcmp(v, "0") != 0;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pkv_status copy_to_host(std::vector<int32_t> &dst, const int32_t *src, size_t n, hipStream_t stream) {
  dst.resize(n);
  if (n == 0) return PKV_OK;
  if (hipMemcpyAsync(dst.data(), src, n * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return PKV_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return PKV_ERR_HIP;
  return PKV_OK;
}

constexpr int kMaxDevices = 64;
constexpr int32_t kMaxGridDim = 65535;  // decode grids are (KV head, sequence, partition)
std::atomic<int32_t> g_cu_count[kMaxDevices];

}  // namespace

extern "C" const char *pkv_status_string(pkv_status status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "invalid size or scale argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported geometry (needs block_size 16, head_dim 64, 4 query heads per KV head)";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small for the context split";
    case PKV_ERR_VALIDATION: return "debug validation rejected the block table, positions or context lengths";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_ALIGNMENT: return "a device buffer is not 16-byte aligned";
    case PKV_ERR_REJECTED: return "request rejected: invalid lengths, or its page credits exceed the whole pool";
    case PKV_ERR_STATE: return "unknown request id, or the id is already queued or active";
    case PKV_ERR_EXHAUSTED: return "the page would exceed the request's admission credits";
    case PKV_ERR_SCRATCH: return "the split needs more than the library's static scratch (PKV_STATIC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

extern "C" int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

extern "C" int32_t pkv_device_cu_count(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int32_t cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return -1;
  if (dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

namespace {
// The plan for a batch whose longest context spans `longest` pages (<= the table width).
// Fitted to the fused step replayed from a HIP graph, 16 layers per step, over 27 batches (1-64
// sequences: uniform 256/384/512/1024/2048-token contexts, geometric mean-256 and uniform random
// lengths), every size from 4 to 128 pages: on average this rule lands within 2% of the fastest
// size.  A context of up to 24 pages runs fastest unsplit (the in-launch merge costs more than the
// shorter page loop saves); above that, about one workgroup per compute unit over the longest
// context is best, down to 8-page partitions (two pages per wavefront); and from 3/4 of a
// workgroup per compute unit the unsplit launch is fastest.
constexpr int64_t kMinSplitPages = 24;
constexpr int64_t kMinPartitionPages = 8;
int32_t plan_pages(int64_t pairs, int32_t max_blocks_per_seq, int64_t longest, int32_t num_cus) {
  const int32_t cap = max_blocks_per_seq < pkv::kMaxPartitionPages ? max_blocks_per_seq : pkv::kMaxPartitionPages;
  if (pairs == 0) return cap;
  if (4 * pairs >= 3LL * num_cus) return cap;
  if (longest <= kMinSplitPages) return cap;
  // About one workgroup per compute unit over the longest context, in equal shares for the 4
  // wavefronts, and at least 8 pages.
  const int64_t parts = (num_cus + pairs - 1) / pairs;
  int64_t pages = (longest + parts - 1) / parts;
  pages = ((pages + 3) / 4) * 4;
  if (pages < kMinPartitionPages) pages = kMinPartitionPages;
  return pages >= longest || pages >= cap ? cap : (int32_t)pages;
}
}  // namespace

extern "C" int32_t pkv_plan_partition_pages(int32_t batch, int32_t num_kv_heads, int32_t max_blocks_per_seq,
                                            int32_t num_cus) {
  if (batch < 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 || num_cus <= 0) return -1;
  return plan_pages((int64_t)batch * num_kv_heads, max_blocks_per_seq, max_blocks_per_seq, num_cus);
}

extern "C" int32_t pkv_plan_partition_pages_for_context(int32_t batch, int32_t num_kv_heads,
                                                        int32_t max_blocks_per_seq, int32_t max_context_len,
                                                        int32_t num_cus) {
  if (batch < 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 || num_cus <= 0) return -1;
  if (max_context_len < 0) return pkv_plan_partition_pages(batch, num_kv_heads, max_blocks_per_seq, num_cus);
  int64_t longest = ((int64_t)max_context_len + pkv::kBlock - 1) / pkv::kBlock;
  if (longest > max_blocks_per_seq) longest = max_blocks_per_seq;
  return plan_pages((int64_t)batch * num_kv_heads, max_blocks_per_seq, longest, num_cus);
}

namespace {
// Pages per partition actually used for a requested (positive) size.
int32_t resolved_partition_pages(int32_t requested, int32_t max_blocks_per_seq) {
  int32_t pp = requested;
  if (pp > max_blocks_per_seq) pp = max_blocks_per_seq;
  if (pp > pkv::kMaxPartitionPages) pp = pkv::kMaxPartitionPages;
  return pp;
}
}  // namespace

namespace {
// Split workspace: partial outputs f32[batch][num_q_heads][parts][64], then (max, denominator)
// pairs f32[batch][num_q_heads][parts][2], then, from the next 128-byte boundary, one counter per
// (sequence, KV head) every kCounterStride words.
constexpr size_t kCounterAlign = 128;
size_t counter_offset(int64_t slots) { return (size_t)slots * (pkv::kHeadDim + 2) * sizeof(float); }
size_t counter_bytes(int64_t pairs) { return (size_t)pairs * pkv::kCounterStride * sizeof(uint32_t); }
}  // namespace

extern "C" size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                             int32_t partition_pages) {
  if (batch < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 || partition_pages <= 0) return 0;
  const int32_t pp = resolved_partition_pages(partition_pages, max_blocks_per_seq);
  const int64_t parts = ((int64_t)max_blocks_per_seq + pp - 1) / pp;
  if (parts <= 1) return 0;
  const int64_t slots = (int64_t)batch * num_q_heads * parts;
  const int64_t pairs = ((int64_t)batch * num_q_heads + pkv::kGroup - 1) / pkv::kGroup;
  // the counters' 128-byte alignment may need up to 112 bytes of padding after a 16-byte base
  return counter_offset(slots) + kCounterAlign + counter_bytes(pairs);
}

extern "C" pkv_status pkv_kv_append(const pkv_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                    const int32_t *positions, const void *k_new, const void *v_new, int32_t batch,
                                    void *stream) {
  if (!pool) return PKV_ERR_NULL;
  if (batch < 0 || max_blocks_per_seq <= 0 || pool->num_pages <= 0 || pool->num_kv_heads <= 0) return PKV_ERR_SHAPE;
  if (pool->head_dim != pkv::kHeadDim || pool->block_size != pkv::kBlock) return PKV_ERR_UNSUPPORTED;
  if (batch == 0) return PKV_OK;
  if (!pool->k_pool || !pool->v_pool || !block_tables || !positions || !k_new || !v_new) return PKV_ERR_NULL;
  if (!aligned16(pool->k_pool) || !aligned16(pool->v_pool) || !aligned16(k_new) || !aligned16(v_new))
    return PKV_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (debug_validate_enabled()) {
    std::vector<int32_t> bt, pos;
    pkv_status st = copy_to_host(bt, block_tables, (size_t)batch * max_blocks_per_seq, s);
    if (st == PKV_OK) st = copy_to_host(pos, positions, (size_t)batch, s);
    if (st != PKV_OK) return st;
    st = pkv_validate_append_host(bt.data(), max_blocks_per_seq, pos.data(), batch, pool->num_pages, nullptr);
    if (st != PKV_OK) return st;
  }

  pkv::AppendParams p;
  p.k_pool = static_cast<uint16_t *>(pool->k_pool);
  p.v_pool = static_cast<uint16_t *>(pool->v_pool);
  p.block_tables = block_tables;
  p.positions = positions;
  p.k_new = static_cast<const uint16_t *>(k_new);
  p.v_new = static_cast<const uint16_t *>(v_new);
  p.num_pages = pool->num_pages;
  p.num_kv_heads = pool->num_kv_heads;
  p.max_blocks = max_blocks_per_seq;
  p.batch = batch;
  return pkv::launch_kv_append(p, s) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" pkv_status pkv_rope_kv_append(const pkv_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                         const int32_t *positions, const void *q, void *q_out, int32_t num_q_heads,
                                         const void *k_new, const void *v_new, const float *cos_table,
                                         const float *sin_table, int32_t table_rows, int32_t batch, void *stream) {
  if (!pool) return PKV_ERR_NULL;
  if (batch < 0 || max_blocks_per_seq <= 0 || pool->num_pages <= 0 || pool->num_kv_heads <= 0 || num_q_heads <= 0 ||
      table_rows <= 0)
    return PKV_ERR_SHAPE;
  if (pool->head_dim != pkv::kHeadDim || pool->block_size != pkv::kBlock) return PKV_ERR_UNSUPPORTED;
  if (batch == 0) return PKV_OK;
  if (!pool->k_pool || !pool->v_pool || !block_tables || !positions || !q || !q_out || !k_new || !v_new ||
      !cos_table || !sin_table)
    return PKV_ERR_NULL;
  if (!aligned16(pool->k_pool) || !aligned16(pool->v_pool) || !aligned16(q) || !aligned16(q_out) ||
      !aligned16(k_new) || !aligned16(v_new) || !aligned16(cos_table) || !aligned16(sin_table))
    return PKV_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (debug_validate_enabled()) {
    std::vector<int32_t> bt, pos;
    pkv_status st = copy_to_host(bt, block_tables, (size_t)batch * max_blocks_per_seq, s);
    if (st == PKV_OK) st = copy_to_host(pos, positions, (size_t)batch, s);
    if (st != PKV_OK) return st;
    st = pkv_validate_append_host(bt.data(), max_blocks_per_seq, pos.data(), batch, pool->num_pages, nullptr);
    if (st != PKV_OK) return st;
    for (int32_t b = 0; b < batch; ++b)
      if (pos[b] >= table_rows) return PKV_ERR_VALIDATION;
  }

  pkv::RopeAppendParams p;
  p.app.k_pool = static_cast<uint16_t *>(pool->k_pool);
  p.app.v_pool = static_cast<uint16_t *>(pool->v_pool);
  p.app.block_tables = block_tables;
  p.app.positions = positions;
  p.app.k_new = static_cast<const uint16_t *>(k_new);
  p.app.v_new = static_cast<const uint16_t *>(v_new);
  p.app.num_pages = pool->num_pages;
  p.app.num_kv_heads = pool->num_kv_heads;
  p.app.max_blocks = max_blocks_per_seq;
  p.app.batch = batch;
  p.q = static_cast<const uint16_t *>(q);
  p.q_out = static_cast<uint16_t *>(q_out);
  p.cos_table = cos_table;
  p.sin_table = sin_table;
  p.table_rows = table_rows;
  p.num_q_heads = num_q_heads;
  return pkv::launch_rope_append(p, s) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

namespace {

// Scratch for pkv_decode_step_static: one array per device, resolved once per device with
// hipGetSymbolAddress and only ever passed to kernels through that address.  Static storage starts
// zero-filled, and every decode call leaves its split scratch all-zero again (the partition that
// merges a split resets its counter and zeroes the partials it read), which is the state a split
// needs when it starts.
static __device__ __align__(256) unsigned char scratch[PKV_STATIC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // written and read under g_scratch_mutex

pkv_status static_scratch_address(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return PKV_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

namespace {

// Shared by the attention call and the fused decode step.  `positions` != nullptr selects the
// fused step: the context is positions[b] + 1 and k_new / v_new are appended on the way.
pkv_status decode_common(const void *q, const void *k_pool, const void *v_pool, int32_t num_pages,
                         const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                         const int32_t *positions, const void *k_new, const void *v_new, void *out,
                         pkv_out_dtype out_dtype, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, float scale, int32_t partition_pages, void *workspace,
                         size_t workspace_bytes, void *stream, bool static_scratch = false) {
  const bool fused = positions != nullptr;
  if (batch < 0 || num_pages <= 0 || max_blocks_per_seq <= 0 || num_q_heads <= 0 || num_kv_heads <= 0)
    return PKV_ERR_SHAPE;
  if (!(scale > 0.0f) || !isfinite(scale)) return PKV_ERR_SHAPE;
  if (out_dtype != PKV_OUT_BF16 && out_dtype != PKV_OUT_F32) return PKV_ERR_SHAPE;
  if (head_dim != pkv::kHeadDim || block_size != pkv::kBlock || num_q_heads != pkv::kGroup * num_kv_heads)
    return PKV_ERR_UNSUPPORTED;
  if (batch == 0) return PKV_OK;
  if (batch > kMaxGridDim) return PKV_ERR_SHAPE;  // one grid dimension per sequence
  if (!q || !k_pool || !v_pool || !block_tables || !out) return PKV_ERR_NULL;
  if (fused ? (!k_new || !v_new) : !context_lens) return PKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out)) return PKV_ERR_ALIGNMENT;
  if (fused && (!aligned16(k_new) || !aligned16(v_new))) return PKV_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);

  int32_t cus = 0;  // queried only when the plan needs it, after the argument checks otherwise
  int32_t part_pages = partition_pages;
  if (part_pages <= 0) {
    cus = pkv_device_cu_count();
    if (cus <= 0) return PKV_ERR_HIP;
    part_pages = pkv_plan_partition_pages(batch, num_kv_heads, max_blocks_per_seq, cus);
  }
  part_pages = resolved_partition_pages(part_pages, max_blocks_per_seq);
  const int32_t num_parts = (max_blocks_per_seq + part_pages - 1) / part_pages;
  if (num_parts > kMaxGridDim) return PKV_ERR_SHAPE;
  if (num_parts > 1) {
    const size_t need = pkv_decode_workspace_bytes(batch, num_q_heads, max_blocks_per_seq, part_pages);
    if (static_scratch) {
      if (need > PKV_STATIC_SCRATCH_BYTES) return PKV_ERR_SCRATCH;
      pkv_status st = static_scratch_address(&workspace);
      if (st != PKV_OK) return st;
      workspace_bytes = PKV_STATIC_SCRATCH_BYTES;
    }
    if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PKV_ERR_ALIGNMENT;
  }

  if (num_parts == 1 && cus <= 0) {  // the unsplit kernel flavour depends on the device size
    cus = pkv_device_cu_count();
    if (cus <= 0) return PKV_ERR_HIP;
  }
  uint32_t *counters = nullptr;
  int64_t slots = 0;
  if (num_parts > 1) {
    slots = (int64_t)batch * num_q_heads * num_parts;
    const uintptr_t c = reinterpret_cast<uintptr_t>(workspace) + counter_offset(slots);
    counters = reinterpret_cast<uint32_t *>((c + kCounterAlign - 1) & ~(uintptr_t)(kCounterAlign - 1));
  }

  if (!static_scratch && debug_validate_enabled()) {  // the static-scratch entry allocates nothing
    std::vector<int32_t> bt, lens;
    pkv_status st = copy_to_host(bt, block_tables, (size_t)batch * max_blocks_per_seq, s);
    if (st == PKV_OK) st = copy_to_host(lens, fused ? positions : context_lens, (size_t)batch, s);
    if (st != PKV_OK) return st;
    if (fused) {
      st = pkv_validate_append_host(bt.data(), max_blocks_per_seq, lens.data(), batch, num_pages, nullptr);
      for (auto &l : lens) l += 1;  // the context after the append
    }
    if (st == PKV_OK) st = pkv_validate_decode_host(bt.data(), max_blocks_per_seq, lens.data(), batch, num_pages, nullptr);
    if (st != PKV_OK) return st;
    if (counters) {  // a split needs the workspace's counters at zero (as every call leaves them)
      std::vector<int32_t> ctr;
      st = copy_to_host(ctr, reinterpret_cast<const int32_t *>(counters),
                        counter_bytes((int64_t)batch * num_kv_heads) / sizeof(int32_t), s);
      if (st != PKV_OK) return st;
      for (int32_t v : ctr)
        if (v != 0) return PKV_ERR_VALIDATION;
    }
  }

  pkv::DecodeParams p;
  p.q = static_cast<const uint16_t *>(q);
  p.k_pool = static_cast<const uint16_t *>(k_pool);
  p.v_pool = static_cast<const uint16_t *>(v_pool);
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = out;
  p.part_o = nullptr;
  p.part_ml = nullptr;
  p.counters = counters;
  if (num_parts > 1) {
    p.part_o = static_cast<float *>(workspace);
    p.part_ml = p.part_o + slots * pkv::kHeadDim;
  }
  p.num_pages = num_pages;
  p.max_blocks = max_blocks_per_seq;
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.part_pages = part_pages;
  p.num_parts = num_parts;
  // The matrix-core kernel for every split and for batches with fewer (sequence, KV head) pairs
  // than compute units, where each workgroup's chain of dependent latencies sets the time; the
  // vector-ALU kernel (slightly faster when HBM is the bound) for the rest.
  p.matrix_cores = (num_parts > 1 || (int64_t)batch * num_kv_heads < (int64_t)cus) ? 1 : 0;
  p.score_log2 = scale * 1.4426950408889634f;
  p.positions = positions;
  p.k_new = static_cast<const uint16_t *>(k_new);
  p.v_new = static_cast<const uint16_t *>(v_new);
  p.k_pool_w = fused ? const_cast<uint16_t *>(p.k_pool) : nullptr;
  p.v_pool_w = fused ? const_cast<uint16_t *>(p.v_pool) : nullptr;
  return pkv::launch_paged_decode(p, out_dtype == PKV_OUT_BF16, s) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

extern "C" pkv_status pkv_paged_decode_attention(const void *q, const void *k_pool, const void *v_pool,
                                                 int32_t num_pages, const int32_t *block_tables,
                                                 int32_t max_blocks_per_seq, const int32_t *context_lens, void *out,
                                                 pkv_out_dtype out_dtype, int32_t batch, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                 float scale, int32_t partition_pages, void *workspace,
                                                 size_t workspace_bytes, void *stream) {
  return decode_common(q, k_pool, v_pool, num_pages, block_tables, max_blocks_per_seq, context_lens, nullptr, nullptr,
                       nullptr, out, out_dtype, batch, num_q_heads, num_kv_heads, head_dim, block_size, scale,
                       partition_pages, workspace, workspace_bytes, stream);
}

extern "C" pkv_status pkv_decode_step(const pkv_pool *pool, const void *q, const int32_t *block_tables,
                                      int32_t max_blocks_per_seq, const int32_t *positions, const void *k_new,
                                      const void *v_new, void *out, pkv_out_dtype out_dtype, int32_t batch,
                                      int32_t num_q_heads, float scale, int32_t partition_pages, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  if (!pool) return PKV_ERR_NULL;
  if (batch > 0 && !positions) return PKV_ERR_NULL;
  return decode_common(q, pool->k_pool, pool->v_pool, pool->num_pages, block_tables, max_blocks_per_seq, nullptr,
                       positions, k_new, v_new, out, out_dtype, batch, num_q_heads, pool->num_kv_heads, pool->head_dim,
                       pool->block_size, scale, partition_pages, workspace, workspace_bytes, stream);
}

extern "C" pkv_status pkv_decode_step_static(const pkv_pool *pool, const void *q, const int32_t *block_tables,
                                             int32_t max_blocks_per_seq, const int32_t *positions, const void *k_new,
                                             const void *v_new, void *out, pkv_out_dtype out_dtype, int32_t batch,
                                             int32_t num_q_heads, float scale, int32_t partition_pages, void *stream) {
  if (!pool) return PKV_ERR_NULL;
  if (batch > 0 && !positions) return PKV_ERR_NULL;
  return decode_common(q, pool->k_pool, pool->v_pool, pool->num_pages, block_tables, max_blocks_per_seq, nullptr,
                       positions, k_new, v_new, out, out_dtype, batch, num_q_heads, pool->num_kv_heads, pool->head_dim,
                       pool->block_size, scale, partition_pages, nullptr, 0, stream, /*static_scratch=*/true);
}

namespace {

pkv_status copy_bytes_to_host(void *dst, const void *src, size_t n, hipStream_t stream) {
  if (n == 0) return PKV_OK;
  if (hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToHost, stream) != hipSuccess) return PKV_ERR_HIP;
  return PKV_OK;
}

// Debug validation of the prompt rows' values (after the table / bounds checks passed): every K
// and V value of every sequence's prompt rows must be finite, since the attention kernel gives a
// masked (later) key weight 0 and 0 times an infinity or NaN would reach earlier rows of the same
// query tile.  The append checks k_new / v_new; the attention checks the same rows in the pool
// (where the append put them), copied page by page through the table.
pkv_status check_prompt_rows_finite(const pkv_pool *pool, const std::vector<int32_t> &bt, int32_t max_blocks,
                                    const std::vector<int32_t> &cu, const std::vector<int32_t> &st, int32_t batch,
                                    const void *k_new, const void *v_new, hipStream_t s) {
  const int32_t hkv = pool->num_kv_heads;
  const size_t row_elems = (size_t)hkv * pkv::kHeadDim;
  if (k_new) {
    const int32_t r0 = cu[0], r1 = cu[batch];  // validated: non-decreasing, inside [0, num_tokens]
    std::vector<uint16_t> k((size_t)(r1 - r0) * row_elems), v(k.size());
    const size_t off = (size_t)r0 * row_elems;
    pkv_status r = copy_bytes_to_host(k.data(), static_cast<const uint16_t *>(k_new) + off, k.size() * 2, s);
    if (r == PKV_OK) r = copy_bytes_to_host(v.data(), static_cast<const uint16_t *>(v_new) + off, v.size() * 2, s);
    if (r != PKV_OK) return r;
    if (hipStreamSynchronize(s) != hipSuccess) return PKV_ERR_HIP;
    r = pkv_validate_finite_rows_host(k.data(), r1 - r0, (int32_t)row_elems, nullptr);
    if (r == PKV_OK) r = pkv_validate_finite_rows_host(v.data(), r1 - r0, (int32_t)row_elems, nullptr);
    return r;
  }
  const size_t page_elems = row_elems * pkv::kBlock;
  std::vector<uint16_t> kp(page_elems), vp(page_elems);
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = cu[b + 1] - cu[b], start = st[b];
    for (int64_t pos0 = start; pos0 < start + n;) {
      const int64_t blk = pos0 / pkv::kBlock;
      const int64_t pos1 = std::min<int64_t>(start + n, (blk + 1) * pkv::kBlock);  // this page's prompt slots
      const int32_t page = bt[(size_t)b * max_blocks + blk];
      pkv_status r = copy_bytes_to_host(kp.data(), static_cast<const uint16_t *>(pool->k_pool) + page * page_elems,
                                        page_elems * 2, s);
      if (r == PKV_OK)
        r = copy_bytes_to_host(vp.data(), static_cast<const uint16_t *>(pool->v_pool) + page * page_elems,
                               page_elems * 2, s);
      if (r != PKV_OK) return r;
      if (hipStreamSynchronize(s) != hipSuccess) return PKV_ERR_HIP;
      const int32_t s0 = (int32_t)(pos0 % pkv::kBlock), count = (int32_t)(pos1 - pos0);
      for (int32_t g = 0; g < hkv && r == PKV_OK; ++g) {
        const size_t first = ((size_t)g * pkv::kBlock + s0) * pkv::kHeadDim;
        r = pkv_validate_finite_rows_host(kp.data() + first, count, pkv::kHeadDim, nullptr);
        if (r == PKV_OK) r = pkv_validate_finite_rows_host(vp.data() + first, count, pkv::kHeadDim, nullptr);
      }
      if (r != PKV_OK) return r;
      pos0 = pos1;
    }
  }
  return PKV_OK;
}

// Synchronous checks shared by both prefill calls.  `append` selects which copy of the prompt
// rows debug validation checks for finite values: k_new / v_new (append) or the pool (attention).
pkv_status prefill_checks(const pkv_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                          const int32_t *cu_seqlens, const int32_t *start_pos, int32_t batch, int32_t num_tokens,
                          int32_t max_prompt_len, bool append, const void *k_new, const void *v_new, hipStream_t s) {
  if (!pool) return PKV_ERR_NULL;
  if (batch < 0 || num_tokens < 0 || max_prompt_len < 0 || max_blocks_per_seq <= 0 || pool->num_pages <= 0 ||
      pool->num_kv_heads <= 0)
    return PKV_ERR_SHAPE;
  if (pool->head_dim != pkv::kHeadDim || pool->block_size != pkv::kBlock) return PKV_ERR_UNSUPPORTED;
  if (batch > 65535 || max_prompt_len > 16 * 65535) return PKV_ERR_SHAPE;  // grid y / z limits
  if (batch == 0 || num_tokens == 0 || max_prompt_len == 0) return PKV_OK;
  if (!pool->k_pool || !pool->v_pool || !block_tables || !cu_seqlens || !start_pos) return PKV_ERR_NULL;
  if (!aligned16(pool->k_pool) || !aligned16(pool->v_pool)) return PKV_ERR_ALIGNMENT;
  if (debug_validate_enabled()) {
    std::vector<int32_t> bt, cu, st;
    pkv_status r = copy_to_host(bt, block_tables, (size_t)batch * max_blocks_per_seq, s);
    if (r == PKV_OK) r = copy_to_host(cu, cu_seqlens, (size_t)batch + 1, s);
    if (r == PKV_OK) r = copy_to_host(st, start_pos, (size_t)batch, s);
    if (r != PKV_OK) return r;
    r = pkv_validate_prefill_host(bt.data(), max_blocks_per_seq, cu.data(), st.data(), batch, num_tokens,
                                  max_prompt_len, pool->num_pages, nullptr);
    if (r != PKV_OK) return r;
    r = check_prompt_rows_finite(pool, bt, max_blocks_per_seq, cu, st, batch, append ? k_new : nullptr,
                                 append ? v_new : nullptr, s);
    if (r != PKV_OK) return r;
  }
  return PKV_OK;
}

pkv::PrefillParams prefill_params(const pkv_pool *pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                  const int32_t *cu_seqlens, const int32_t *start_pos, int32_t batch,
                                  int32_t num_tokens, int32_t max_prompt_len) {
  pkv::PrefillParams p{};
  p.k_pool = static_cast<uint16_t *>(pool->k_pool);
  p.v_pool = static_cast<uint16_t *>(pool->v_pool);
  p.block_tables = block_tables;
  p.cu_seqlens = cu_seqlens;
  p.start_pos = start_pos;
  p.num_pages = pool->num_pages;
  p.num_kv_heads = pool->num_kv_heads;
  p.max_blocks = max_blocks_per_seq;
  p.batch = batch;
  p.num_tokens = num_tokens;
  p.max_prompt_len = max_prompt_len;
  return p;
}

}  // namespace

extern "C" pkv_status pkv_prefill_kv_append(const pkv_pool *pool, const int32_t *block_tables,
                                            int32_t max_blocks_per_seq, const int32_t *cu_seqlens,
                                            const int32_t *start_pos, const void *k_new, const void *v_new,
                                            int32_t batch, int32_t num_tokens, int32_t max_prompt_len, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pool && batch > 0 && num_tokens > 0 && max_prompt_len > 0) {
    if (!k_new || !v_new) return PKV_ERR_NULL;
    if (!aligned16(k_new) || !aligned16(v_new)) return PKV_ERR_ALIGNMENT;
  }
  pkv_status st = prefill_checks(pool, block_tables, max_blocks_per_seq, cu_seqlens, start_pos, batch, num_tokens,
                                 max_prompt_len, true, k_new, v_new, s);
  if (st != PKV_OK || batch == 0 || num_tokens == 0 || max_prompt_len == 0) return st;
  pkv::PrefillParams p =
      prefill_params(pool, block_tables, max_blocks_per_seq, cu_seqlens, start_pos, batch, num_tokens, max_prompt_len);
  p.k_new = static_cast<const uint16_t *>(k_new);
  p.v_new = static_cast<const uint16_t *>(v_new);
  return pkv::launch_prefill_append(p, s) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" pkv_status pkv_paged_prefill_attention(const pkv_pool *pool, const void *q, const int32_t *block_tables,
                                                  int32_t max_blocks_per_seq, const int32_t *cu_seqlens,
                                                  const int32_t *start_pos, void *out, pkv_out_dtype out_dtype,
                                                  int32_t batch, int32_t num_tokens, int32_t max_prompt_len,
                                                  int32_t num_q_heads, float scale, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!(scale > 0.0f) || !isfinite(scale)) return PKV_ERR_SHAPE;
  if (out_dtype != PKV_OUT_BF16 && out_dtype != PKV_OUT_F32) return PKV_ERR_SHAPE;
  if (num_q_heads <= 0) return PKV_ERR_SHAPE;
  if (pool && pool->num_kv_heads > 0 && num_q_heads != pkv::kGroup * pool->num_kv_heads) return PKV_ERR_UNSUPPORTED;
  if (pool && batch > 0 && num_tokens > 0 && max_prompt_len > 0) {
    if (!q || !out) return PKV_ERR_NULL;
    if (!aligned16(q) || !aligned16(out)) return PKV_ERR_ALIGNMENT;
  }
  pkv_status st = prefill_checks(pool, block_tables, max_blocks_per_seq, cu_seqlens, start_pos, batch, num_tokens,
                                 max_prompt_len, false, nullptr, nullptr, s);
  if (st != PKV_OK || batch == 0 || num_tokens == 0 || max_prompt_len == 0) return st;
  pkv::PrefillParams p =
      prefill_params(pool, block_tables, max_blocks_per_seq, cu_seqlens, start_pos, batch, num_tokens, max_prompt_len);
  p.q = static_cast<const uint16_t *>(q);
  p.out = out;
  p.num_q_heads = num_q_heads;
  p.score_log2 = scale * 1.4426950408889634f;
  const int32_t cus = pkv_device_cu_count();
  if (cus <= 0) return PKV_ERR_HIP;
  return pkv::launch_prefill_attention(p, out_dtype == PKV_OUT_BF16, cus, s) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
