// kv_append: write each sequence's new K/V row into slot (pos % 16) of page table[pos / 16].
//
// The decode step appends one new token per sequence at its absolute position into the shared
// BF16 page pool ("6 Hours of YouTube and 85 handtyped pages of notes on LLM Inference", section "What works so far"); the page is the block-table entry of
// logical block pos / 16 ("The prefill path: flowing the entire prompt at once", section "Distributing K/V into paged
// blocks").  With the [page][kv_head][token][dim] layout every (sequence, KV head) row is one
// 128-byte run in K and one in V, so the kernel is a scatter of 16-byte vectors: one lane per
// 16 bytes, 8 lanes per row.  Bits are copied unchanged.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kVecPerRow = kHeadDim * 2 / 16;  // 16-byte vectors per 128-byte row

__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(AppendParams p) {
  // Lane -> (sequence b, KV head g, K-or-V, vector c).  Consecutive lanes cover one K row, then
  // the matching V row, so every load and store instruction touches whole 128-byte runs.
  const int64_t i = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
  const int64_t per_seq = (int64_t)p.num_kv_heads * 2 * kVecPerRow;
  const int64_t b = i / per_seq;
  if (b >= p.batch) return;
  const int r = (int)(i - b * per_seq);
  const int g = r / (2 * kVecPerRow);
  const int is_v = (r / kVecPerRow) & 1;
  const int c = r % kVecPerRow;

  const int32_t pos = p.positions[b];
  if (pos < 0 || pos >= p.max_blocks * kBlock) return;  // never dereference outside the table
  const int32_t page = p.block_tables[b * p.max_blocks + pos / kBlock];
  if (page < 0 || page >= p.num_pages) return;  // never write outside the pool

  const int64_t src_row = b * p.num_kv_heads + g;
  const int64_t dst_row = ((int64_t)page * p.num_kv_heads + g) * kBlock + (pos % kBlock);
  const uint4 *src = reinterpret_cast<const uint4 *>(is_v ? p.v_new : p.k_new) + src_row * kVecPerRow + c;
  uint4 *dst = reinterpret_cast<uint4 *>(is_v ? p.v_pool : p.k_pool) + dst_row * kVecPerRow + c;
  *dst = *src;
}

}  // namespace

hipError_t launch_kv_append(const AppendParams &p, hipStream_t stream) {
  const int64_t lanes = (int64_t)p.batch * p.num_kv_heads * 2 * kVecPerRow;
  if (lanes == 0) return hipSuccess;
  const int64_t blocks = (lanes + kAppendThreads - 1) / kAppendThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(kAppendThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
