// Internal declarations shared by the C-ABI layer and the HIP kernels of libpagedkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Compiled geometry: 16-token pages, head_dim 64, four query heads per KV head.
constexpr int kBlock = 16;
constexpr int kHeadDim = 64;
constexpr int kGroup = 4;
// A decode workgroup has 4 wavefronts and each holds one block-table entry per lane, so one
// partition covers at most 4 * 64 pages; longer tables are always split.
constexpr int kMaxPartitionPages = 256;
// Split-context counters sit 128 bytes apart (one per L2 line), so partitions of different
// (sequence, KV head) pairs never contend for a line.
constexpr int kCounterStride = 32;
// Wavefronts per decode workgroup.
constexpr int kWaves = 4;

struct AppendParams {
  uint16_t *k_pool;
  uint16_t *v_pool;
  const int32_t *block_tables;
  const int32_t *positions;
  const uint16_t *k_new;
  const uint16_t *v_new;
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t batch;
};

struct DecodeParams {
  const uint16_t *q;
  const uint16_t *k_pool;
  const uint16_t *v_pool;
  const int32_t *block_tables;
  const int32_t *context_lens;
  void *out;
  float *part_o;   // [batch][num_q_heads][num_parts][kHeadDim], un-normalised partial sums
  float *part_ml;  // [batch][num_q_heads][num_parts][2]: (running max in log2 units, denominator)
  // [batch][num_kv_heads][kCounterStride]: partitions of a (sequence, KV head) that have published
  // their partials; zero between launches (the last partition to arrive resets it).
  uint32_t *counters;
  int32_t num_pages;
  int32_t max_blocks;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t part_pages;  // pages per partition
  int32_t num_parts;   // ceil(max_blocks / part_pages)
  int32_t matrix_cores;  // 1: the MFMA kernel (every split launch, small batches), 0: the vector-ALU kernel
  float score_log2;    // scale * log2(e): scores are kept in log2 units so exp2 does the softmax
  // Fused decode step (positions != nullptr): the context is positions[b] + 1 and the new rows
  // k_new / v_new are written at that position by the workgroup that reads the last page.
  const int32_t *positions;
  const uint16_t *k_new;  // [batch][num_kv_heads][kHeadDim]
  const uint16_t *v_new;
  uint16_t *k_pool_w;     // the same pools, writable
  uint16_t *v_pool_w;
};

struct RopeAppendParams {
  AppendParams app;       // pools, tables, positions, k_new (rotated on the way), v_new
  const uint16_t *q;      // [batch][num_q_heads][kHeadDim]
  uint16_t *q_out;        // rotated q (may equal q)
  const float *cos_table; // [table_rows][kHeadDim]
  const float *sin_table;
  int32_t table_rows;
  int32_t num_q_heads;
};

// Paged prefill: sequence b owns packed rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of q / k_new /
// v_new / out, and its prompt token i sits at absolute position start_pos[b] + i.
struct PrefillParams {
  const uint16_t *q;       // [num_tokens][num_q_heads][kHeadDim]
  uint16_t *k_pool;        // [num_pages][num_kv_heads][kBlock][kHeadDim]
  uint16_t *v_pool;
  const int32_t *block_tables;  // [batch][max_blocks]
  const int32_t *cu_seqlens;    // [batch + 1]
  const int32_t *start_pos;     // [batch]
  const uint16_t *k_new;   // [num_tokens][num_kv_heads][kHeadDim]
  const uint16_t *v_new;
  void *out;               // [num_tokens][num_q_heads][kHeadDim], FP32 or BF16
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t max_blocks;
  int32_t batch;
  int32_t max_prompt_len;  // bound on every prompt length: sets the grid
  int32_t num_tokens;      // rows of q / k_new / v_new / out
  float score_log2;
};

hipError_t launch_kv_append(const AppendParams &p, hipStream_t stream);
hipError_t launch_prefill_append(const PrefillParams &p, hipStream_t stream);
hipError_t launch_prefill_attention(const PrefillParams &p, bool out_bf16, int32_t num_cus, hipStream_t stream);
hipError_t launch_rope_append(const RopeAppendParams &p, hipStream_t stream);
hipError_t launch_paged_decode(const DecodeParams &p, bool out_bf16, hipStream_t stream);

}  // namespace pkv
