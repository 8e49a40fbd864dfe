// rope_kv_append: rotary embedding of the decode token's q heads and new K row at the token's
// absolute position, then the K/V append ("The prefill path: flowing the entire prompt at once",
// section "RoPE: a rotation that references a table": within each 64-wide head, element i is
// paired with element i + 32 and rotated by the table angle at slot 2i of the position's row;
// queries and keys are rotated, values are not; "6 Hours of YouTube and 85 handtyped pages of
// notes on LLM Inference", section "What works so far": decode appends the new token at its
// absolute RoPE position).
//
// Every product and the sum/difference are separate FP32 operations (contraction is switched off
// below), then the value is rounded to BF16 to nearest even, so the result is one fixed bit
// pattern per input.  One lane per rotated pair; the V row is copied as 16-byte vectors.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kHalf = kHeadDim / 2;
constexpr int kVecPerRow = kHeadDim * 2 / 16;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// y_i = x_i c - x_{i+32} s,  y_{i+32} = x_i s + x_{i+32} c, each operation rounded on its own.
__device__ __forceinline__ void rotate_pair(float x1, float x2, float c, float s, float &y1, float &y2) {
#pragma clang fp contract(off)
  const float a = x1 * c;
  const float b = x2 * s;
  const float d = x1 * s;
  const float e = x2 * c;
  y1 = a - b;
  y2 = d + e;
}

// Position of sequence b if its row may be touched (inside the table and, for the append, inside
// the block table with a valid page), else -1.
__device__ __forceinline__ int32_t usable_pos(const RopeAppendParams &p, int64_t b, int32_t *page) {
  const int32_t pos = p.app.positions[b];
  if (pos < 0 || pos >= p.table_rows || pos >= p.app.max_blocks * kBlock) return -1;
  const int32_t pg = p.app.block_tables[b * p.app.max_blocks + pos / kBlock];
  if (pg < 0 || pg >= p.app.num_pages) return -1;
  *page = pg;
  return pos;
}

__global__ __launch_bounds__(kRopeThreads) void rope_append_kernel(RopeAppendParams p) {
  const int64_t i = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
  const int hq = p.num_q_heads, hkv = p.app.num_kv_heads;
  const int64_t q_lanes = (int64_t)p.app.batch * hq * kHalf;
  const int64_t k_lanes = (int64_t)p.app.batch * hkv * kHalf;
  const int64_t v_lanes = (int64_t)p.app.batch * hkv * kVecPerRow;
  int32_t page = 0;
  if (i < q_lanes) {  // query pair
    const int64_t row = i / kHalf;  // b * hq + h
    const int pair = (int)(i % kHalf);
    const int32_t pos = usable_pos(p, row / hq, &page);
    if (pos < 0) return;
    const uint16_t *x = p.q + row * kHeadDim;
    const float c = p.cos_table[(int64_t)pos * kHeadDim + 2 * pair];
    const float s = p.sin_table[(int64_t)pos * kHeadDim + 2 * pair];
    float y1, y2;
    rotate_pair(bf16_to_f32(x[pair]), bf16_to_f32(x[pair + kHalf]), c, s, y1, y2);
    uint16_t *y = p.q_out + row * kHeadDim;
    y[pair] = f32_to_bf16(y1);
    y[pair + kHalf] = f32_to_bf16(y2);
  } else if (i < q_lanes + k_lanes) {  // new key pair -> rotated into its page slot
    const int64_t j = i - q_lanes;
    const int64_t row = j / kHalf;  // b * hkv + g
    const int pair = (int)(j % kHalf);
    const int64_t b = row / hkv;
    const int g = (int)(row % hkv);
    const int32_t pos = usable_pos(p, b, &page);
    if (pos < 0) return;
    const uint16_t *x = p.app.k_new + row * kHeadDim;
    const float c = p.cos_table[(int64_t)pos * kHeadDim + 2 * pair];
    const float s = p.sin_table[(int64_t)pos * kHeadDim + 2 * pair];
    float y1, y2;
    rotate_pair(bf16_to_f32(x[pair]), bf16_to_f32(x[pair + kHalf]), c, s, y1, y2);
    uint16_t *dst = p.app.k_pool + (((int64_t)page * hkv + g) * kBlock + pos % kBlock) * kHeadDim;
    dst[pair] = f32_to_bf16(y1);
    dst[pair + kHalf] = f32_to_bf16(y2);
  } else if (i < q_lanes + k_lanes + v_lanes) {  // new value row, unrotated
    const int64_t j = i - q_lanes - k_lanes;
    const int64_t row = j / kVecPerRow;
    const int c = (int)(j % kVecPerRow);
    const int64_t b = row / hkv;
    const int g = (int)(row % hkv);
    const int32_t pos = usable_pos(p, b, &page);
    if (pos < 0) return;
    const uint4 *src = reinterpret_cast<const uint4 *>(p.app.v_new) + row * kVecPerRow + c;
    uint4 *dst = reinterpret_cast<uint4 *>(p.app.v_pool) + (((int64_t)page * hkv + g) * kBlock + pos % kBlock) * kVecPerRow + c;
    *dst = *src;
  }
}

}  // namespace

hipError_t launch_rope_append(const RopeAppendParams &p, hipStream_t stream) {
  const int64_t lanes = (int64_t)p.app.batch * (p.num_q_heads * kHalf + p.app.num_kv_heads * (kHalf + kVecPerRow));
  if (lanes == 0) return hipSuccess;
  const int64_t blocks = (lanes + kRopeThreads - 1) / kRopeThreads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_append_kernel, dim3((unsigned)blocks), dim3(kRopeThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
