// Paged prefill: write a prompt's K/V rows into their pages, then causal attention over those
// pages ("The prefill path: flowing the entire prompt at once", sections "Distributing K/V into
// paged blocks", "Per-head attention scores and GQA", "causalMask and online softmax" and
// "Scores×V → O → residual → SwiGLU").
//
// The article materialises a [tokens][tokens] BF16 score matrix per head, masks it, runs a
// softmax kernel over it and multiplies by V with library GEMMs.  Here no score matrix exists:
// a workgroup owns 16 query rows of one sequence and the 4 query heads of one KV head (one head
// per wavefront), streams the sequence's pages 32 keys at a time through LDS, and runs both
// products on the matrix cores (v_mfma_f32_16x16x32_bf16) with an FP32 online softmax in between.
//
// Register layout of the 16x16x32 BF16 MFMA on gfx950 (lane l, element i):
//   A operand: row l % 16, reduction index 8 (l / 16) + i
//   B operand: column l % 16, reduction index 8 (l / 16) + i
//   C/D:       column l % 16, row 4 (l / 16) + i
// Scores are computed transposed, S^T = K Q^T (rows = keys, columns = the 16 queries), with the
// 16 A-operand rows of key tile t mapped to keys 8 (r / 4) + 4 t + r % 4 of the 32-key step.
// Then lane l holds, for query l % 16, exactly keys 8 (l / 16) .. 8 (l / 16) + 7 of the step in
// its two C tiles, which is the B-operand layout of P^T in O^T = V^T P^T: the probabilities
// never leave their registers.  V is staged transposed in LDS so that V^T rows are contiguous.
// The probabilities enter the second product as two BF16 terms (hi + lo), so the weights keep
// about 16 significant bits; Q, K and V are BF16 inputs and are exact in the products.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTileQ = 16;                 // query rows per workgroup
constexpr int kChunk = 32;                 // keys per step (two pages)
constexpr int kVecPerRow = kHeadDim * 2 / 16;  // 16-byte vectors per 64-wide BF16 row
constexpr int kKStride = kHeadDim + 8;     // BF16 elements per staged K row (144 bytes)
constexpr int kVStride = kChunk + 8;       // BF16 elements per staged V^T row (80 bytes)

// Packed rows of sequence b, or false when they fall outside [0, num_tokens) or exceed the
// prompt-length bound the grid was sized for (such a sequence is left untouched).
__device__ __forceinline__ bool sequence_rows(const PrefillParams &p, int b, int32_t &row0, int32_t &n) {
  row0 = p.cu_seqlens[b];
  const int32_t end = p.cu_seqlens[b + 1];
  n = end - row0;
  return row0 >= 0 && n >= 0 && end <= p.num_tokens && n <= p.max_prompt_len;
}

// ---------------------------------------------------------------------------------------------
// Append: one lane per 16-byte vector of a prompt row's K (and the same vector of V).
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void prefill_append_kernel(PrefillParams p) {
  const int b = blockIdx.y;
  const int per_row = p.num_kv_heads * kVecPerRow;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t i = idx / per_row;
  int32_t row0, n;
  if (!sequence_rows(p, b, row0, n) || i >= n) return;
  const int r = (int)(idx - i * per_row);  // g * kVecPerRow + vector
  const int32_t start = p.start_pos[b];
  const int64_t pos = (int64_t)start + i;
  if (start < 0 || pos >= (int64_t)p.max_blocks * kBlock) return;
  const int32_t page = p.block_tables[(int64_t)b * p.max_blocks + pos / kBlock];
  if (page < 0 || page >= p.num_pages) return;
  const int g = r / kVecPerRow, c = r % kVecPerRow;
  const int64_t src = (row0 + i) * per_row + r;
  const int64_t dst = (((int64_t)page * p.num_kv_heads + g) * kBlock + pos % kBlock) * kVecPerRow + c;
  reinterpret_cast<uint4 *>(p.k_pool)[dst] = reinterpret_cast<const uint4 *>(p.k_new)[src];
  reinterpret_cast<uint4 *>(p.v_pool)[dst] = reinterpret_cast<const uint4 *>(p.v_new)[src];
}

// ---------------------------------------------------------------------------------------------
// Attention
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_xor_max(float x, int mask) { return fmaxf(x, __shfl_xor(x, mask, 64)); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <bool kOutBf16>
__device__ __forceinline__ void store_row4(void *out, int64_t elem, f32x4 v) {
  if constexpr (kOutBf16) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 o;
    o[0] = (__bf16)v[0];
    o[1] = (__bf16)v[1];
    o[2] = (__bf16)v[2];
    o[3] = (__bf16)v[3];
    *reinterpret_cast<bf16x4 *>(static_cast<uint16_t *>(out) + elem) = o;
  } else {
    *reinterpret_cast<f32x4 *>(static_cast<float *>(out) + elem) = v;
  }
}

// grid = (num_kv_heads, batch, ceil(max_prompt_len / 16)); the query tile runs backwards in z so
// the workgroups with the most keys are dispatched first.
template <bool kOutBf16>
__global__ __launch_bounds__(kThreads) void prefill_attention_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kChunk * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][kHeadDim * kVStride];

  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int tile = (int)(gridDim.z - 1 - blockIdx.z);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int h = g * kGroup + (tid >> 6);  // one query head per wavefront
  const int r = lane & 15;                 // this lane's query column
  const int j = lane >> 4;                 // this lane's group of 8 keys / 8 dims

  int32_t row0, n;
  if (!sequence_rows(p, b, row0, n)) return;
  const int q_lo = tile * kTileQ;
  if (q_lo >= n) return;
  const int q_rows = min(kTileQ, n - q_lo);
  const int32_t start = p.start_pos[b];
  const int32_t *table = p.block_tables + (int64_t)b * p.max_blocks;

  // The whole sequence must be addressable: every page up to its last prompt position.
  int bad = !(start >= 0 && (int64_t)start + n <= (int64_t)p.max_blocks * kBlock);
  if (!bad) {
    const int need = (start + n + kBlock - 1) / kBlock;
    for (int e = tid; e < need; e += kThreads) {
      const int32_t pg = table[e];
      bad |= pg < 0 || pg >= p.num_pages;
    }
  }
  bad = __syncthreads_or(bad);
  const int64_t out_row = (int64_t)row0 + q_lo + r;  // this lane's output row
  if (bad) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    if (r < q_rows)
      for (int dt = 0; dt < 4; ++dt)
        store_row4<kOutBf16>(p.out, (out_row * p.num_q_heads + h) * kHeadDim + 16 * dt + 4 * j, zero);
    return;
  }

  const int n_keys = start + q_lo + q_rows;  // keys 0 .. last query position of the tile
  const int n_chunks = (n_keys + kChunk - 1) / kChunk;
  const int q_pos = start + q_lo + r;        // this lane's query position

  // Q^T as the B operand of S^T = K Q^T: query column r, dims 32 half + 8 j .. + 7.
  u32x4 qf[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  if (r < q_rows) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(p.q + (out_row * p.num_q_heads + h) * kHeadDim);
    qf[0] = src[j];
    qf[1] = src[4 + j];
  }

  // Staging: thread -> key (tid % 32) of the step and dims 8 (tid / 32) .. + 7.
  const int st_key = tid & 31;
  const int st_dim = (tid >> 5) * 8;
  auto load_step = [&](int c, u32x4 &kr, u32x4 &vr) {
    const int kp = c * kChunk + st_key;
    kr = u32x4{0, 0, 0, 0};
    vr = u32x4{0, 0, 0, 0};
    if (kp < n_keys) {  // keys past the tile's last query stay zero (no stale NaN reaches V)
      const int32_t pg = table[kp / kBlock];
      const int64_t off = (((int64_t)pg * p.num_kv_heads + g) * kBlock + kp % kBlock) * kHeadDim + st_dim;
      kr = *reinterpret_cast<const u32x4 *>(p.k_pool + off);
      vr = *reinterpret_cast<const u32x4 *>(p.v_pool + off);
    }
  };
  auto stage = [&](int buf, const u32x4 &kr, const u32x4 &vr) {
    *reinterpret_cast<u32x4 *>(&s_k[buf][st_key * kKStride + st_dim]) = kr;
    uint16_t *vt = &s_vt[buf][st_dim * kVStride + st_key];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vt[(2 * e) * kVStride] = (uint16_t)(vr[e] & 0xFFFFu);
      vt[(2 * e + 1) * kVStride] = (uint16_t)(vr[e] >> 16);
    }
  };

  u32x4 kr, vr;
  load_step(0, kr, vr);
  stage(0, kr, vr);
  __syncthreads();

  f32x4 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;  // running max in log2 units, shared by the 4 lanes of a query
  float l = 0.f;        // this lane's part of the denominator
  const float c_log2 = p.score_log2;

  for (int c = 0; c < n_chunks; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < n_chunks;
    if (more) load_step(c + 1, kr, vr);  // in flight while this step computes

    // S^T for the two key tiles of the step.
    f32x4 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key_row = 8 * (r >> 2) + 4 * t + (r & 3);
      const uint16_t *krow = &s_k[buf][key_row * kKStride + 8 * j];
      const u32x4 k0 = *reinterpret_cast<const u32x4 *>(krow);
      const u32x4 k1 = *reinterpret_cast<const u32x4 *>(krow + 32);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k0), as_bf16x8(qf[0]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k1), as_bf16x8(qf[1]), acc, 0, 0, 0);
      s[t] = acc;
    }

    // Causal mask and the online softmax (scores in log2 units).
    const int key0 = c * kChunk + 8 * j;  // keys key0 + 4 t + i
    float x[8];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool visible = key0 + 4 * t + i <= q_pos;
        const float v = visible ? s[t][i] * c_log2 : -INFINITY;
        x[4 * t + i] = v;
        mx = fmaxf(mx, v);
      }
    mx = wave_xor_max(mx, 16);
    mx = wave_xor_max(mx, 32);
    const float m_new = fmaxf(m, mx);  // finite: key 0 is visible to every query
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    // Each weight is carried as a sum of two BF16 values (hi + lo, ~16 significant bits): with a
    // single BF16 weight a short context keeps the 2^-9 rounding of its few large weights.
    bf16x8 ph, pl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = __builtin_amdgcn_exp2f(x[e] - m);
      l += pe;
      const __bf16 hi = (__bf16)pe;
      ph[e] = hi;
      pl[e] = (__bf16)(pe - (float)hi);  // the difference is exact in FP32
    }

    // O^T += V^T P^T, one 16-dim tile at a time.
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const u32x4 vf = *reinterpret_cast<const u32x4 *>(&s_vt[buf][(16 * dt + r) * kVStride + 8 * j]);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf), ph, o[dt], 0, 0, 0);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf), pl, o[dt], 0, 0, 0);
    }

    if (more) stage(buf ^ 1, kr, vr);
    __syncthreads();
  }

  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  const float inv = 1.0f / l;
  if (r < q_rows)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      store_row4<kOutBf16>(p.out, (out_row * p.num_q_heads + h) * kHeadDim + 16 * dt + 4 * j, o[dt] * inv);
}

}  // namespace

hipError_t launch_prefill_append(const PrefillParams &p, hipStream_t stream) {
  const int64_t lanes = (int64_t)p.max_prompt_len * p.num_kv_heads * kVecPerRow;
  if (lanes == 0 || p.batch == 0) return hipSuccess;
  const int64_t blocks = (lanes + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffff || p.batch > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefill_append_kernel, dim3((unsigned)blocks, (unsigned)p.batch), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_prefill_attention(const PrefillParams &p, bool out_bf16, hipStream_t stream) {
  const int64_t tiles = ((int64_t)p.max_prompt_len + kTileQ - 1) / kTileQ;
  if (tiles == 0 || p.batch == 0) return hipSuccess;
  if (tiles > 65535 || p.batch > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)p.num_kv_heads, (unsigned)p.batch, (unsigned)tiles);
  if (out_bf16)
    hipLaunchKernelGGL(prefill_attention_kernel<true>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_attention_kernel<false>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
