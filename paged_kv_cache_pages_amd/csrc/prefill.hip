// Paged prefill: write a prompt's K/V rows into their pages, then causal attention over those
// pages ("The prefill path: flowing the entire prompt at once", sections "Distributing K/V into
// paged blocks", "Per-head attention scores and GQA", "causalMask and online softmax" and
// "Scores×V → O → residual → SwiGLU").
//
// The article materialises a [tokens][tokens] BF16 score matrix per head, masks it, runs a
// softmax kernel over it and multiplies by V with library GEMMs.  Here no score matrix exists:
// a workgroup owns 16 or 32 query rows of one sequence and the 4 query heads of one KV head (one
// head per wavefront), streams the sequence's pages 64 (or 32) keys at a time through LDS, and
// runs both products on the matrix cores (v_mfma_f32_16x16x32_bf16 and _f16) with an FP32 online
// softmax in between.
//
// Register layout of the 16x16x32 BF16 MFMA on gfx950 (lane l, element i):
//   A operand: row l % 16, reduction index 8 (l / 16) + i
//   B operand: column l % 16, reduction index 8 (l / 16) + i
//   C/D:       column l % 16, row 4 (l / 16) + i
// Scores are computed transposed, S^T = K Q^T (rows = keys, columns = the 16 queries), with the
// 16 A-operand rows of key tile t mapped to keys 8 (r / 4) + 4 t + r % 4 of a 32-key half step.
// Then lane l holds, for query l % 16, exactly keys 8 (l / 16) .. 8 (l / 16) + 7 of the half in
// its two C tiles, which is the B-operand layout of P^T in O^T = V^T P^T: the probabilities
// never leave their registers.  V is staged row-major like K; the A operand of V^T comes from the
// transposing LDS read (ds_read_b64_tr_b16), so no transpose happens at staging.
// Q and K enter the first product as the BF16 inputs they are (exact).  For the second product V
// is staged as FP16, which holds every BF16 value up to 65280 exactly (smaller than 2^-14 in
// magnitude only to within 2^-25), and the probabilities enter as FP16 (11 significant bits,
// round to nearest even, scaled by 2^7 so that they leave FP16's subnormal range only below 2^-21
// of the anchor's weight), so the second product needs one FP16 MFMA per tile.  A tile whose V
// holds a larger finite magnitude is computed again in a second pass with BF16 V and each
// probability carried as two BF16 terms (hi + lo, about 16 significant bits; not exact).  The
// prompt's own K/V rows must be finite: a causally masked key still enters the second product
// with weight 0, and 0 times an infinity or NaN reaches the earlier rows of the query tile.
#include <type_traits>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kVecPerRow = kHeadDim * 2 / 16;  // 16-byte vectors per 64-wide BF16 row
constexpr int kKStride = kHeadDim + 8;     // BF16 elements per staged K or V row (144 bytes)

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
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// Eight BF16 values to FP16 (exact for every finite BF16 value up to 65280; the next one, 65536,
// becomes infinity), and the largest magnitude seen so far, so the caller can tell whether all of
// them fit: one above 65280 does not.  The magnitude is an IEEE maximum (v_maximum3 with absolute
// value modifiers, one instruction per pair; a NaN propagates and fails the caller's test).
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 x, float &mag) {
  u32x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __builtin_bit_cast(float, x[i] << 16);
    const float hi = __builtin_bit_cast(float, x[i] & 0xFFFF0000u);
    mag = __builtin_elementwise_maximum(mag, __builtin_elementwise_maximum(__builtin_fabsf(lo), __builtin_fabsf(hi)));
    f2 v;
    v[0] = lo;
    v[1] = hi;
    y[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
  }
  return y;
}

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

// One workgroup per (sequence, KV head, query tile of 16 * kSub rows), 1-D grid.  Wavefront w is
// query head 4g + w and takes all the tile's rows, as kSub MFMA column blocks of 16 queries, so
// every K and V fragment it reads from LDS feeds kSub products.  The query tile is the slowest
// index and runs backwards, so the workgroups with the most keys are dispatched first and the
// light ones fill the tail.  (Grouping a sequence's tiles on one XCD for L2 reuse was slower: it
// gives up that order and unbalances the XCDs when prompts differ in length.)
constexpr int kLdsPages = 256;  // block-table entries kept in LDS (4096 tokens); the rest from HBM
// Tables up to this width are copied to LDS whole (2 KiB; every launch shape still fits its
// workgroups per CU) and every page id is an LDS read.  With wider tables the ids past kLdsPages
// come from the table in memory, and the choice between the two becomes one flat load per step,
// whose completion every LDS wait of the step also waits for.
constexpr int kLdsTableMax = 512;
constexpr float kF16MaxBf16 = 65280.0f;  // the largest BF16 magnitude FP16 holds

// kChunk keys per step: 64 (two 32-key halves; 165 VGPRs with kSub = 2, 3 waves per SIMD) or 32
// (one half; fits 128 VGPRs, so 4 waves per SIMD, at twice the steps and barriers per key).
template <int kSub, int kChunk, bool kOutBf16, bool kTableLds>
__device__ __forceinline__ void prefill_attention_body(const PrefillParams &p, int32_t tiles) {
  constexpr int kHalves = kChunk / 32;  // 32-key halves per step
  constexpr int kVecs = kChunk / 32;    // 16-byte K (and V) vectors each thread stages per step
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kChunk * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[2][kChunk * kKStride];  // FP16 (BF16 in a second pass)
  constexpr int kPageSlots = kTableLds ? kLdsTableMax : kLdsPages;
  // Slots past the sequence's pages that a step's page-id lookup may reach (keys past the tile's
  // last query, up to two steps ahead): they hold the sequence's first page (valid; those keys
  // are masked), so the lookup needs no bounds test.
  constexpr int kTail = kTableLds ? 2 * kChunk / kBlock : 0;
  __shared__ int32_t s_pages[kPageSlots + kTail];
  __shared__ int32_t s_bad[kThreads / 64];
  __shared__ int32_t s_wide[2];  // step index whose staged V holds a value past FP16's range
  constexpr int kRows = 16 * kSub;  // query rows per workgroup

  const uint32_t pairs = gridDim.x / (uint32_t)tiles;  // batch * num_kv_heads
  const int tile = tiles - 1 - (int)(blockIdx.x / pairs);
  const uint32_t pair = blockIdx.x % pairs;  // b * num_kv_heads + g
  const int g = (int)(pair % (uint32_t)p.num_kv_heads);
  const int b = (int)(pair / (uint32_t)p.num_kv_heads);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int h = g * kGroup + (tid >> 6);  // one query head per wavefront
  const int r = lane & 15;                 // this lane's query column within each block of 16
  const int j = lane >> 4;                 // this lane's group of 8 keys / 8 dims

  // The prologue is a chain of dependent reads; each one is issued as soon as its address is
  // known: start_pos with cu_seqlens (b < batch by construction of the grid; the empty asm
  // consumes it before the early return, so the compiler cannot sink the load below it), the
  // tile's Q rows (inside the checked prompt) before the table pass.
  const int32_t start = p.start_pos[b];
  int32_t row0, n;
  const bool rows_ok = sequence_rows(p, b, row0, n);
  asm volatile("" ::"s"(start));
  if (!rows_ok) return;
  const int q_lo = tile * kRows;
  if (q_lo >= n) return;
  const int q_rows = min(kRows, n - q_lo);
  const int32_t *table = p.block_tables + (int64_t)b * p.max_blocks;
  auto out_elem = [&](int sub) -> int64_t {  // first of this lane's outputs of block `sub`
    return (((int64_t)row0 + q_lo + 16 * sub + r) * p.num_q_heads + h) * kHeadDim + 4 * j;
  };

  // Q^T as the B operand of S^T = K Q^T: query column r of block sub, dims 32 half + 8 j .. + 7.
  u32x4 qf[kSub][2];
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
    qf[sub][0] = qf[sub][1] = u32x4{0, 0, 0, 0};
    if (16 * sub + r < q_rows) {
      const u32x4 *src = reinterpret_cast<const u32x4 *>(p.q + out_elem(sub) - 4 * j);
      qf[sub][0] = src[j];
      qf[sub][1] = src[4 + j];
    }
  }

  // The whole sequence must be addressable: every page up to its last prompt position.
  int bad = !(start >= 0 && (int64_t)start + n <= (int64_t)p.max_blocks * kBlock);
  if (!bad) {
    const int need = (start + n + kBlock - 1) / kBlock;
    for (int e = tid; e < need + kTail; e += kThreads) {
      if (e < need) {
        const int32_t pg = table[e];
        bad |= pg < 0 || pg >= p.num_pages;
        if (e < kPageSlots) s_pages[e] = pg;
      } else {
        s_pages[e] = table[0];  // checked by the thread that reads entry 0 (need >= 1)
      }
    }
  }
  // Workgroup OR of `bad`: one flag per wavefront in LDS and one barrier, which also publishes
  // s_pages.  (__syncthreads_or would read the workgroup size from the dispatch arguments with
  // two dependent global loads and take three barriers.)
  const bool wave_bad = __builtin_amdgcn_ballot_w64(bad != 0) != 0;
  if (lane == 0) s_bad[tid >> 6] = wave_bad;
  if (tid < 2) s_wide[tid] = -1;
  __syncthreads();
  bad = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) bad |= s_bad[w];
  if (bad) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub)
      if (16 * sub + r < q_rows)
        for (int dt = 0; dt < 4; ++dt) store_row4<kOutBf16>(p.out, out_elem(sub) + 16 * dt, zero);
    return;
  }

  const int n_keys = start + q_lo + q_rows;  // keys 0 .. last query position of the tile
  const int n_chunks = (n_keys + kChunk - 1) / kChunk;

  // Staging: thread -> key (tid % kChunk) of the step and dims d0 .. d0 + 7 (and d0 + 32 .. d0 + 39
  // for 64-key steps) with d0 = 8 (tid / kChunk).
  const int st_key = tid & (kChunk - 1);
  const int st_dim = (tid / kChunk) * 8;
  // Page ids run one step ahead of the data: the id of step c + 1 is in hand when that step's K/V
  // loads issue, so no load inside a step waits on another.  A key past the tile's last query
  // reads the sequence's first page instead (validated, so in bounds); its V row is zeroed when
  // staged and its score is masked.
  auto page_of = [&](int c) -> int32_t {
    const int kp = c * kChunk + st_key;
    if constexpr (kTableLds) {
      // c <= n_chunks, so kp < n_keys + 2 kChunk: the index stays below need + kTail.
      return s_pages[kp >> 4];
    } else {
      const int e = kp < n_keys ? kp >> 4 : 0;
      return e < kLdsPages ? s_pages[e] : table[e];
    }
  };
  struct Rows {
    u32x4 k[kVecs], v[kVecs];
  };
  // This thread's row of a page (KV head g, token slot, dims) sits at the same offset inside every
  // page (a step spans whole pages), so a step's address is one page-stride product away.
  static_assert(kChunk % kBlock == 0, "steps cover whole pages");
  // Page ids are validated (0 <= id < num_pages), so the offset is one unsigned 32 x 32 -> 64-bit
  // multiply-add.
  const uint32_t page_bytes = (uint32_t)p.num_kv_heads * kBlock * kHeadDim * sizeof(uint16_t);
  const int64_t row_elems = ((int64_t)g * kBlock + (st_key & (kBlock - 1))) * kHeadDim + st_dim;
  const char *const k_row = reinterpret_cast<const char *>(p.k_pool + row_elems);
  const char *const v_row = reinterpret_cast<const char *>(p.v_pool + row_elems);
  auto load_step = [&](int c, int32_t pg, Rows &x) {
    const uint64_t off = (uint64_t)(uint32_t)pg * page_bytes;
#pragma unroll
    for (int e = 0; e < kVecs; ++e) {
      x.k[e] = *reinterpret_cast<const u32x4 *>(k_row + off + 64 * e);
      x.v[e] = *reinterpret_cast<const u32x4 *>(v_row + off + 64 * e);
    }
  };
  // kWide = false: V is staged as FP16, and a step whose V holds a magnitude past FP16's largest
  // finite value marks itself in s_wide (the flag holds the step index, so flags
  // of earlier steps never need clearing).  kWide = true: V is staged as BF16.
  auto stage = [&](int c, int buf, Rows &x, auto wide_tag) {
    constexpr bool kWide = decltype(wide_tag)::value;
    if (c * kChunk + kChunk > n_keys) {  // the last step only: no stale NaN reaches V
      if (c * kChunk + st_key >= n_keys)
#pragma unroll
        for (int e = 0; e < kVecs; ++e) x.v[e] = u32x4{0, 0, 0, 0};
    }
    float mag = 0.0f;
#pragma unroll
    for (int e = 0; e < kVecs; ++e) {
      *reinterpret_cast<u32x4 *>(&s_k[buf][st_key * kKStride + st_dim + 32 * e]) = x.k[e];
      *reinterpret_cast<u32x4 *>(&s_v[buf][st_key * kKStride + st_dim + 32 * e]) =
          kWide ? x.v[e] : bf16x8_to_f16x8(x.v[e], mag);
    }
    if (!kWide && !(mag <= kF16MaxBf16)) s_wide[buf] = c;
  };

  // Per column block: output tile, softmax anchor (log2 units, shared by the 4 lanes of a query,
  // less the weight shift; it moves only when a score outgrows the headroom, so most steps leave
  // the accumulators alone) and the denominator (an MFMA accumulator, the same in all 4 rows).
  f32x4 o[kSub][4];
  f32x4 lsum[kSub];
  float m[kSub];
  // Every weight carries an extra factor 2^7 (numerator and denominator alike, so the output is
  // unchanged): in FP16, weights down to 2^-21 of the anchor's stay normal numbers (unscaled,
  // everything below 2^-14 would be subnormal and below 2^-25 zero).  The anchor moves when a
  // score lies more than 8 (log2 units) above it, so every weight is at most 2^(8 + 7) = 32768,
  // finite in FP16 (largest 65504).  The test takes each lane's largest raw score as soon as the
  // score products are done, off the exponentials' path.
  constexpr float kShift = 7.0f;              // log2 of the weight factor
  constexpr float kLimit = 8.0f + kShift;     // largest exponent of a weight
  const u32x4 kOnes = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};     // BF16 1.0 x 8
  const u32x4 kOnesF16 = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};  // FP16 1.0 x 8
  const float c_log2 = p.score_log2;
  const int first_q = start + q_lo;  // smallest query position of the tile

  // One pass over the tile's keys.  kWide = false: FP16 V and weights; returns whether a step met
  // a V value past FP16's range (workgroup-uniform), in which case the caller runs the tile again
  // with kWide = true: BF16 V and weights carried as hi + lo BF16 pairs.  (Two passes one after
  // the other rather than a branch per step: with both product flavours inside the loop body the
  // kernel no longer fits its registers.)
  auto run = [&](auto wide_tag) -> bool {
    constexpr bool kWide = decltype(wide_tag)::value;
#pragma unroll
    for (int sub = 0; sub < kSub; ++sub) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[sub][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      lsum[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
      m[sub] = -INFINITY;
    }
    Rows rows;
    load_step(0, page_of(0), rows);
    int32_t pg_next = page_of(1);
    stage(0, 0, rows, wide_tag);
    __syncthreads();
    bool any_wide = false;

    // One step; `buf` is a compile-time constant at both call sites (the loop is unrolled by two),
    // so every LDS address of the step is a register base plus an immediate offset.
    auto step = [&](int c, auto buf_tag) {
      constexpr int buf = decltype(buf_tag)::value;
      const bool more = c + 1 < n_chunks;
      if (more) {  // in flight while this step computes
        load_step(c + 1, pg_next, rows);
        pg_next = page_of(c + 2);
      }

      // S^T for the four 16-key tiles of the step (half hs, tile t), every column block.
      f32x4 s[kSub][kHalves][2];
#pragma unroll
      for (int hs = 0; hs < kHalves; ++hs)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int key_row = 32 * hs + 8 * (r >> 2) + 4 * t + (r & 3);
          const uint16_t *krow = &s_k[buf][key_row * kKStride + 8 * j];
          const u32x4 k0 = *reinterpret_cast<const u32x4 *>(krow);
          const u32x4 k1 = *reinterpret_cast<const u32x4 *>(krow + 32);
#pragma unroll
          for (int sub = 0; sub < kSub; ++sub) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k0), as_bf16x8(qf[sub][0]), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k1), as_bf16x8(qf[sub][1]), acc, 0, 0, 0);
            s[sub][hs][t] = acc;
          }
        }

      // Causal mask, only on steps that reach past the tile's first query.
      if (c * kChunk + kChunk - 1 > first_q) {
#pragma unroll
        for (int sub = 0; sub < kSub; ++sub) {
          // this lane holds keys c * kChunk + 8 j + 32 hs + 4 t + i for query first_q + 16 sub + r
          const int room = first_q + 16 * sub + r - (c * kChunk + 8 * j);
#pragma unroll
          for (int hs = 0; hs < kHalves; ++hs)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (32 * hs + 4 * t + i > room) s[sub][hs][t][i] = -INFINITY;
        }
      }

      // Anchor test: does a score of the block, scaled, exceed the anchor by more than the limit
      // (always so on the tile's first step, where the anchor is -inf)?  The exact row maximum is
      // taken only on the rare step that moves the anchor.
      // (IEEE maximum, NaN-propagating: v_maximum3 needs no quieting of its inputs, unlike fmaxf.)
      bool over = false;
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub) {
        float smax = s[sub][0][0][0];
#pragma unroll
        for (int e = 1; e < 8 * kHalves; ++e)
          smax = __builtin_elementwise_maximum(smax, s[sub][e >> 3][(e >> 2) & 1][e & 3]);
        over |= __builtin_fmaf(smax, c_log2, -m[sub]) > kLimit;  // NaN (both -inf) is false
      }
      if (__builtin_amdgcn_ballot_w64(over)) {  // wave-uniform
        const bool first = c == 0;
#pragma unroll
        for (int sub = 0; sub < kSub; ++sub) {
          float mx = -INFINITY;
#pragma unroll
          for (int hs = 0; hs < kHalves; ++hs)
#pragma unroll
            for (int t = 0; t < 2; ++t)
              mx = fmaxf(mx, fmaxf(fmaxf(s[sub][hs][t][0], s[sub][hs][t][1]),
                                   fmaxf(s[sub][hs][t][2], s[sub][hs][t][3])));
          mx = wave_xor_max(mx, 16);
          mx = wave_xor_max(mx, 32);
          // scale > 0; finite: key 0 is visible to every query in step 0.  The shift goes in as
          // -4 - 2 - 1, inline constants: a 7.0 literal would take a register the loop lacks.
          static_assert(kShift == 4.0f + 2.0f + 1.0f, "weight shift");
          mx = __builtin_fmaf(mx, c_log2, -4.0f) - 2.0f - 1.0f;
          const float m_new = fmaxf(m[sub], mx);
          if (!first) {  // on a tile's first step the sums are still zero: nothing to rescale
            const float alpha = __builtin_amdgcn_exp2f(m[sub] - m_new);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) o[sub][dt] *= alpha;
            lsum[sub] *= alpha;
          }
          m[sub] = m_new;
        }
      }

      // Weights with the current anchor: 2^(x - m), at most 2^15; the FP16 pass packs them to FP16
      // (nearest even) as they are made.
      float pe[kSub][kHalves][8];
      u32x4 pw[kSub][kHalves];
#pragma unroll
      for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
        for (int hs = 0; hs < kHalves; ++hs) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pe[sub][hs][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][hs][e >> 2][e & 3], c_log2, -m[sub]));
          if constexpr (!kWide) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              f2 w2;
              w2[0] = pe[sub][hs][2 * e];
              w2[1] = pe[sub][hs][2 * e + 1];
              pw[sub][hs][e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(w2, h2));
            }
          }
        }

      // O^T += V^T P^T for the step.  kWide: the weights as hi + lo BF16 pairs against BF16 V;
      // otherwise as FP16 against the FP16 staged V.
      auto pv = [&](auto wide_tag) {
        constexpr bool kWide = decltype(wide_tag)::value;
#pragma unroll
        for (int hs = 0; hs < kHalves; ++hs) {
          // V^T fragments straight from the row-major staged rows with the transposing LDS read:
          // within each 16-lane group, lane L of the read receives element L % 4 of the 4-element
          // rows read by lanes L / 4 + 4 i, i = 0..3.  So lane M reads row key0 + M / 4 at dims
          // 4 (M % 4) .. + 3 of the tile, and lane (j, r) ends up with keys key0 .. key0 + 3 of
          // dim r; two reads (key0 = 32 hs + 8 j and + 4) give the 8 keys of the A operand.
          u32x4 vf[4];
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const uint16_t *vrow = &s_v[buf][(32 * hs + 8 * j + (r >> 2)) * kKStride + 16 * dt + 4 * (r & 3)];
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)vrow);
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16 *)(vrow + 4 * kKStride));
            const u32x2 a = __builtin_bit_cast(u32x2, lo), b2v = __builtin_bit_cast(u32x2, hi);
            vf[dt] = u32x4{a[0], a[1], b2v[0], b2v[1]};
          }
#pragma unroll
          for (int sub = 0; sub < kSub; ++sub) {
            if constexpr (!kWide) {
              // The weights enter the product as FP16 (11 significant bits, round to nearest even),
              // packed when they were computed.
              const u32x4 ph = pw[sub][hs];
              // One 16-dim tile at a time; the denominator rides along as an all-ones tile (every
              // row of it is the query's sum of the same FP16 weights).
#pragma unroll
              for (int dt = 0; dt < 4; ++dt)
                o[sub][dt] =
                    __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(vf[dt]), as_f16x8(ph), o[sub][dt], 0, 0, 0);
              lsum[sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(kOnesF16), as_f16x8(ph), lsum[sub], 0, 0, 0);
            } else {
              // Each weight as a sum of two BF16 values (hi + lo, ~16 significant bits).
              u32x4 ph, pl;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                f2 w2;
                w2[0] = pe[sub][hs][2 * e];
                w2[1] = pe[sub][hs][2 * e + 1];
                const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(w2, b2));
                ph[e] = hi;
                f2 rest;  // exact in FP32: each value minus its own BF16 rounding
                rest[0] = w2[0] - __builtin_bit_cast(float, hi << 16);
                rest[1] = w2[1] - __builtin_bit_cast(float, hi & 0xFFFF0000u);
                pl[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rest, b2));
              }
#pragma unroll
              for (int dt = 0; dt < 4; ++dt) {
                o[sub][dt] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf[dt]), as_bf16x8(ph), o[sub][dt], 0, 0, 0);
                o[sub][dt] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf[dt]), as_bf16x8(pl), o[sub][dt], 0, 0, 0);
              }
              lsum[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kOnes), as_bf16x8(ph), lsum[sub], 0, 0, 0);
              lsum[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kOnes), as_bf16x8(pl), lsum[sub], 0, 0, 0);
            }
          }
        }
      };
      if constexpr (!kWide) any_wide |= s_wide[buf] == c;  // workgroup-uniform
      pv(wide_tag);

      if (more) stage(c + 1, buf ^ 1, rows, wide_tag);
      __syncthreads();
    };
    for (int c = 0; c < n_chunks; c += 2) {
      step(c, std::integral_constant<int, 0>{});
      if (c + 1 < n_chunks) step(c + 1, std::integral_constant<int, 1>{});
    }
    return any_wide;
  };
  if (run(std::false_type{})) run(std::true_type{});

#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
    const float inv = 1.0f / lsum[sub][0];
    if (16 * sub + r < q_rows)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) store_row4<kOutBf16>(p.out, out_elem(sub) + 16 * dt, o[sub][dt] * inv);
  }
}


template <int kSub, bool kOutBf16, bool kTableLds>
__global__ __launch_bounds__(kThreads) void prefill_attention_kernel(PrefillParams p, int32_t tiles) {
  prefill_attention_body<kSub, 64, kOutBf16, kTableLds>(p, tiles);
}

template <int kSub, bool kOutBf16, bool kTableLds>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void prefill_attention_kernel_k32(
    PrefillParams p, int32_t tiles) {
  prefill_attention_body<kSub, 32, kOutBf16, kTableLds>(p, tiles);
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

template <int kSub, bool kK32, bool kTableLds>
hipError_t launch_attention_table(const PrefillParams &p, bool out_bf16, hipStream_t stream) {
  const int64_t tiles = ((int64_t)p.max_prompt_len + 16 * kSub - 1) / (16 * kSub);
  const int64_t blocks = tiles * p.batch * p.num_kv_heads;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(kThreads);
  if constexpr (kK32) {
    if (out_bf16) hipLaunchKernelGGL((prefill_attention_kernel_k32<kSub, true, kTableLds>), grid, block, 0, stream, p, (int32_t)tiles);
    else hipLaunchKernelGGL((prefill_attention_kernel_k32<kSub, false, kTableLds>), grid, block, 0, stream, p, (int32_t)tiles);
  } else {
    if (out_bf16) hipLaunchKernelGGL((prefill_attention_kernel<kSub, true, kTableLds>), grid, block, 0, stream, p, (int32_t)tiles);
    else hipLaunchKernelGGL((prefill_attention_kernel<kSub, false, kTableLds>), grid, block, 0, stream, p, (int32_t)tiles);
  }
  return hipGetLastError();
}

template <int kSub, bool kK32>
hipError_t launch_attention(const PrefillParams &p, bool out_bf16, hipStream_t stream) {
  if (p.max_blocks <= kLdsTableMax) return launch_attention_table<kSub, kK32, true>(p, out_bf16, stream);
  return launch_attention_table<kSub, kK32, false>(p, out_bf16, stream);
}

// Two 16-query blocks per wavefront halve the LDS traffic, staging and barriers per score (16
// prompts x 512: 55.6 vs 64.1 us) but halve the workgroup count; below two workgroups per compute
// unit (one 512-token prompt: 128 workgroups) one block per wavefront is faster (11.8 vs 15.5 us).
// From four workgroups per compute unit the grid keeps every SIMD busy and 32-key steps at 4
// waves per SIMD hide more latency than 64-key steps at 3 (16 x 512: 46.6-48.4 vs 51.1-51.7 us);
// with fewer workgroups the longer chain of steps costs more (six chunked prompts, 3 per CU:
// 39.2 vs 37.1 us; one 512-token prompt 12.5 vs 10.7 us).
hipError_t launch_prefill_attention(const PrefillParams &p, bool out_bf16, int32_t num_cus, hipStream_t stream) {
  const int64_t tiles2 = ((int64_t)p.max_prompt_len + 31) / 32;
  const int64_t groups2 = tiles2 * p.batch * p.num_kv_heads;
  if (groups2 >= 4 * (int64_t)num_cus) return launch_attention<2, true>(p, out_bf16, stream);
  if (groups2 >= 2 * (int64_t)num_cus) return launch_attention<2, false>(p, out_bf16, stream);
  return launch_attention<1, false>(p, out_bf16, stream);
}

}  // namespace pkv
