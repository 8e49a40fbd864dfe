// Paged decode attention for gfx950: one workgroup per (sequence, KV head, context partition).
//
// What is computed ("6 Hours of YouTube and 85 handtyped pages of notes on LLM Inference", section "What works so far"; "The prefill path: flowing the entire prompt at once",
// sections "Per-head attention scores and GQA" and "causalMask and online softmax"): for the
// four query heads that share KV head g, scores s_t = scale * <q_h, K_t> over the sequence's
// cached tokens, softmax over t, and the softmax-weighted sum of the V rows.  The pages' decode
// kernel streams the non-contiguous pages directly with an FP32 online softmax, gathering no
// contiguous prefix and storing no scores; so do these.
//
// Design for CDNA4 (64-lane wavefronts, DPP cross-lane ops, v_dot2 on BF16 pairs, MFMA):
//   * One workgroup serves the whole GQA group of a KV head, so each K/V byte is read from HBM
//     exactly once for all four query heads.
//   * 4 wavefronts per workgroup; wavefront w takes pages w, w+4, w+8, ... of the partition and
//     keeps its own softmax state, so the main loop has no barriers.  The four states are
//     merged in LDS at the end with the pairwise (max, sum) rule.
//   * Two flavours of the per-page arithmetic.  The vector-ALU kernel (paged_decode_kernel, used
//     for unsplit launches with at least one workgroup per compute unit, where HBM is the bound):
//     lane = 8 * token + 16-byte chunk, so a wavefront loads a 2 KiB page of one KV head with two
//     fully coalesced 16-byte loads per lane; QK with v_dot2_f32_bf16 and three DPP adds, PV with
//     FMAs.  The matrix-core kernel (paged_decode_mfma_kernel, every split launch and small
//     batches, where the chain of dependent latencies inside a wavefront is the bound): two pages
//     per step, both contractions on v_mfma_f32_16x16x32_bf16, only the softmax on the VALU.
//   * Softmax in log2 units with a lazily moved anchor: scores are compared with the anchor
//     plus 8; only when a page exceeds it does the wavefront recompute the anchor and rescale
//     its accumulators (the result is independent of the anchor; fp32 holds 2^8 of headroom).
//   * Long contexts with few (sequence, KV head) pairs are cut into partitions.  Each publishes
//     its (max, sum, partial output) per query head to the workspace with device-scope atomic
//     swaps and counts itself on a per-(sequence, KV head) counter; the partition that arrives
//     last swaps the others' partials out (leaving zeros) and writes the output, so the split
//     needs no second kernel.  Workgroup ids are partition-major, so every partition index is
//     spread over all 8 XCDs.
// Block-table entries are read straight into a VGPR (one entry per lane) and moved to scalar
// registers with v_readlane; every entry is range-checked before a page is touched.
#include <math.h>

#include "pkv_internal.h"

namespace pkv {
namespace {


constexpr int kThreads = kWaves * 64;
constexpr float kAnchorHeadroom = 8.0f;  // log2 units
// s_waitcnt immediate (gfx9 encoding): vmcnt(0), expcnt and lgkmcnt left alone.
constexpr int kWaitVmcnt0 = 0x0F70;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// DPP controls (CDNA encoding).
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int kRowRor8 = 0x128;       // rotate each 16-lane row by 8

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, true));
}

// Sum over the 8 lanes of a token (lanes 8t..8t+7); every lane receives the total.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  x += dpp<kRowHalfMirror>(x);
  return x;
}

__device__ __forceinline__ float fmax_plain(float a, float b) { return a > b ? a : b; }

// Maximum over the whole wavefront of a value that is already uniform within 8-lane groups:
// fold the two groups of each 16-lane row with DPP, then take the four rows' values with
// readlane (no LDS permute).  The result is wave-uniform.
__device__ __forceinline__ float wave_max_of_groups(float x) {
  x = fmax_plain(x, dpp<kRowRor8>(x));
  const int b = __builtin_bit_cast(int, x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return fmax_plain(fmax_plain(r0, r1), fmax_plain(r2, r3));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

struct WaveState {
  float acc[kGroup][8];  // un-normalised sum of p * V for dims 8*chunk..8*chunk+7
  float lsum[kGroup];    // sum of p over this lane's token slots
  float m[kGroup];       // softmax anchor (log2 units), uniform across the wavefront
  float thr[kGroup];     // anchor + headroom: a score above it moves the anchor (uniform)
};

// K and V of one page of one KV head: tokens 0..7 in ka/va, tokens 8..15 in kb/vb.
struct PageRegs {
  uint4 ka, kb, va, vb;
};

__device__ __forceinline__ float uniform(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}


// One page.  `valid` is the number of its tokens inside the context (only the sequence's last
// page can have fewer than 16; that one is processed with kPartial = true).
template <bool kPartial>
__device__ __forceinline__ void process_page(WaveState &st, const uint32_t (&qv)[kGroup][4], PageRegs r, int tok,
                                             int valid, float c_log2) {
  float sa[kGroup], sb[kGroup];
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    float x = dot2_bf16(qv[h][0], r.ka.x, 0.0f);
    x = dot2_bf16(qv[h][1], r.ka.y, x);
    x = dot2_bf16(qv[h][2], r.ka.z, x);
    x = dot2_bf16(qv[h][3], r.ka.w, x);
    float y = dot2_bf16(qv[h][0], r.kb.x, 0.0f);
    y = dot2_bf16(qv[h][1], r.kb.y, y);
    y = dot2_bf16(qv[h][2], r.kb.z, y);
    y = dot2_bf16(qv[h][3], r.kb.w, y);
    // Scores in log2 units.  Scaling before the anchor subtraction (instead of one fma) makes
    // p exactly 1 for the token that set the anchor.
    sa[h] = sum8(x) * c_log2;
    sb[h] = sum8(y) * c_log2;
  }
  if (kPartial) {
    // Tokens past the context are never used: their score becomes -inf (p = 0) and their V
    // registers are zeroed so that stale or NaN slot contents cannot reach the accumulators.
    const bool a_ok = tok < valid;
    const bool b_ok = tok + 8 < valid;
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      sa[h] = a_ok ? sa[h] : -INFINITY;
      sb[h] = b_ok ? sb[h] : -INFINITY;
    }
    if (!a_ok) r.va = make_uint4(0u, 0u, 0u, 0u);
    if (!b_ok) r.vb = make_uint4(0u, 0u, 0u, 0u);
  }

  float smax[kGroup];
  uint64_t over = 0;
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    smax[h] = fmax_plain(sa[h], sb[h]);
    over |= __builtin_amdgcn_ballot_w64(smax[h] > st.thr[h]);
  }
  if (over != 0) {  // wave-uniform and rare: the anchor of some head has to move up
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      const float m_new = fmax_plain(st.m[h], wave_max_of_groups(smax[h]));
      const float alpha = __builtin_amdgcn_exp2f(st.m[h] - m_new);  // 0 on the first page
#pragma unroll
      for (int d = 0; d < 8; ++d) st.acc[h][d] *= alpha;
      st.lsum[h] *= alpha;
      st.m[h] = m_new;
      st.thr[h] = uniform(m_new + kAnchorHeadroom);
    }
  }

#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    sa[h] = __builtin_amdgcn_exp2f(sa[h] - st.m[h]);
    sb[h] = __builtin_amdgcn_exp2f(sb[h] - st.m[h]);
    st.lsum[h] += sa[h] + sb[h];
  }
  const uint32_t vw[8] = {r.va.x, r.va.y, r.va.z, r.va.w, r.vb.x, r.vb.y, r.vb.z, r.vb.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a_lo = bf16_lo(vw[j]), a_hi = bf16_hi(vw[j]);
    const float b_lo = bf16_lo(vw[4 + j]), b_hi = bf16_hi(vw[4 + j]);
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      st.acc[h][2 * j] = __builtin_fmaf(sa[h], a_lo, st.acc[h][2 * j]);
      st.acc[h][2 * j + 1] = __builtin_fmaf(sa[h], a_hi, st.acc[h][2 * j + 1]);
      st.acc[h][2 * j] = __builtin_fmaf(sb[h], b_lo, st.acc[h][2 * j]);
      st.acc[h][2 * j + 1] = __builtin_fmaf(sb[h], b_hi, st.acc[h][2 * j + 1]);
    }
  }
}

__device__ __forceinline__ uint4 load16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// K/V pages are read exactly once per launch: non-temporal loads (the `nt` policy) stream them
// past the caches, which measured ~13% more read bandwidth than default-policy loads here.
__device__ __forceinline__ uint4 load16_stream(const uint16_t *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Issue the four 16-byte loads of one page (K first: it is consumed first).
__device__ __forceinline__ void load_page(PageRegs &r, const uint16_t *kbase, const uint16_t *vbase, int64_t off) {
  r.ka = load16_stream(kbase + off);
  r.kb = load16_stream(kbase + off + 512);
  r.va = load16_stream(vbase + off);
  r.vb = load16_stream(vbase + off + 512);
}

// Context length of sequence b: context_lens[b], or, for the fused decode step, positions[b] + 1
// (a position outside the block table gives an invalid length, hence a zero output row).
template <bool kFused>
__device__ __forceinline__ int context_length(const DecodeParams &p, int b) {
  if (!kFused) return p.context_lens[b];
  const int pos = p.positions[b];
  return (pos >= 0 && pos < p.max_blocks * kBlock) ? pos + 1 : -1;
}

// The arguments the prologue's first loads depend on lead the kernel signature as scalars, so the
// hardware preloads them into SGPRs before the wavefront starts (the build asks for 14 dwords of
// preload): the table row, context or position, q and the new row are then requested by the very
// first instructions instead of behind a kernel-argument load.  The struct follows for the rest.
#define PKV_PRELOADED_ARGS                                                                           \
  const int32_t *pre_tables, const int32_t *pre_lens, const uint16_t *pre_q, const uint16_t *pre_k_new, \
      const uint16_t *pre_v_new, int32_t pre_max_blocks, int32_t pre_kv_heads, int32_t pre_batch,     \
      int32_t pre_part_pages
#define PKV_TAKE_PRELOADED_ARGS(p)   \
  do {                               \
    (p).block_tables = pre_tables;   \
    if (kFused) (p).positions = pre_lens; \
    else (p).context_lens = pre_lens; \
    (p).q = pre_q;                   \
    (p).k_new = pre_k_new;           \
    (p).v_new = pre_v_new;           \
    (p).max_blocks = pre_max_blocks; \
    (p).num_kv_heads = pre_kv_heads; \
    (p).num_q_heads = kGroup * pre_kv_heads; \
    (p).batch = pre_batch;           \
    (p).part_pages = pre_part_pages; \
  } while (0)

// Partitions one merging workgroup reads at once (the swaps of a chunk go out together).
constexpr int kMergeChunk = 16;

// Ends a workgroup once its wavefronts' states are combined: thread (h, d) holds, for query head
// 4 g + h and dim d, the partition's anchor M (log2 units), denominator Ls and un-normalised output
// O; any_bad is set when the partition met an invalid table entry.  Unsplit, or a sequence whose
// pages fit one partition: out = O / Ls (zeros when any_bad).  Otherwise the partition publishes
// (M, Ls or -1, O) with device-scope atomic swaps, counts itself on the (sequence, KV head)
// counter, and the partition that arrives last merges all of them with the pairwise (max, sum) rule
// ("The prefill path: flowing the entire prompt at once", section "causalMask and online
// softmax"): M* = max M_i, out = sum 2^(M_i - M*) O_i / sum 2^(M_i - M*) Ls_i, or zeros when a
// partition marked itself invalid (a NaN in a partition's keys or values reaches the output as it
// does unsplit).  The merging partition reads the partials with swaps that
// leave zeros behind and resets the counter, so the workspace is all-zero again when the launch
// ends.  Swaps stand in for plain stores and loads because a device-scope atomic's round trip
// (about 0.4 us on MI355X) is well under that of a device-coherent store's acknowledgement or a
// device-coherent load (about 1 us), and on a split step the publish, count and read-back are
// the tail of the critical path.
template <bool kSplit, bool kOutBf16>
__device__ __forceinline__ void finish_group(const DecodeParams &p, int b, int g, int part, int n_pages, float M,
                                             float O, float Ls, bool any_bad) {
  __shared__ uint32_t s_ticket;
  const int h = threadIdx.x >> 6;
  const int d = threadIdx.x & 63;
  const int qh = g * kGroup + h;
  const int64_t o_idx = ((int64_t)b * p.num_q_heads + qh) * kHeadDim + d;
  auto store_out = [&](float r) {
    if (kOutBf16) static_cast<uint16_t *>(p.out)[o_idx] = f32_to_bf16_rne(r);
    else static_cast<float *>(p.out)[o_idx] = r;
  };
  const int n_parts = kSplit ? (n_pages + p.part_pages - 1) / p.part_pages : 1;
  if (n_parts <= 1) {  // workgroup-uniform
    store_out(any_bad ? 0.0f : O / Ls);
    return;
  }
  const int64_t slot0 = ((int64_t)b * p.num_q_heads + qh) * p.num_parts;
  const int64_t slot = slot0 + part;
  __hip_atomic_exchange(p.part_o + slot * kHeadDim + d, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (d == 0) {
    __hip_atomic_exchange(p.part_ml + slot * 2, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_exchange(p.part_ml + slot * 2 + 1, any_bad ? -1.0f : Ls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Count the partition only once its swaps are acknowledged: a partition on another XCD then
  // finds them with its own device-scope swaps, and no whole-L2 write-back or invalidation is
  // needed.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  uint32_t *ctr = p.counters + ((int64_t)b * p.num_kv_heads + g) * kCounterStride;
  if (threadIdx.x == 0) s_ticket = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_ticket != (uint32_t)(n_parts - 1)) return;  // workgroup-uniform
  if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  float *ml = p.part_ml + slot0 * 2;
  float *po = p.part_o + slot0 * kHeadDim + d;
  float Mg = -INFINITY, Og = 0.0f, Lg = 0.0f;
  bool bad = false;
  for (int i0 = 0; i0 < n_parts; i0 += kMergeChunk) {
    float mv[kMergeChunk], lv[kMergeChunk], ov[kMergeChunk];
    // Lane 2 u + j takes word j of partition i0 + u's (max, denominator) pair: the chunk's
    // pairs are contiguous, so one swap instruction reads (and zeroes) all of them.
    float mlw = 0.0f;
    if (d < 2 * kMergeChunk && i0 + (d >> 1) < n_parts)
      mlw = __hip_atomic_exchange(ml + 2 * i0 + d, 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      const int i = i0 + u;  // wave-uniform
      if (i < n_parts)
        ov[u] = __hip_atomic_exchange(po + (int64_t)i * kHeadDim, 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      mv[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mlw), 2 * u));
      lv[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mlw), 2 * u + 1));
    }
    float Mc = Mg;
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u)
      if (i0 + u < n_parts) Mc = fmax_plain(Mc, mv[u]);
    const float rescale = __builtin_amdgcn_exp2f(Mg - Mc);  // 0 for the first chunk
    Og *= rescale;
    Lg *= rescale;
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      if (i0 + u < n_parts) {
        const float e = __builtin_amdgcn_exp2f(mv[u] - Mc);
        Og = __builtin_fmaf(e, ov[u], Og);
        Lg = __builtin_fmaf(e, lv[u], Lg);
        bad |= lv[u] < 0.0f;  // -1: an invalid table entry (a NaN sum propagates, as unsplit)
      }
    }
    Mg = Mc;
  }
  store_out(bad ? 0.0f : Og / Lg);
}

template <bool kSplit, bool kOutBf16, bool kFused>
__global__ __launch_bounds__(kThreads) void paged_decode_kernel(PKV_PRELOADED_ARGS, DecodeParams p) {
  PKV_TAKE_PRELOADED_ARGS(p);
  __shared__ float s_acc[kWaves][4][kGroup][kHeadDim];  // [wave][16-lane row][head][dim]
  __shared__ float s_l[kWaves][4][kGroup];
  __shared__ float s_m[kWaves][kGroup];
  __shared__ int s_bad[kWaves];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Partition-major order: consecutive workgroup ids go to the 8 XCDs in turn, so with the
  // partition as the fast index (and 8 partitions) partition k would always land on XCD k, and the
  // XCD holding every sequence's first partition would do most of the work.  With the (sequence,
  // KV head) pair fast, each partition is spread over all XCDs.
  // Grid (KV head, sequence, partition): workgroups are dispatched x-fastest, so the linear order
  // is partition-major as described above, and no index needs a division.
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int part = blockIdx.z;
  const int qh0 = g * kGroup;  // first query head of the group

  const int p0 = part * p.part_pages;
  const int tok = lane >> 3;    // token within each half page
  const int chunk = lane & 7;   // 16-byte chunk of the row: dims 8*chunk .. 8*chunk+7

  // Reads whose addresses do not depend on the context length go out before it is known, so the
  // prologue is one round trip: this wavefront's table entries (lane k: logical page
  // p0 + wave + kWaves * k, read while it lies inside the sequence's table row), q, and in the
  // fused step the new token's K/V row.
  const int32_t *bt = p.block_tables + (int64_t)b * p.max_blocks;
  const int e_lane = p0 + wave + kWaves * lane;
  const int ids_row = e_lane < p.max_blocks ? bt[e_lane] : 0;
  uint32_t qv[kGroup][4];
  {
    const uint16_t *qb = p.q + ((int64_t)b * p.num_q_heads + qh0) * kHeadDim + chunk * 8;
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      const uint4 t = load16(qb + h * kHeadDim);
      qv[h][0] = t.x; qv[h][1] = t.y; qv[h][2] = t.z; qv[h][3] = t.w;
    }
  }
  uint4 knew = make_uint4(0u, 0u, 0u, 0u), vnew = knew;
  if (kFused) {
    const int64_t row = ((int64_t)b * p.num_kv_heads + g) * kHeadDim + chunk * 8;
    knew = load16(p.k_new + row);
    vnew = load16(p.v_new + row);
  }
  const int L = context_length<kFused>(p, b);
  const bool len_ok = L >= 0 && L <= p.max_blocks * kBlock;
  const int n_pages = len_ok ? (L + kBlock - 1) / kBlock : 0;
  const int p1 = min(p0 + p.part_pages, n_pages);
  // The parameter-struct fields used past the prologue are requested now too, so their scalar
  // loads share the prologue's round trip instead of taking one of their own after it.
  const int num_pages = p.num_pages;
  const float c_log2 = p.score_log2;
  const uint16_t *const k_pool = p.k_pool;
  const uint16_t *const v_pool = p.v_pool;
  asm volatile("" ::"s"(num_pages), "s"(c_log2), "s"(k_pool), "s"(v_pool));
  if (kSplit) {
    asm volatile("" ::"s"(p.out), "s"(p.part_o), "s"(p.part_ml), "s"(p.counters), "s"(p.num_parts));
  } else {
    asm volatile("" ::"s"(p.out));
  }
  if (kFused) asm volatile("" ::"s"(p.k_pool_w), "s"(p.v_pool_w));
  // Keep those reads above the branch below (the compiler would otherwise sink them past it,
  // behind the length read).
  asm volatile("" ::"v"(ids_row));
#pragma unroll
  for (int h = 0; h < kGroup; ++h) asm volatile("" ::"v"(qv[h][0]), "v"(qv[h][1]), "v"(qv[h][2]), "v"(qv[h][3]));
  if (kFused) asm volatile("" ::"v"(knew.x), "v"(knew.y), "v"(knew.z), "v"(knew.w), "v"(vnew.x), "v"(vnew.y), "v"(vnew.z), "v"(vnew.w));

  if (p0 >= p1) {
    // An empty partition has nothing to do; partition 0 is empty only for an empty or invalid
    // sequence, and writes the group's 4 x 64 zeros.
    if (kSplit && part != 0) return;
    const int64_t o = ((int64_t)b * p.num_q_heads + qh0) * kHeadDim + threadIdx.x;
    if (kOutBf16) static_cast<uint16_t *>(p.out)[o] = 0;
    else static_cast<float *>(p.out)[o] = 0.0f;
    return;
  }

  // Pages of this wavefront: local index k -> logical page p0 + wave + kWaves * k, k < n_w <= 64
  // (a partition holds at most kMaxPartitionPages pages).
  int n_w = (p1 - p0 - wave + kWaves - 1) / kWaves;
  if (n_w < 0) n_w = 0;
  // One table entry per lane, range-checked before any page is touched.
  const int ids = lane < n_w ? ids_row : 0;
  const bool bad = __builtin_amdgcn_ballot_w64(ids < 0 || ids >= num_pages) != 0;
  // The wavefront holding the sequence's last page (it always holds the new token).
  const bool holds_last = n_w > 0 && p1 == n_pages && p0 + wave + kWaves * (n_w - 1) == n_pages - 1;
  // Like pkv_kv_append, the fused append depends only on its own page entry: an invalid entry
  // elsewhere in the sequence zeroes the output but does not stop the append.
  const int last_id = holds_last ? __builtin_amdgcn_readlane(ids, n_w - 1) : -1;
  const bool do_append = kFused && last_id >= 0 && last_id < num_pages;
  if (bad) n_w = 0;
  const bool owns_last = n_w > 0 && holds_last;
  // q and the table entries must have landed before the first page load is issued (the page
  // addresses need the entries anyway).  Waiting here explicitly also tells the compiler that q
  // is resident inside the page loop, so the loop's waits only count the page loads in flight.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  WaveState st;
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
#pragma unroll
    for (int d = 0; d < 8; ++d) st.acc[h][d] = 0.0f;
    st.lsum[h] = 0.0f;
    st.m[h] = -INFINITY;
    st.thr[h] = -INFINITY;
  }

  const int64_t head_elems = (int64_t)kBlock * kHeadDim;
  const int64_t page_elems = (int64_t)p.num_kv_heads * head_elems;
  const uint16_t *kbase = k_pool + g * head_elems + lane * 8;
  const uint16_t *vbase = v_pool + g * head_elems + lane * 8;
  auto page_off = [&](int k) -> int64_t { return (int64_t)__builtin_amdgcn_readlane(ids, k) * page_elems; };

  // The sequence's last page can be partial (L % 16 != 0) and, in the fused step, receives the
  // new token.  The wavefront that owns it always takes it first, outside the pipelined loop, so
  // the loop only sees ordinary full pages and the fused and unfused kernels add up the pages in
  // the same order (their results are bit-identical).
  const int tail_valid = L - (n_pages - 1) * kBlock;
  const bool own_partial = owns_last;
  const int n_full = own_partial ? n_w - 1 : n_w;
  if (do_append) {
    // Append: the 8 lanes that hold the new token's slot write its K and V rows (16 B each) into
    // the pool.  The same rows replace that slot in registers below, so the attention never
    // depends on when these stores become visible.
    const int slot = tail_valid - 1;  // position % 16
    if (tok == (slot & 7)) {
      const int64_t dst = ((int64_t)last_id * p.num_kv_heads + g) * (kBlock * kHeadDim) + slot * kHeadDim + chunk * 8;
      *reinterpret_cast<uint4 *>(p.k_pool_w + dst) = knew;
      *reinterpret_cast<uint4 *>(p.v_pool_w + dst) = vnew;
    }
  }
  // Swap the new token's row into the last page's registers (fused step only).
  auto with_new_token = [&](PageRegs r) -> PageRegs {
    if (kFused) {
      const int slot = tail_valid - 1;
      const bool hi = slot >= 8;
      const bool mine = tok == (slot & 7);
      if (mine && !hi) { r.ka = knew; r.va = vnew; }
      if (mine && hi) { r.kb = knew; r.vb = vnew; }
    }
    return r;
  };

  // Three page buffers: two pages in flight while one is computed.  The pipelined loop is only
  // entered from a path where both prefetches were issued unconditionally and it only runs while
  // every load it issues exists, so the compiler's waits count exactly the newer loads in flight
  // (a merge with a path that skipped a prefetch would make it wait for a whole page instead).
  PageRegs b0, b1, b2;
  if (own_partial) load_page(b2, kbase, vbase, page_off(n_w - 1));
  if (n_full >= 5) {
    int k = 0;
    load_page(b0, kbase, vbase, page_off(0));
    load_page(b1, kbase, vbase, page_off(1));
    if (own_partial) process_page<true>(st, qv, with_new_token(b2), tok, tail_valid, c_log2);
    for (; k + 4 < n_full; k += 3) {
      load_page(b2, kbase, vbase, page_off(k + 2));
      process_page<false>(st, qv, b0, tok, kBlock, c_log2);
      load_page(b0, kbase, vbase, page_off(k + 3));
      process_page<false>(st, qv, b1, tok, kBlock, c_log2);
      load_page(b1, kbase, vbase, page_off(k + 4));
      process_page<false>(st, qv, b2, tok, kBlock, c_log2);
    }
    // At most four full pages remain: k (in b0) and k + 1 (in b1) are already issued.
    const int rem = n_full - k;
    if (rem >= 3) load_page(b2, kbase, vbase, page_off(k + 2));
    if (rem >= 1) process_page<false>(st, qv, b0, tok, kBlock, c_log2);
    if (rem >= 4) load_page(b0, kbase, vbase, page_off(k + 3));
    if (rem >= 2) process_page<false>(st, qv, b1, tok, kBlock, c_log2);
    if (rem >= 3) process_page<false>(st, qv, b2, tok, kBlock, c_log2);
    if (rem >= 4) process_page<false>(st, qv, b0, tok, kBlock, c_log2);
  } else if (n_w > 0) {
    // Short chain (at most four full pages): every load is issued before any page is processed,
    // so the wave pays one memory latency, not one per buffer turn.  The four full-page loads are
    // unconditional (slots past the wave's pages read pool page 0: table lanes past n_w hold 0;
    // in bounds and never processed), so the issue order, and with it every wait, is the same on
    // every path.
    PageRegs b3, b4;
    load_page(b0, kbase, vbase, page_off(0));
    load_page(b1, kbase, vbase, page_off(1));
    load_page(b3, kbase, vbase, page_off(2));
    load_page(b4, kbase, vbase, page_off(3));
    if (own_partial) process_page<true>(st, qv, with_new_token(b2), tok, tail_valid, c_log2);
    if (n_full >= 1) process_page<false>(st, qv, b0, tok, kBlock, c_log2);
    if (n_full >= 2) process_page<false>(st, qv, b1, tok, kBlock, c_log2);
    if (n_full >= 3) process_page<false>(st, qv, b3, tok, kBlock, c_log2);
    if (n_full >= 4) process_page<false>(st, qv, b4, tok, kBlock, c_log2);
  }

  // Wavefront -> LDS.  Fold token t and t+1 (the two halves of each 16-lane row) first.
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
#pragma unroll
    for (int d = 0; d < 8; ++d) st.acc[h][d] += dpp<kRowRor8>(st.acc[h][d]);
    st.lsum[h] += dpp<kRowRor8>(st.lsum[h]);
  }
  const int row = lane >> 4;
  if ((lane & 8) == 0) {
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      float4 *dst = reinterpret_cast<float4 *>(&s_acc[wave][row][h][chunk * 8]);
      dst[0] = make_float4(st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]);
      dst[1] = make_float4(st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]);
    }
    if (chunk == 0) {
#pragma unroll
      for (int h = 0; h < kGroup; ++h) s_l[wave][row][h] = st.lsum[h];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < kGroup; ++h) s_m[wave][h] = st.m[h];
    s_bad[wave] = bad ? 1 : 0;
  }
  __syncthreads();

  // Merge the wavefronts: thread -> (head h, dim d).
  const int h = threadIdx.x >> 6;
  const int d = threadIdx.x & 63;
  const bool any_bad = (s_bad[0] | s_bad[1] | s_bad[2] | s_bad[3]) != 0;
  float M = s_m[0][h];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmax_plain(M, s_m[w][h]);
  float O = 0.0f, Ls = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float e = __builtin_amdgcn_exp2f(s_m[w][h] - M);  // 0 for a wavefront without pages
    const float a = s_acc[w][0][h][d] + s_acc[w][1][h][d] + s_acc[w][2][h][d] + s_acc[w][3][h][d];
    const float l = s_l[w][0][h] + s_l[w][1][h] + s_l[w][2][h] + s_l[w][3][h];
    O = __builtin_fmaf(e, a, O);
    Ls = __builtin_fmaf(e, l, Ls);
  }

  finish_group<kSplit, kOutBf16>(p, b, g, part, n_pages, M, O, Ls, any_bad);
}

// ---------------------------------------------------------------------------------------------
// Matrix-core flavour of the same kernel: the two contractions of a 32-key step (two pages) run
// on v_mfma_f32_16x16x32_bf16 and only the softmax stays on the vector ALUs.
//
// Register layout of the 16x16x32 BF16 MFMA on gfx950 (lane l, element i):
//   A operand: row l % 16, reduction index 8 (l / 16) + i;  B operand: column l % 16, same k;
//   C/D: column l % 16, row 4 (l / 16) + i.
// Scores are computed transposed, S^T = K Q^T: the A operand is K straight from the pool (row =
// key, 8 consecutive dims per lane) and the B operand is Q^T with the group's 4 query heads in
// columns 0..3 and zeros in columns 4..15.  The A rows of tile t (t = 0, 1) are the step's keys
// 8 (r / 4) + 4 t + r % 4 (keys 0..15 are the first page's tokens, 16..31 the second's), so that
// lane l ends up holding keys 8 (l / 16) .. + 7 of head l % 16 across its two C tiles: exactly the
// B-operand layout of P^T in O^T = V^T P^T, so the weights never leave their registers.  V is
// loaded in the coalesced layout, staged row-major in this wavefront's LDS region and read back
// transposed (ds_read_b64_tr_b16) as the A operand of V^T.  The weights enter the second product
// as hi + lo BF16 pairs (about 16 significant bits; V is exact in BF16), and the denominator is
// the same product against an all-ones tile.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));

constexpr int kStepKeys = 32;           // two pages per step
constexpr int kVStride = kHeadDim + 8;  // staged V row in elements (144 bytes: conflict-free reads)

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ u32x4_t as_u32x4(uint4 v) { return u32x4_t{v.x, v.y, v.z, v.w}; }
__device__ __forceinline__ u32x4_t load16_stream_v(const uint16_t *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}

// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four key groups of one MFMA
// column): each permlane swap hands every lane the pair {x[l], x[l ^ 16]} (or ^ 32) as its two
// results, a VALU exchange with no LDS round trip.  The pair is reinterpreted as a whole: with
// this compiler a bit cast whose operand is one element of a vector (a[1]) reads element 0.
__device__ __forceinline__ float max_over_key_groups(float x) {
  const f2_t a = __builtin_bit_cast(
      f2_t, __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x), false, false));
  x = fmax_plain(a[0], a[1]);
  const f2_t c = __builtin_bit_cast(
      f2_t, __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x), false, false));
  return fmax_plain(c[0], c[1]);
}

// One step's loads: K rows in the A-operand layout ([tile][dim half]) and V in the coalesced
// layout ([page of the step]: tokens tok and tok + 8).
struct StepRegs {
  u32x4_t k[2][2];
  uint4 va[2], vb[2];
};

template <bool kSplit, bool kOutBf16, bool kFused>
__global__ __launch_bounds__(kThreads) void paged_decode_mfma_kernel(PKV_PRELOADED_ARGS, DecodeParams p) {
  PKV_TAKE_PRELOADED_ARGS(p);
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kWaves][kStepKeys * kVStride];
  __shared__ __attribute__((aligned(16))) float s_o[kWaves][kGroup][kHeadDim];
  __shared__ float s_l[kWaves][kGroup];
  __shared__ float s_m[kWaves][kGroup];
  __shared__ int s_bad[kWaves];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.x;  // grid (KV head, sequence, partition), as in paged_decode_kernel
  const int b = blockIdx.y;
  const int part = blockIdx.z;
  const int qh0 = g * kGroup;
  const int p0 = part * p.part_pages;
  const int tok = lane >> 3;    // coalesced layout: token within each half page
  const int chunk = lane & 7;   //   and 16-byte chunk of its row
  const int r = lane & 15;      // MFMA row / column
  const int kg = lane >> 4;     // MFMA reduction group

  const int32_t *bt = p.block_tables + (int64_t)b * p.max_blocks;
  const int e_lane = p0 + wave + kWaves * lane;
  const int ids_row = e_lane < p.max_blocks ? bt[e_lane] : 0;
  // Q^T as the B operand: column r < 4 is query head qh0 + r, dims 32 hf + 8 kg .. + 7.
  u32x4_t qf[2] = {u32x4_t{0u, 0u, 0u, 0u}, u32x4_t{0u, 0u, 0u, 0u}};
  if (r < kGroup) {
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(p.q + ((int64_t)b * p.num_q_heads + qh0 + r) * kHeadDim);
    qf[0] = src[kg];
    qf[1] = src[4 + kg];
  }
  uint4 knew = make_uint4(0u, 0u, 0u, 0u), vnew = knew;
  u32x4_t kn[2] = {u32x4_t{0u, 0u, 0u, 0u}, u32x4_t{0u, 0u, 0u, 0u}};
  if (kFused) {
    const int64_t row = ((int64_t)b * p.num_kv_heads + g) * kHeadDim;
    knew = load16(p.k_new + row + chunk * 8);
    vnew = load16(p.v_new + row + chunk * 8);
    kn[0] = *reinterpret_cast<const u32x4_t *>(p.k_new + row + 8 * kg);
    kn[1] = *reinterpret_cast<const u32x4_t *>(p.k_new + row + 32 + 8 * kg);
  }
  const int L = context_length<kFused>(p, b);
  const bool len_ok = L >= 0 && L <= p.max_blocks * kBlock;
  const int n_pages = len_ok ? (L + kBlock - 1) / kBlock : 0;
  const int p1 = min(p0 + p.part_pages, n_pages);
  // The parameter-struct fields used past the prologue: their scalar loads are requested here and
  // consumed with the prologue's vector loads below, so they arrive in the same round trip rather
  // than in one of their own after it (the compiler would otherwise issue them after the branch).
  const int num_pages = p.num_pages;
  const float c_log2 = p.score_log2;
  const uint16_t *const k_pool = p.k_pool;
  const uint16_t *const v_pool = p.v_pool;
  asm volatile("" ::"s"(num_pages), "s"(c_log2), "s"(k_pool), "s"(v_pool));
  if (kSplit) {
    asm volatile("" ::"s"(p.out), "s"(p.part_o), "s"(p.part_ml), "s"(p.counters), "s"(p.num_parts));
  } else {
    asm volatile("" ::"s"(p.out));
  }
  if (kFused) asm volatile("" ::"s"(p.k_pool_w), "s"(p.v_pool_w));
  asm volatile("" ::"v"(ids_row));
  asm volatile("" ::"v"(qf[0].x), "v"(qf[0].y), "v"(qf[0].z), "v"(qf[0].w), "v"(qf[1].x), "v"(qf[1].y), "v"(qf[1].z), "v"(qf[1].w));
  if (kFused) {
    asm volatile("" ::"v"(knew.x), "v"(knew.y), "v"(knew.z), "v"(knew.w), "v"(vnew.x), "v"(vnew.y), "v"(vnew.z), "v"(vnew.w));
    asm volatile("" ::"v"(kn[0].x), "v"(kn[0].y), "v"(kn[0].z), "v"(kn[0].w), "v"(kn[1].x), "v"(kn[1].y), "v"(kn[1].z), "v"(kn[1].w));
  }

  if (p0 >= p1) {
    if (kSplit && part != 0) return;  // see paged_decode_kernel
    const int64_t o = ((int64_t)b * p.num_q_heads + qh0) * kHeadDim + threadIdx.x;
    if (kOutBf16) static_cast<uint16_t *>(p.out)[o] = 0;
    else static_cast<float *>(p.out)[o] = 0.0f;
    return;
  }

  int n_w = (p1 - p0 - wave + kWaves - 1) / kWaves;
  if (n_w < 0) n_w = 0;
  const int ids = lane < n_w ? ids_row : 0;
  const bool bad = __builtin_amdgcn_ballot_w64(ids < 0 || ids >= num_pages) != 0;
  const bool holds_last = n_w > 0 && p1 == n_pages && p0 + wave + kWaves * (n_w - 1) == n_pages - 1;
  const int last_id = holds_last ? __builtin_amdgcn_readlane(ids, n_w - 1) : -1;
  const bool do_append = kFused && last_id >= 0 && last_id < num_pages;
  if (bad) n_w = 0;
  const bool owns_last = n_w > 0 && holds_last;
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  const int64_t head_elems = (int64_t)kBlock * kHeadDim;
  const int64_t page_elems = (int64_t)p.num_kv_heads * head_elems;
  const uint16_t *kbase = k_pool + g * head_elems;
  const uint16_t *vbase = v_pool + g * head_elems + lane * 8;
  const int tail_valid = L - (n_pages - 1) * kBlock;
  if (do_append) {
    const int slot = tail_valid - 1;
    if (tok == (slot & 7)) {
      const int64_t dst = ((int64_t)last_id * p.num_kv_heads + g) * (kBlock * kHeadDim) + slot * kHeadDim + chunk * 8;
      *reinterpret_cast<uint4 *>(p.k_pool_w + dst) = knew;
      *reinterpret_cast<uint4 *>(p.v_pool_w + dst) = vnew;
    }
  }

  // The wavefront's pages in processing order: the sequence's last page (partial, and the fused
  // step's new token) first, then the others in logical order.  Position j of that list is local
  // page j - 1 (or n_w - 1 for j = 0) when the wavefront owns the last page, else local page j.
  auto page_off = [&](int j) -> int64_t {
    const int local = owns_last ? (j == 0 ? n_w - 1 : j - 1) : j;
    return (int64_t)__builtin_amdgcn_readlane(ids, local) * page_elems;
  };
  // K row of A row r in tile t: page r < 8 ? first : second, token 8 ((r / 4) & 1) + 4 t + r % 4.
  const int k_tok0 = 8 * ((r >> 2) & 1) + (r & 3);
  auto load_step = [&](int s, StepRegs &x) {
    const int j0 = 2 * s;
    const int j1 = 2 * s + 1 < n_w ? 2 * s + 1 : j0;  // a missing second page re-reads the first (masked)
    const int64_t offA = page_off(j0), offB = page_off(j1);
    const uint16_t *kp = kbase + (r < 8 ? offA : offB) + k_tok0 * kHeadDim + 8 * kg;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      x.k[t][0] = load16_stream_v(kp + 4 * t * kHeadDim);
      x.k[t][1] = load16_stream_v(kp + 4 * t * kHeadDim + 32);
    }
    x.va[0] = load16_stream(vbase + offA);
    x.vb[0] = load16_stream(vbase + offA + 512);
    x.va[1] = load16_stream(vbase + offB);
    x.vb[1] = load16_stream(vbase + offB + 512);
  };

  f32x4_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t lsum = {0.f, 0.f, 0.f, 0.f};
  // Anchor (log2 units) of head r; columns 4..15 are padding and keep anchor 0 with weight 0.
  float m = r < kGroup ? -INFINITY : 0.0f;
  float thr = r < kGroup ? -INFINITY : INFINITY;
  const u32x4_t kOnes = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // BF16 1.0 x 8
  uint16_t *sv = s_v[wave];

  auto compute_step = [&](int s, StepRegs x) {
    const int j1 = 2 * s + 1;
    const int validA = (owns_last && s == 0) ? tail_valid : kBlock;
    const int validB = j1 < n_w ? kBlock : 0;
    if (kFused && owns_last && s == 0) {
      // The new token (slot tail_valid - 1 of the first page) replaces its row in registers.
      const int slot = tail_valid - 1;
      const int r_s = 4 * (slot >> 3) + (slot & 3);
      if (r == r_s) {
        if ((slot >> 2) & 1) { x.k[1][0] = kn[0]; x.k[1][1] = kn[1]; }
        else { x.k[0][0] = kn[0]; x.k[0][1] = kn[1]; }
      }
      if (tok == (slot & 7)) {
        if (slot < 8) x.va[0] = vnew;
        else x.vb[0] = vnew;
      }
    }
    // Only a step holding the sequence's partial last page or a missing second page has rows to
    // mask (wave-uniform): rows past a page's valid tokens are zeroed before staging, so stale or
    // NaN slot contents never reach the product (their weights are 0 as well).
    const bool partial = validA < kBlock || validB < kBlock;
    if (partial) {
      const uint4 z = make_uint4(0u, 0u, 0u, 0u);
      if (tok >= validA) x.va[0] = z;
      if (tok + 8 >= validA) x.vb[0] = z;
      if (tok >= validB) x.va[1] = z;
      if (tok + 8 >= validB) x.vb[1] = z;
    }
    *reinterpret_cast<uint4 *>(sv + tok * kVStride + chunk * 8) = x.va[0];
    *reinterpret_cast<uint4 *>(sv + (tok + 8) * kVStride + chunk * 8) = x.vb[0];
    *reinterpret_cast<uint4 *>(sv + (tok + 16) * kVStride + chunk * 8) = x.va[1];
    *reinterpret_cast<uint4 *>(sv + (tok + 24) * kVStride + chunk * 8) = x.vb[1];
    // V^T fragments, read back right away so the LDS latency overlaps the score products and the
    // softmax (this wavefront's LDS operations complete in order, so the reads see the rows just
    // written).  Within each 16-lane group, lane L of a transposing read receives element L % 4 of
    // the 4-element rows read by lanes L / 4 + 4 i; so lane (kg, r) reading row 8 kg + r / 4 at
    // dims 16 dt + 4 (r % 4) ends up with keys 8 kg .. + 3 of dim 16 dt + r, and a second read four
    // rows down gives keys + 4 .. + 7: the A operand of V^T for dims 16 dt .. + 15.
    u32x4_t vf[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const uint16_t *vrow = sv + (8 * kg + (r >> 2)) * kVStride + 16 * dt + 4 * (r & 3);
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t *)vrow);
      const v4i16_t hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t *)(vrow + 4 * kVStride));
      const u32x2_t a = __builtin_bit_cast(u32x2_t, lo), c = __builtin_bit_cast(u32x2_t, hi);
      vf[dt] = u32x4_t{a[0], a[1], c[0], c[1]};
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the softmax

    f32x4_t sc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(x.k[t][0]), as_bf16x8(qf[0]), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(x.k[t][1]), as_bf16x8(qf[1]), acc, 0, 0, 0);
      sc[t] = acc;
    }
    // This lane holds keys 8 kg + 4 t + i of head r: page kg / 2 of the step, token 8 (kg & 1) + 4 t + i.
    // Columns r >= 4 are padding (q = 0): their weights only reach output columns nobody reads,
    // and their anchor threshold is infinite, so they never move an anchor.
    // The lane's largest score is an IEEE maximum (v_maximum3, three inputs per instruction and no
    // quieting of its inputs); scores are finite or -inf, so it equals the plain maximum.
    const int valid_k = kg < 2 ? validA : validB;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int token = 8 * (kg & 1) + 4 * t + i;
        const float x2 = sc[t][i] * c_log2;  // scaled first: p is exactly 1 for the anchor's key
        sc[t][i] = (partial && token >= valid_k) ? -INFINITY : x2;
      }
    float smax = sc[0][0];
#pragma unroll
    for (int e = 1; e < 8; ++e) smax = __builtin_elementwise_maximum(smax, sc[e >> 2][e & 3]);
    if (__builtin_amdgcn_ballot_w64(smax > thr) != 0) {  // wave-uniform and rare
      const float mx = max_over_key_groups(smax);
      const float m_new = fmax_plain(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 on the first step of a head
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      lsum *= alpha;
      m = m_new;
      thr = r < kGroup ? m_new + kAnchorHeadroom : INFINITY;
    }
    u32x4_t ph, pl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f2_t w2;
      w2[0] = __builtin_amdgcn_exp2f(sc[e >> 1][2 * (e & 1)] - m);
      w2[1] = __builtin_amdgcn_exp2f(sc[e >> 1][2 * (e & 1) + 1] - m);
      const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(w2, b2_t));
      f2_t rest;  // exact in FP32: each weight minus its own BF16 rounding
      rest[0] = w2[0] - __builtin_bit_cast(float, hi << 16);
      rest[1] = w2[1] - __builtin_bit_cast(float, hi & 0xFFFF0000u);
      ph[e] = hi;
      pl[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rest, b2_t));
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf[dt]), as_bf16x8(ph), o[dt], 0, 0, 0);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf[dt]), as_bf16x8(pl), o[dt], 0, 0, 0);
    }
    lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kOnes), as_bf16x8(ph), lsum, 0, 0, 0);
    lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kOnes), as_bf16x8(pl), lsum, 0, 0, 0);
  };

  const int n_steps = (n_w + 1) >> 1;
  if (n_steps == 1) {  // one step (short contexts): no second buffer, no loads beyond the pages
    StepRegs x0;
    load_step(0, x0);
    compute_step(0, x0);
  } else if (n_steps > 1) {
    // Two step buffers; both first loads are unconditional, and the steady-state loop only runs
    // while both reloads exist, so the compiler's waits count exactly the newer loads in flight.
    StepRegs x0, x1;
    load_step(0, x0);
    load_step(1, x1);
    int s = 0;
    for (; s + 3 < n_steps; s += 2) {
      compute_step(s, x0);
      load_step(s + 2, x0);
      compute_step(s + 1, x1);
      load_step(s + 3, x1);
    }
    const int rem = n_steps - s;  // 1 .. 3
    compute_step(s, x0);
    if (rem >= 3) load_step(s + 2, x0);
    if (rem >= 2) compute_step(s + 1, x1);
    if (rem >= 3) compute_step(s + 2, x0);
  }

  // Lanes r < 4 hold head r: o[dt][i] is dim 16 dt + 4 kg + i, lsum the denominator.
  if (r < kGroup) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4_t *>(&s_o[wave][r][16 * dt + 4 * kg]) = o[dt];
    if (kg == 0) {
      s_l[wave][r] = lsum[0];
      s_m[wave][r] = m;
    }
  }
  if (lane == 0) s_bad[wave] = bad ? 1 : 0;
  __syncthreads();

  const int h = threadIdx.x >> 6;
  const int d = threadIdx.x & 63;
  bool any_bad = false;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    any_bad |= s_bad[w] != 0;
    M = fmax_plain(M, s_m[w][h]);
  }
  float O = 0.0f, Ls = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float e = __builtin_amdgcn_exp2f(s_m[w][h] - M);
    O = __builtin_fmaf(e, s_o[w][h][d], O);
    Ls = __builtin_fmaf(e, s_l[w][h], Ls);
  }
  finish_group<kSplit, kOutBf16>(p, b, g, part, n_pages, M, O, Ls, any_bad);
}

}  // namespace

template <bool kFused>
hipError_t launch_variant(const DecodeParams &p, bool out_bf16, hipStream_t stream) {
  const int64_t groups = (int64_t)p.batch * p.num_kv_heads * p.num_parts;
  if (groups == 0) return hipSuccess;
  if (groups > 0x7fffffff || p.batch > 65535 || p.num_parts > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)p.num_kv_heads, (unsigned)p.batch, (unsigned)p.num_parts), block(kThreads);
  const bool split = p.num_parts > 1;
#define PKV_LAUNCH(kernel, kSplit, kBf16)                                                                   \
  hipLaunchKernelGGL((kernel<kSplit, kBf16, kFused>), grid, block, 0, stream, p.block_tables,                \
                     kFused ? p.positions : p.context_lens, p.q, p.k_new, p.v_new, p.max_blocks, p.num_kv_heads, \
                     p.batch, p.part_pages, p)
  if (p.matrix_cores) {
    if (split) {
      if (out_bf16) PKV_LAUNCH(paged_decode_mfma_kernel, true, true);
      else PKV_LAUNCH(paged_decode_mfma_kernel, true, false);
    } else {
      if (out_bf16) PKV_LAUNCH(paged_decode_mfma_kernel, false, true);
      else PKV_LAUNCH(paged_decode_mfma_kernel, false, false);
    }
  } else {
    if (split) {
      if (out_bf16) PKV_LAUNCH(paged_decode_kernel, true, true);
      else PKV_LAUNCH(paged_decode_kernel, true, false);
    } else {
      if (out_bf16) PKV_LAUNCH(paged_decode_kernel, false, true);
      else PKV_LAUNCH(paged_decode_kernel, false, false);
    }
  }
#undef PKV_LAUNCH
  return hipGetLastError();
}

hipError_t launch_paged_decode(const DecodeParams &p, bool out_bf16, hipStream_t stream) {
  return p.positions ? launch_variant<true>(p, out_bf16, stream) : launch_variant<false>(p, out_bf16, stream);
}

}  // namespace pkv
