// Paged decode attention for gfx950: one workgroup per (sequence, KV head, context partition).
//
// What is computed ("6 Hours of YouTube and 85 handtyped pages of notes on LLM Inference", section "What works so far"; "The prefill path: flowing the entire prompt at once",
// sections "Per-head attention scores and GQA" and "causalMask and online softmax"): for the
// four query heads that share KV head g, scores s_t = scale * <q_h, K_t> over the sequence's
// cached tokens, softmax over t, and the softmax-weighted sum of the V rows.  The pages' decode
// kernel streams the non-contiguous pages directly with an FP32 online softmax, gathering no
// contiguous prefix and storing no scores; so does this one.
//
// Design for CDNA4 (64-lane wavefronts, DPP cross-lane ops, v_dot2 on BF16 pairs):
//   * One workgroup serves the whole GQA group of a KV head, so each K/V byte is read from HBM
//     exactly once for all four query heads.
//   * 4 wavefronts per workgroup; wavefront w takes pages w, w+4, w+8, ... of the partition and
//     keeps its own softmax state, so the main loop has no barriers.  The four states are
//     merged in LDS at the end with the pairwise (max, sum) rule.
//   * One 16-token page of one KV head is a contiguous 2 KiB run.  A wavefront loads it with
//     two 16-byte loads per lane (lane = 8 * token + chunk): lanes 0..63 cover bytes 0..1023
//     (tokens 0..7), the second load bytes 1024..2047 (tokens 8..15).  The next two pages' K and
//     V are in flight while the current page is computed (a short chain issues all its loads
//     at once).
//   * QK: each lane forms 8-element partial dots with v_dot2_f32_bf16 (BF16 pairs, FP32
//     accumulate) and the 8 lanes of a token are summed with three DPP adds.
//   * Softmax in log2 units with a lazily moved anchor: scores are compared with the anchor
//     plus 8; only when a page exceeds it does the wavefront recompute the anchor and rescale
//     its accumulators (the result is independent of the anchor; fp32 holds 2^8 of headroom).
//   * PV: each lane accumulates p * V for its 8 dims and 4 heads in 32 FP32 registers; the
//     token lanes are summed once at the end.
//   * Long contexts with few (sequence, KV head) pairs are cut into partitions; each writes its
//     (max, sum, partial output) per query head and a merge kernel combines them.  Workgroup ids
//     are partition-major, so every partition index is spread over all 8 XCDs.
// Block-table entries are read straight into a VGPR (one entry per lane) and moved to scalar
// registers with v_readlane; every entry is range-checked before a page is touched.
#include <math.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
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

template <bool kSplit, bool kOutBf16, bool kFused>
__global__ __launch_bounds__(kThreads) void paged_decode_kernel(DecodeParams p) {
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
  const int pairs = p.batch * p.num_kv_heads;
  const int part = blockIdx.x / pairs;
  const int pair = blockIdx.x % pairs;
  const int g = pair % p.num_kv_heads;
  const int b = pair / p.num_kv_heads;
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
  // Keep those reads above the branch below (the compiler would otherwise sink them past it,
  // behind the length read).
  asm volatile("" ::"v"(ids_row));
#pragma unroll
  for (int h = 0; h < kGroup; ++h) asm volatile("" ::"v"(qv[h][0]), "v"(qv[h][1]), "v"(qv[h][2]), "v"(qv[h][3]));
  if (kFused) asm volatile("" ::"v"(knew.x), "v"(knew.y), "v"(knew.z), "v"(knew.w), "v"(vnew.x), "v"(vnew.y), "v"(vnew.z), "v"(vnew.w));

  if (p0 >= p1) {
    if (kSplit) return;  // empty partition (or empty/invalid sequence): the merge handles it
    // Empty or invalid sequence: zeros for the group's 4 x 64 outputs.
    const int64_t o = ((int64_t)b * p.num_q_heads + qh0) * kHeadDim + threadIdx.x;
    if (kOutBf16) static_cast<uint16_t *>(p.out)[o] = 0;
    else static_cast<float *>(p.out)[o] = 0.0f;
    return;
  }

  const float c_log2 = p.score_log2;

  // Pages of this wavefront: local index k -> logical page p0 + wave + kWaves * k, k < n_w <= 64
  // (a partition holds at most kMaxPartitionPages pages).
  int n_w = (p1 - p0 - wave + kWaves - 1) / kWaves;
  if (n_w < 0) n_w = 0;
  // One table entry per lane, range-checked before any page is touched.
  const int ids = lane < n_w ? ids_row : 0;
  const bool bad = __builtin_amdgcn_ballot_w64(ids < 0 || ids >= p.num_pages) != 0;
  // The wavefront holding the sequence's last page (it always holds the new token).
  const bool holds_last = n_w > 0 && p1 == n_pages && p0 + wave + kWaves * (n_w - 1) == n_pages - 1;
  // Like pkv_kv_append, the fused append depends only on its own page entry: an invalid entry
  // elsewhere in the sequence zeroes the output but does not stop the append.
  const int last_id = holds_last ? __builtin_amdgcn_readlane(ids, n_w - 1) : -1;
  const bool do_append = kFused && last_id >= 0 && last_id < p.num_pages;
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
  const uint16_t *kbase = p.k_pool + g * head_elems + lane * 8;
  const uint16_t *vbase = p.v_pool + g * head_elems + lane * 8;
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

  if (kSplit) {
    // A partition that met an invalid table entry marks its slot with a negative denominator (a
    // real one is positive), so the merge zeroes the sequence without reading the table again.
    const int64_t slot = ((int64_t)b * p.num_q_heads + qh0 + h) * p.num_parts + part;
    p.part_o[slot * kHeadDim + d] = O;
    if (d == 0) {
      p.part_ml[slot * 2 + 0] = M;
      p.part_ml[slot * 2 + 1] = any_bad ? -1.0f : Ls;
    }
  } else {
    const float r = any_bad ? 0.0f : O / Ls;
    const int64_t o = ((int64_t)b * p.num_q_heads + qh0 + h) * kHeadDim + d;
    if (kOutBf16) static_cast<uint16_t *>(p.out)[o] = f32_to_bf16_rne(r);
    else static_cast<float *>(p.out)[o] = r;
  }
}

// Combine the partitions of one (sequence, query head): M = max m_i, O = sum o_i 2^(m_i - M),
// l = sum l_i 2^(m_i - M), out = O / l.  One wavefront: the partitions' (m, l) pairs are spread
// over the lanes for the max and the weighted sum; lane d accumulates dim d of the partial outputs
// with the weights broadcast from the lanes that hold them.  A slot marked invalid by its
// partition (negative l) zeroes the sequence, as the unsplit kernel does.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmax_plain(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Partitions whose partial outputs the merge holds in registers at once.
constexpr int kMergeRegParts = 16;

template <bool kOutBf16, bool kFused>
__global__ __launch_bounds__(64) void merge_partitions_kernel(DecodeParams p) {
  const int b = blockIdx.x / p.num_q_heads;
  const int h = blockIdx.x % p.num_q_heads;
  const int lane = threadIdx.x;
  const int64_t slot0 = ((int64_t)b * p.num_q_heads + h) * p.num_parts;
  const float *ml = p.part_ml + slot0 * 2;
  const float *po = p.part_o + slot0 * kHeadDim + lane;

  // The kernel is latency-bound: the (m, l) pairs of the first 64 slots and the partial outputs of
  // the first kMergeRegParts slots are loaded together with the context length, in one round trip.
  // Slot indexes are clamped to the launch's partition count, so every load is in bounds; slots
  // past the sequence's own partitions hold stale data and are discarded by index below.
  const int last = p.num_parts - 1;
  const float2 mlv = *reinterpret_cast<const float2 *>(ml + 2 * min(lane, last));
  float v[kMergeRegParts];
#pragma unroll
  for (int u = 0; u < kMergeRegParts; ++u) v[u] = po[(int64_t)min(u, last) * kHeadDim];
  // Keep the scheduler from placing these loads after the wait for the context length.
  __builtin_amdgcn_sched_barrier(0);

  const int L = context_length<kFused>(p, b);
  const bool len_ok = L > 0 && L <= p.max_blocks * kBlock;
  const int n_pages = len_ok ? (L + kBlock - 1) / kBlock : 0;
  const int n_parts = (n_pages + p.part_pages - 1) / p.part_pages;  // <= num_parts
  // Up to kMergeRegParts partitions, straight from the registers.  This runs unconditionally (the
  // masks make it harmless otherwise) so the compiler keeps the loads above ahead of every branch.
  const bool mine = lane < n_parts;
  const float m = mine ? mlv.x : -INFINITY;
  const float l = mine ? mlv.y : 0.0f;
  const bool bad = __builtin_amdgcn_ballot_w64(mine && !(l >= 0.0f)) != 0;
  const float M = wave_max(m);
  const float e = mine ? __builtin_amdgcn_exp2f(m - M) : 0.0f;
  const float Ls = wave_sum(e * l);
  const int eb = __builtin_bit_cast(int, e);
  float O = 0.0f;
#pragma unroll
  for (int u = 0; u < kMergeRegParts; ++u)
    if (u < n_parts) O = __builtin_fmaf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(eb, u)), v[u], O);
  float r = (n_parts > 0 && n_parts <= kMergeRegParts && !bad) ? O / Ls : 0.0f;
  if (n_parts > kMergeRegParts) {
    // Long splits: the pairs 64 at a time, the partial outputs 8 at a time per lane.
    bool any_bad = false;
    float Mg = -INFINITY;
    for (int i0 = 0; i0 < n_parts; i0 += 64) {
      const int i = i0 + lane;
      if (i < n_parts) {
        Mg = fmax_plain(Mg, ml[2 * i]);
        any_bad |= !(ml[2 * i + 1] >= 0.0f);
      }
    }
    if (__builtin_amdgcn_ballot_w64(any_bad) == 0) {
      Mg = wave_max(Mg);
      float Og = 0.0f, Lg = 0.0f;
      for (int i0 = 0; i0 < n_parts; i0 += 64) {
        const int i = i0 + lane;
        const float ei = i < n_parts ? __builtin_amdgcn_exp2f(ml[2 * i] - Mg) : 0.0f;  // 0 past the end
        Lg += i < n_parts ? ei * ml[2 * i + 1] : 0.0f;
        const int cnt = min(64, n_parts - i0);
        const int eib = __builtin_bit_cast(int, ei);
        for (int j0 = 0; j0 < cnt; j0 += 8) {  // j0 <= 56, so j0 + u <= 63 below
          float w[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) w[u] = j0 + u < cnt ? po[(int64_t)(i0 + j0 + u) * kHeadDim] : 0.0f;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float ej = __builtin_bit_cast(float, __builtin_amdgcn_readlane(eib, j0 + u));
            Og = __builtin_fmaf(ej, w[u], Og);
          }
        }
      }
      r = Og / wave_sum(Lg);
    }
  }
  const int64_t o = ((int64_t)b * p.num_q_heads + h) * kHeadDim + lane;
  if (kOutBf16) static_cast<uint16_t *>(p.out)[o] = f32_to_bf16_rne(r);
  else static_cast<float *>(p.out)[o] = r;
}

}  // namespace

template <bool kFused>
hipError_t launch_variant(const DecodeParams &p, bool out_bf16, hipStream_t stream) {
  const int64_t groups = (int64_t)p.batch * p.num_kv_heads * p.num_parts;
  if (groups == 0) return hipSuccess;
  if (groups > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)groups), block(kThreads);
  if (p.num_parts == 1) {
    if (out_bf16) hipLaunchKernelGGL((paged_decode_kernel<false, true, kFused>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((paged_decode_kernel<false, false, kFused>), grid, block, 0, stream, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((paged_decode_kernel<true, true, kFused>), grid, block, 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 mgrid((unsigned)((int64_t)p.batch * p.num_q_heads));
  if (out_bf16) hipLaunchKernelGGL((merge_partitions_kernel<true, kFused>), mgrid, dim3(64), 0, stream, p);
  else hipLaunchKernelGGL((merge_partitions_kernel<false, kFused>), mgrid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_paged_decode(const DecodeParams &p, bool out_bf16, hipStream_t stream) {
  return p.positions ? launch_variant<true>(p, out_bf16, stream) : launch_variant<false>(p, out_bf16, stream);
}

}  // namespace pkv
